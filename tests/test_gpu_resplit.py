"""Inserts under the re-sort split (ICE_SPLIT_RESORT), GPU against the
oracle's insert with ``resplit=True`` through the C ABI: levels exact,
parents within the near-tie band, page ids, owners and chains exact, the
order of every owner's members exact up to near-equal distances, the K and V
rows of every page slot bit-exact, then selection and attention on the
resulting index. A large-owner case crosses ICE_RESPLIT_MAX members. Every
case prints its name and shape before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import gpu_support as gs
from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth
from ann_retrieval_amd.api import IceIndex
from oracle import icecache as ic

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import say  # noqa: E402


def _pool_rows_exact(ix, h, g, K, V):
    """Every occupied slot of the level-0 pool holds its token's raw K and V
    row; empty slots are zero."""
    P = len(g.tables[0]["pages"])
    npd = np.int16 if ix.dtype == "bf16" else np.int32
    kp = ix.export(h, L.ICE_EXP_PAGE_K, 0, np_dtype=npd).reshape(-1, 16, ix.d)[:P]
    vp = ix.export(h, L.ICE_EXP_PAGE_V, 0, np_dtype=npd).reshape(-1, 16, ix.d)[:P]
    tok = g.tables[0]["tok"]
    valid = tok >= 0
    Kr, Vr = gs.raw_rows(K), gs.raw_rows(V)
    assert np.array_equal(kp[valid], Kr[tok[valid]]), "K rows do not follow their tokens"
    assert np.array_equal(vp[valid], Vr[tok[valid]]), "V rows do not follow their tokens"
    assert not kp[~valid].any() and not vp[~valid].any()


def _run(H, G, N, d, dtype, C, seed, levels, plog2, sizes, budget, checks):
    say(f"resort inserts H={H} N={N} d={d} {dtype} L={levels} p=2^-{plog2} sizes={sizes}")
    w, gen = synth.clustered_kv(H, N, d, C, dtype, seed, device="cpu")
    n_ins = sum(sizes)
    ix = IceIndex(H, G, d, dtype, N + n_ins, levels, plog2, seed, max_budget=budget, resort=True)
    ix.ice_build(w.K.cuda(), w.V.cuda())
    torch.cuda.synchronize()
    refs = gs.check_build(w, ix, list(range(H)), seed, levels, plog2)
    append = {h: ic.build_head(gs.to64(w.K[h]), gs.to64(w.V[h]), h, seed, levels, plog2) for h in range(H)}
    walk = synth.QueryWalk(w, G, gen, seg=16)
    Ks, Vs = [w.K], [w.V]
    for n_new in sizes:
        ks, vs = zip(*[walk.step()[1:] for _ in range(n_new)])
        k = torch.cat(ks, 1).contiguous()
        v = torch.cat(vs, 1).contiguous()
        Ks.append(k)
        Vs.append(v)
        say(f"insert n_new={n_new} at n={ix.n_tokens()}")
        ix.ice_insert(k.cuda(), v.cuda())
        torch.cuda.synchronize()
        Kall, Vall = torch.cat(Ks, 1), torch.cat(Vs, 1)
        for h in range(H):
            g = gs.read_head(ix, h)
            ref = refs[h]
            gs.replay_inserts(ref, g, k[h], v[h], h, seed, levels, plog2, resplit=True)
            for j in range(n_new):
                # the append-split twin takes the same parents
                t = ref.n - n_new + j
                lam = int(ref.lev[t])
                po = int(ref.parent[lam][t]) if lam < ref.L_top else None
                ic.insert(append[h], gs.to64(k[h, j]), gs.to64(v[h, j]), parent_override=po)
            assert np.array_equal(g.lev, ref.lev)
            gs.check_table_structure(g, ix.capacity)
            gs.compare_layout(ref, g, ix.capacity)
            assert g.stats["splits"] == ref.splits and g.stats["overflow"] == 0
            _pool_rows_exact(ix, h, g, Kall[h], Vall[h])
    # the re-sort did move tokens: some owner's member order differs from the append split
    moved = sum(refs[h].pages != append[h].pages for h in range(H))
    assert moved > 0 and sum(r.splits for r in refs.values()) > 0
    for h in range(H):
        gs.adopt_gpu_slots(refs[h], gs.read_head(ix, h))
    w2 = synth.Workload(K=torch.cat(Ks, 1), V=torch.cat(Vs, 1), mix=w.mix, dtype=w.dtype)
    for bgt, beam in checks:
        gs.check_decode(w2, ix, refs, walk.step()[0], bgt, beam)
    return refs


def test_resort_inserts_bf16():
    _run(2, 4, 1500, 128, "bf16", 24, 4, 3, 4, [1, 1, 2, 5, 16, 50, 1, 100, 24], 128, [(128, 8), (64, 16)])


def test_resort_inserts_f32_fused_decode():
    refs = _run(2, 2, 900, 64, "f32", 12, 11, 3, 3, [40, 1, 120], 64, [(64, 4)])
    assert all(r.L_top >= 1 for r in refs.values())


def test_resort_large_owners():
    """One level above the pages, promotion 2^-9: owners of several hundred
    to over a thousand members, so re-sorts stage up to ICE_RESPLIT_MAX rows
    in several passes, and an owner past the limit splits by appending."""
    refs = _run(1, 2, 2600, 64, "f32", 8, 30, 2, 9, [300, 1, 99], 64, [(64, 4)])
    counts = sorted(sum(len(refs[0].pages[p]) for p in ps) for ps in refs[0].owner_pages.values())
    say(f"owner sizes {counts}")
    assert counts[-1] > L.ICE_RESPLIT_MAX and any(600 < c <= L.ICE_RESPLIT_MAX for c in counts)


def test_resort_rejects_the_host_pool():
    say("resort with host pool is refused")
    with pytest.raises(L.IceError):
        IceIndex(1, 1, 64, "f32", 64, 3, 4, 0, max_budget=64, host_pool=True, resort=True)


def test_resort_inserts_f32_d128():
    _run(1, 2, 1200, 128, "f32", 10, 13, 3, 4, [64, 1, 90], 64, [(64, 4)])
