"""Builds with P-DCI parents (ice_build_pdci), GPU against the oracle's build
with the same directions and budgets through the C ABI: levels exact, P-DCI
parents exact up to near-equal distances among the same candidates, layout
and pools exact after replay, then selection and attention. With budgets
that cover every candidate the result is the exact search's. Every case
prints its name and shape before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import gpu_support as gs
from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth
from ann_retrieval_amd.api import IceIndex
from oracle import icecache as ic
from oracle import pdci as pd

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import say  # noqa: E402


def _pdci_case(H, N, d, dtype, C, seed, m, l, visits, cands, levels=3, plog2=4, G=2, budget=64):
    say(f"pdci build H={H} N={N} d={d} {dtype} m={m} l={l} visits={visits} cands={cands} L={levels} p=2^-{plog2}")
    w, gen = synth.clustered_kv(H, N, d, C, dtype, seed, device="cpu")
    dirs = synth.projection_dirs(m * l, d, seed + 1)
    ix = IceIndex(H, G, d, dtype, N, levels, plog2, seed, max_budget=budget)
    ix.ice_build_pdci(w.K.cuda(), w.V.cuda(), dirs.cuda(), m, l, visits, cands)
    torch.cuda.synchronize()
    cfg = pd.Pdci(dirs.double().numpy(), m, l, visits, cands)
    refs, ties, differs = {}, 0, 0
    for h in range(H):
        g = gs.read_head(ix, h)
        K64, V64 = gs.to64(w.K[h]), gs.to64(w.V[h])
        ref = ic.build_head(K64, V64, h, seed, levels, plog2, pdci=cfg)
        exact = ic.build_head(K64, V64, h, seed, levels, plog2)
        differs += sum(int(np.sum(ref.parent[lv] != exact.parent[lv])) for lv in range(ref.L_top))
        assert np.array_equal(g.lev, ref.lev) and g.L_top == ref.L_top
        gs.check_table_structure(g, ix.capacity)
        # a P-DCI parent that differs must be a near-tie of the oracle's in
        # both directions (a better parent than P-DCI finds is a mismatch too)
        X = ref.X()
        for lv in range(ref.L_top):
            for i in np.nonzero(ref.parent[lv] != g.parent[lv])[0]:
                da = float(((X[i] - X[ref.parent[lv][i]]) ** 2).sum())
                db = float(((X[i] - X[g.parent[lv][i]]) ** 2).sum())
                assert abs(da - db) <= gs.BAND * max(da, db), f"level {lv} token {i}: D {db:.9g} vs {da:.9g}"
        replay, t = gs.validate_parents(ref, g)
        ties += t
        if t:
            ref = gs.oracle_replay(K64, V64, h, seed, levels, plog2, replay)
        if gs.compare_layout(ref, g, ix.capacity):
            gs.adopt_gpu_slots(ref, g)
        refs[h] = ref
    say(f"pdci parity ok: parent near-ties={ties}, parents differing from the exact search={differs}")
    for _ in range(2):
        gs.check_decode(w, ix, refs, synth.decode_queries(w, G, gen), budget, 4)
    return differs


def test_pdci_build_bf16():
    assert _pdci_case(2, 3000, 128, "bf16", 24, 31, m=2, l=2, visits=32, cands=4) > 0


def test_pdci_build_f32_three_simple_indices():
    assert _pdci_case(1, 2000, 64, "f32", 16, 32, m=1, l=3, visits=16, cands=2) > 0


def test_pdci_unbounded_budgets_match_the_exact_search():
    """Visits and candidates that cover every candidate parent: the exact
    parents (the oracle's P-DCI then reduces to its exact search)."""
    assert _pdci_case(2, 1200, 128, "bf16", 12, 33, m=2, l=2, visits=10 ** 6, cands=10 ** 6) == 0


def test_pdci_argument_checks():
    say("pdci argument checks")
    ix = IceIndex(1, 1, 64, "f32", 64, 3, 4, 0, max_budget=64)
    K = torch.zeros(1, 8, 64, device="cuda")
    dirs = torch.zeros(16 * 2, 65, device="cuda")
    with pytest.raises(L.IceError):
        ix.ice_build_pdci(K, K, dirs[:5], 1, 5, 4, 1)          # l above ICE_PDCI_MAX_L
    with pytest.raises(L.IceError):
        ix.ice_build_pdci(K, K, dirs[:20], 5, 4, 4, 1)         # m*l above ICE_PDCI_MAX_KEYS
    with pytest.raises(L.IceError):
        ix.ice_build_pdci(K, K, dirs[:2], 1, 2, 0, 1)          # no visits


@pytest.mark.parametrize("n", [0, 1, 17, 300])
def test_pdci_edge_builds(n):
    """Empty, single-token and tiny builds (often no promoted point, so no
    parent search at all) give the oracle's layout."""
    say(f"pdci edge build n={n}")
    w, gen = synth.clustered_kv(1, max(n, 1), 64, 4, "f32", 40 + n, device="cpu")
    K, V = w.K[:, :n].contiguous(), w.V[:, :n].contiguous()
    dirs = synth.projection_dirs(4, 64, 41)
    ix = IceIndex(1, 1, 64, "f32", max(n, 1), 3, 2, 40 + n, max_budget=64)
    ix.ice_build_pdci(K.cuda(), V.cuda(), dirs.cuda(), 2, 2, 8, 2)
    torch.cuda.synchronize()
    g = gs.read_head(ix, 0)
    ref = ic.build_head(gs.to64(K[0]), gs.to64(V[0]), 0, 40 + n, 3, 2, pdci=pd.Pdci(dirs.double().numpy(), 2, 2, 8, 2))
    assert g.n == ref.n == n and np.array_equal(g.lev, ref.lev)
    replay, t = gs.validate_parents(ref, g)
    if t:
        ref = gs.oracle_replay(gs.to64(K[0]), gs.to64(V[0]), 0, 40 + n, 3, 2, replay)
    gs.compare_layout(ref, g, ix.capacity)


def test_pdci_build_then_inserts():
    """Inserts into a P-DCI-built index search their parents exactly, as
    they do after an exact build (bf16, d=64)."""
    H, N, d, seed = 2, 1500, 64, 42
    say(f"pdci build then inserts H={H} N={N} d={d} bf16")
    w, gen = synth.clustered_kv(H, N, d, 16, "bf16", seed, device="cpu")
    dirs = synth.projection_dirs(4, d, seed + 1)
    ix = IceIndex(H, 2, d, "bf16", N + 200, 3, 4, seed, max_budget=64)
    ix.ice_build_pdci(w.K.cuda(), w.V.cuda(), dirs.cuda(), 2, 2, 32, 4)
    torch.cuda.synchronize()
    cfg = pd.Pdci(dirs.double().numpy(), 2, 2, 32, 4)
    refs = {}
    for h in range(H):
        g = gs.read_head(ix, h)
        K64, V64 = gs.to64(w.K[h]), gs.to64(w.V[h])
        ref = ic.build_head(K64, V64, h, seed, 3, 4, pdci=cfg)
        replay, t = gs.validate_parents(ref, g)
        if t:
            ref = gs.oracle_replay(K64, V64, h, seed, 3, 4, replay)
        if gs.compare_layout(ref, g, ix.capacity):
            gs.adopt_gpu_slots(ref, g)
        refs[h] = ref
    walk = synth.QueryWalk(w, 2, gen, seg=16)
    ks, vs = zip(*[walk.step()[1:] for _ in range(200)])
    k, v = torch.cat(ks, 1).contiguous(), torch.cat(vs, 1).contiguous()
    say("insert n_new=200")
    ix.ice_insert(k.cuda(), v.cuda())
    torch.cuda.synchronize()
    for h in range(H):
        g = gs.read_head(ix, h)
        gs.replay_inserts(refs[h], g, k[h], v[h], h, seed, 3, 4)
        assert np.array_equal(g.lev, refs[h].lev)
        gs.check_table_structure(g, ix.capacity)
        if gs.compare_layout(refs[h], g, ix.capacity):
            gs.adopt_gpu_slots(refs[h], g)
    w2 = synth.Workload(K=torch.cat([w.K, k], 1), V=torch.cat([w.V, v], 1), mix=w.mix, dtype=w.dtype)
    gs.check_decode(w2, ix, refs, walk.step()[0], 64, 4)
