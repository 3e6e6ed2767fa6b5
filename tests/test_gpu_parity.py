"""GPU vs oracle parity through the C ABI, at sizes the oracle finishes in
seconds: the tiny workload, a ragged multi-tile bf16 case, edge cases,
inserts with splits, determinism. Every case prints its name and shape before
it touches the GPU.
"""
import math

import numpy as np
import pytest
import torch

import gpu_support as gs
from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth
from oracle import icecache as ic

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from ann_retrieval_amd.api import IceIndex  # noqa: E402


from gpu_support import build_case, check_build, check_decode, decode_against_select_attend, say  # noqa: E402


# ---------------------------------------------------------------------------

def test_tiny_workload():
    """1 head, d=64 fp32, N=2048 from 32 Gaussians, 3 levels, p=1/16, 16
    queries at a 64-token budget (4 pages), seed 0."""
    w, gen, ix = build_case(1, 2048, 64, "f32", 32, 0, G=1, budget=64)
    refs = check_build(w, ix, [0], 0, 3, 4)
    for i in range(16):
        Q = synth.decode_queries(w, 1, gen)
        check_decode(w, ix, refs, Q, 64, 4)
    # beam covering every top point: the brute-force page ranking
    Q = synth.decode_queries(w, 1, gen)
    check_decode(w, ix, refs, Q, 64, 256)


def test_bf16_ragged_multi_tile():
    w, gen, ix = build_case(3, 3000, 128, "bf16", 48, 1, G=4, budget=256)
    refs = check_build(w, ix, [0, 1, 2], 1, 3, 4)
    for budget, beam in [(64, 4), (128, 8), (256, 16), (64, 16), (256, 64)]:
        check_decode(w, ix, refs, synth.decode_queries(w, 4, gen), budget, beam)


@pytest.mark.parametrize("case", [
    dict(N=0, d=128, dtype="bf16"),
    dict(N=1, d=128, dtype="bf16"),
    dict(N=17, d=64, dtype="f32"),
    dict(N=300, d=128, dtype="bf16", levels=1),
    dict(N=500, d=128, dtype="bf16", levels=2),
    dict(N=1000, d=64, dtype="bf16"),
    dict(N=700, d=128, dtype="f32"),
    dict(N=3000, d=128, dtype="bf16", levels=4, plog2=2),
    # 2-4 owners per head: buckets of 1,500-4,500 members, past the pack's
    # LDS window of 2,048 (their ranks scan the bucket in global memory)
    dict(N=6000, d=64, dtype="bf16", levels=2, plog2=11),
    dict(N=257, d=64, dtype="f32", G=16),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_edge_builds(case):
    c = dict(levels=3, plog2=4, G=2) | case
    w, gen, ix = build_case(2, c["N"], c["d"], c["dtype"], 8, 3, G=c["G"], levels=c["levels"], plog2=c["plog2"],
                            capacity=max(c["N"], 16), budget=64)
    refs = check_build(w, ix, [0, 1], 3, c["levels"], c["plog2"])
    check_decode(w, ix, refs, synth.decode_queries(w, c["G"], gen), 64, 4)
    check_decode(w, ix, refs, synth.decode_queries(w, c["G"], gen), 32, 1)


def test_long_head_lift_scan_chunks():
    """One head of 270,000 tokens: more than 1,024 token blocks of 256, so the
    level-list scan carries its running counts across chunks of the block
    scan; 2 levels with promotion 1/4096 (about 66 owners, buckets of
    thousands of members, past the pack's LDS window)."""
    N, d, levels, plog2 = 270000, 64, 2, 12
    w, gen, ix = build_case(1, N, d, "bf16", 8, 3, G=2, levels=levels, plog2=plog2, capacity=N, budget=64)
    refs = check_build(w, ix, [0], 3, levels, plog2)
    check_decode(w, ix, refs, synth.decode_queries(w, 2, gen), 64, 4)


def test_max_group_beam_budget():
    """The largest selection the boundary accepts: G = ICE_MAX_GROUP query heads,
    beam = ICE_MAX_BEAM, budget = ICE_MAX_BEAM pages (lists kept in LDS, the
    long union path)."""
    budget = L.ICE_MAX_BEAM * L.ICE_PAGE_CAP
    w, gen, ix = build_case(2, 12000, 128, "bf16", 64, 8, G=L.ICE_MAX_GROUP, budget=budget)
    refs = check_build(w, ix, [0, 1], 8, 3, 4)
    check_decode(w, ix, refs, synth.decode_queries(w, L.ICE_MAX_GROUP, gen), budget, L.ICE_MAX_BEAM)
    check_decode(w, ix, refs, synth.decode_queries(w, L.ICE_MAX_GROUP, gen), 1024, 100)


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", G=4, budget=256, beam=16, d=128),
    dict(dtype="bf16", G=4, budget=64, beam=4, d=128),
    dict(dtype="bf16", G=8, budget=128, beam=8, d=64),
    dict(dtype="bf16", G=8, budget=256, beam=16, d=128),      # union longer than a wave (G*k = 128)
    dict(dtype="bf16", G=16, budget=128, beam=8, d=64),       # union longer than a wave (G*k = 128)
    dict(dtype="bf16", G=16, budget=64, beam=4, d=64),
    dict(dtype="bf16", G=16, budget=256, beam=16, d=64),      # the longest fused union (G*k = 256)
    dict(dtype="bf16", G=5, budget=128, beam=8, d=128),       # 3 waves per query head
    dict(dtype="bf16", G=2, budget=256, beam=100, d=128),     # long lists: the two-kernel path
    dict(dtype="bf16", G=16, budget=128, beam=8, d=128),      # LDS too small for one kernel: two kernels
    dict(dtype="f32", G=4, budget=128, beam=8, d=128),        # fp32: the two-kernel path
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_decode_matches_select_then_attend(case):
    """ice_decode equals ice_select followed by ice_attend: selections and
    unions exactly, attention up to the order of fp32 sums; repeated calls
    are bit-identical; and the oracle."""
    w, gen, ix = build_case(3, 4000, case["d"], case["dtype"], 40, 11, G=case["G"], budget=case["budget"])
    refs = check_build(w, ix, [0, 2], 11, 3, 4)
    for _ in range(2):
        Q = synth.decode_queries(w, case["G"], gen).cuda()
        decode_against_select_attend(ix, refs, Q, case["budget"], case["beam"], str(case))


def test_decode_long_union_qwen_group():
    """The fused step's long-union path at the Qwen3-32B group shape: 64 heads
    x 8,192 tokens, 8 query heads per KV head, d=128 bf16, budget 256 (16
    pages each, unions of up to 128 pages), beam 16; heads 0 and 41 against
    the oracle."""
    w, gen, ix = build_case(64, 8192, 128, "bf16", 512, 13, G=8, budget=256)
    refs = check_build(w, ix, [0, 41], 13, 3, 4)
    for _ in range(3):
        Q = synth.decode_queries(w, 8, gen).cuda()
        out = decode_against_select_attend(ix, refs, Q, 256, 16, "qwen group")
        assert int(out["nuni"].max()) > 64, "the case must reach the long-union path"


@pytest.mark.parametrize("G,budget,beam", [(8, 256, 16), (4, 128, 8), (6, 64, 4)])
def test_decode_two_blocks_per_cu(G, budget, beam):
    """More heads than compute units: the selection blocks take half the waves
    per query head so that two share a CU. Selections, unions and attention
    against select + attend and the oracle, first and last heads."""
    H = torch.cuda.get_device_properties(0).multi_processor_count + 8
    w, gen, ix = build_case(H, 700, 128, "bf16", 12, 17, G=G, budget=budget)
    refs = check_build(w, ix, [0, H - 1], 17, 3, 4)
    for _ in range(2):
        Q = synth.decode_queries(w, G, gen).cuda()
        decode_against_select_attend(ix, refs, Q, budget, beam, f"paired G={G}")


def test_identical_keys():
    say("build identical keys H=1 N=200 d=128 bf16")
    K = torch.ones(1, 200, 128).to(torch.bfloat16)
    V = torch.randn(1, 200, 128, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    ix = IceIndex(1, 2, 128, "bf16", 200, 3, 4, 9, max_budget=64)
    ix.ice_build(K.cuda(), V.cuda())
    w = synth.Workload(K=K, V=V, mix=None, dtype="bf16")
    refs = check_build(w, ix, [0], 9, 3, 4)
    Q = torch.ones(1, 2, 128).to(torch.bfloat16)
    check_decode(w, ix, refs, Q, 64, 4)


def test_inserts_with_splits():
    """Append-only inserts in calls of several sizes; every step checked."""
    H, G, d = 2, 4, 128
    w, gen, ix = build_case(H, 1500, d, "bf16", 24, 4, G=G, capacity=1500 + 400, budget=128)
    refs = check_build(w, ix, [0, 1], 4, 3, 4)
    walk = synth.QueryWalk(w, G, gen, seg=16)
    Ks, Vs = [w.K], [w.V]
    sizes = [1, 1, 2, 5, 16, 50, 1, 100, 24]
    for n_new in sizes:
        ks, vs = [], []
        for _ in range(n_new):
            _, k, v = walk.step()
            ks.append(k)
            vs.append(v)
        k = torch.cat(ks, 1).contiguous()
        v = torch.cat(vs, 1).contiguous()
        say(f"insert n_new={n_new} at n={ix.n_tokens()}")
        ix.ice_insert(k.cuda(), v.cuda())
        torch.cuda.synchronize()
        for h in range(H):
            g = gs.read_head(ix, h)
            ref = refs[h]
            for j in range(n_new):
                t = ref.n
                lam_draw = int(ic.draw_levels(4, h, t, 1, 3, 4)[0])
                lam = min(ref.L_top, lam_draw)
                override = None
                if lam < ref.L_top:
                    cand = np.nonzero(ref.lev >= lam + 1)[0]
                    x = np.concatenate([gs.to64(k[h, j]), [ic.lift_one(gs.to64(k[h, j]), ref.M2)[0]]])
                    jj, D1, D2 = ic.nearest(x[None, :], ref.X()[cand])
                    gp = int(g.parent[lam][t])
                    if gp != int(cand[jj[0]]):
                        dg = float(((ref.X()[gp] - x) ** 2).sum())
                        assert abs(dg - D1[0]) <= gs.BAND * max(dg, D1[0]), f"insert parent of {t} outside the band"
                        override = gp
                ic.insert(ref, gs.to64(k[h, j]), gs.to64(v[h, j]), parent_override=override)
            assert np.array_equal(g.lev, ref.lev)
            gs.check_table_structure(g, ix.capacity)
            gs.compare_layout(ref, g, ix.capacity)
            assert g.stats["splits"] == ref.splits and g.stats["clamps"] == ref.clamps
            assert g.stats["overflow"] == 0
        Ks.append(k)
        Vs.append(v)
    assert sum(r.splits for r in refs.values()) > 0
    w2 = synth.Workload(K=torch.cat(Ks, 1), V=torch.cat(Vs, 1), mix=w.mix, dtype=w.dtype)
    for budget, beam in [(128, 8), (64, 16)]:
        check_decode(w2, ix, refs, walk.step()[0], budget, beam)
    # capacity: the next insert over the limit is refused and changes nothing
    before = gs.read_head(ix, 0)
    big = torch.zeros(H, 2000, d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.IceError) as ei:
        ix.ice_insert(big, big)
    assert ei.value.code == L.ICE_ERR_CAPACITY
    after = gs.read_head(ix, 0)
    assert after.n == before.n and after.tables[0]["pages"] == before.tables[0]["pages"]


def test_insert_into_empty_index():
    say("insert into an empty index H=1 d=64 f32")
    ix = IceIndex(1, 1, 64, "f32", 40, 3, 4, 2, max_budget=64)
    z = torch.zeros(1, 0, 64, device="cuda")
    ix.ice_build(z, z)
    gen = torch.Generator().manual_seed(3)
    k = torch.randn(1, 20, 64, generator=gen)
    v = torch.randn(1, 20, 64, generator=gen)
    ix.ice_insert(k.cuda(), v.cuda())
    g = gs.read_head(ix, 0)
    ref = ic.build_head(np.zeros((0, 64)), np.zeros((0, 64)), 0, 2)
    for j in range(20):
        ic.insert(ref, gs.to64(k[0, j]), gs.to64(v[0, j]))
    gs.compare_layout(ref, g, ix.capacity)
    assert g.stats["clamps"] == ref.clamps == 20
    w = synth.Workload(K=k, V=v, mix=None, dtype="f32")
    check_decode(w, ix, {0: ref}, torch.randn(1, 1, 64, generator=gen), 32, 2)


def test_determinism():
    w, gen, ix = build_case(2, 2500, 128, "bf16", 32, 6, G=4, budget=128)
    a = [ix.export(h, what, 0) for h in range(2) for what in (L.ICE_EXP_PARENT, L.ICE_EXP_PAGE_TOK, L.ICE_EXP_PAGE_K)]
    ix.ice_build(w.K.cuda(), w.V.cuda())
    b = [ix.export(h, what, 0) for h in range(2) for what in (L.ICE_EXP_PARENT, L.ICE_EXP_PAGE_TOK, L.ICE_EXP_PAGE_K)]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    Q = synth.decode_queries(w, 4, gen).cuda()
    r1 = [t.cpu() for t in ix.ice_select(Q, 128, 8)] + [t.cpu() for t in ix.ice_attend(Q, *ix.ice_select(Q, 128, 8)[1:])]
    r2 = [t.cpu() for t in ix.ice_select(Q, 128, 8)] + [t.cpu() for t in ix.ice_attend(Q, *ix.ice_select(Q, 128, 8)[1:])]
    assert all(torch.equal(x, y) for x, y in zip(r1, r2))
    # the fused decode step, many times over: every call gives the same bits
    for budget, beam in [(128, 8), (256, 16), (64, 4)]:
        say(f"decode determinism budget={budget} beam={beam}")
        first = [t.cpu() for t in ix.ice_decode(Q, budget, beam)]
        for _ in range(20):
            again = [t.cpu() for t in ix.ice_decode(Q, budget, beam)]
            assert all(torch.equal(x, y) for x, y in zip(first, again))


def test_argument_errors_leave_state():
    say("argument errors")
    ix = IceIndex(1, 1, 64, "f32", 64, 3, 4, 0, max_budget=64)
    Q = torch.zeros(1, 1, 64, device="cuda")
    with pytest.raises(L.IceError) as e:
        ix.ice_select(Q, 64, 4)
    assert e.value.code == L.ICE_ERR_STATE
    K = torch.randn(1, 64, 64, device="cuda")
    ix.ice_build(K, K)
    for budget, beam in [(0, 1), (24, 1), (64, 0), (64, 300)]:
        with pytest.raises(L.IceError) as e:
            ix.ice_select(Q, budget, beam)
        assert e.value.code == L.ICE_ERR_ARG
    with pytest.raises(L.IceError) as e:
        ix.ice_build(torch.randn(1, 65, 64, device="cuda"), torch.randn(1, 65, 64, device="cuda"))
    assert e.value.code == L.ICE_ERR_CAPACITY


def test_build_timed_equals_build():
    """ice_build_timed builds the same index as ice_build, bit for bit, and
    reports one non-negative time per phase (the parent search of every
    present level among them)."""
    w, gen, ix = build_case(3, 5000, 128, "bf16", 32, 14, G=4, budget=128)
    a = [ix.export(h, what, lv) for h in range(3)
         for what, lv in ((L.ICE_EXP_PARENT, 0), (L.ICE_EXP_PARENT, 1), (L.ICE_EXP_PAGE_TOK, 0), (L.ICE_EXP_PAGE_K, 0),
                          (L.ICE_EXP_PAGE_V, 0), (L.ICE_EXP_TOP, 0))]
    ms = ix.ice_build_timed(w.K.cuda(), w.V.cuda())
    b = [ix.export(h, what, lv) for h in range(3)
         for what, lv in ((L.ICE_EXP_PARENT, 0), (L.ICE_EXP_PARENT, 1), (L.ICE_EXP_PAGE_TOK, 0), (L.ICE_EXP_PAGE_K, 0),
                          (L.ICE_EXP_PAGE_V, 0), (L.ICE_EXP_TOP, 0))]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert ms.shape == (L.ICE_BUILD_PHASES,) and np.all(ms >= 0)
    assert ms[L.ICE_PHASE_PARENT] > 0 and ms[L.ICE_PHASE_PARENT + 4] > 0
    # no level-2 parents with 3 levels: those phases hold no kernel (two
    # events back to back, a few microseconds apart)
    assert np.all(ms[L.ICE_PHASE_OPERAND + 8:L.ICE_PHASE_TOP] < 0.05)
    say(f"build phases (ms): {np.round(ms, 4).tolist()}")
