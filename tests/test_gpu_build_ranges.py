"""Builds of head ranges (one layer at a time, on streams of their own) against
a build of every head, through the C ABI. Every case prints its name and shape
before it touches the GPU.
"""
import numpy as np
import pytest
import torch

from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import say  # noqa: E402


def test_build_by_head_ranges_on_two_streams():
    """Builds of head ranges (two heads each, alternating between two streams,
    all in flight together) give the index a build of every head gives, bit
    for bit; and decode steps agree (selections exactly)."""
    from ann_retrieval_amd.api import IceIndex
    H, N, d = 6, 2200, 128
    say(f"build by head ranges H={H} N={N} d={d} bf16 on two streams")
    w, gen = synth.clustered_kv(H, N, d, 20, "bf16", 24, device="cpu")
    K, V = w.K.cuda(), w.V.cuda()
    full = IceIndex(H, 4, d, "bf16", N + 8, seed=24, max_budget=256)
    full.ice_build(K, V)
    part = IceIndex(H, 4, d, "bf16", N + 8, seed=24, max_budget=256)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for i, h0 in enumerate(range(0, H, 2)):
        part.ice_build_heads(K[h0:h0 + 2], V[h0:h0 + 2], h0, stream=streams[i % 2])
    torch.cuda.synchronize()
    row = d * 2
    for h in range(H):
        sa, sb = full.stats(h), part.stats(h)
        assert sa == sb, f"head {h} header"
        n, np0, n1 = sa["n_tokens"], sa["n_pages"][0], sa["n_pages"][1]
        for what, lv, nbytes in [(L.ICE_EXP_LEVEL, 0, n), (L.ICE_EXP_LIFT, 0, 4 * n), (L.ICE_EXP_PARENT, 0, 4 * n),
                                 (L.ICE_EXP_PARENT, 1, 4 * n), (L.ICE_EXP_PAGE_TOK, 0, 64 * np0),
                                 (L.ICE_EXP_PAGE_TOK, 1, 64 * n1), (L.ICE_EXP_PAGE_K, 0, 16 * row * np0),
                                 (L.ICE_EXP_PAGE_V, 0, 16 * row * np0), (L.ICE_EXP_TOP, 0, 4 * sa["n_top"])]:
            a = full.export(h, what, lv, np_dtype=np.uint8)[:nbytes]
            b = part.export(h, what, lv, np_dtype=np.uint8)[:nbytes]
            assert np.array_equal(a, b), f"head {h} export {what} level {lv}"
    # the range-built index against the oracle, head by head
    import gpu_support as gs
    refs = gs.check_build(w, part, [0, 3, 5], 24, 3, 4)
    Q = synth.decode_queries(w, 4, gen).cuda()
    r1 = full.ice_decode(Q, 256, 16)
    r2 = part.ice_decode(Q, 256, 16)
    torch.cuda.synchronize()
    # equal indexes decode to equal bits (the fused step is deterministic)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)
    out = gs.run_decode(part, Q, 256, 16)
    gs.compare_decode(part, refs, out)
    # a range build must keep the index's token count
    with pytest.raises(L.IceError):
        part.ice_build_heads(K[:2, :N - 1], V[:2, :N - 1], 0)


def host_pool_bytes(ix) -> np.ndarray:
    import ctypes
    return np.ctypeslib.as_array((ctypes.c_uint8 * ix.pool.nbytes).from_address(ix.pool.data_ptr())).copy()


@pytest.mark.parametrize("dtype,d,host_pool", [("bf16", 128, False), ("f32", 64, False), ("bf16", 128, True)])
def test_pipelined_build_equals_one_stream(dtype, d, host_pool):
    """A build of 37 heads runs as a two-stream pipeline over ranges of heads
    (10, 10, 10 and 7 heads). It leaves the blob, and the host pool, bit for
    bit as the one-stream build leaves them (ice_build_timed, which never
    pipelines). Work enqueued after it on its stream sees all of it. The heads
    at the ranges' edges match the oracle."""
    import gpu_support as gs
    from ann_retrieval_amd.api import IceIndex
    H, N, seed = 37, 2600, 31
    say(f"pipelined build H={H} N={N} d={d} {dtype} host_pool={host_pool}")
    w, gen = synth.clustered_kv(H, N, d, 24, dtype, seed, device="cpu")
    K, V = w.K.cuda(), w.V.cuda()
    ix = IceIndex(H, 4, d, dtype, N + 8, seed=seed, max_budget=256, host_pool=host_pool)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ix.ice_build(K, V)
        piped = ix.blob.clone()       # on the build's stream: after all of the build
    torch.cuda.synchronize()
    pool_piped = host_pool_bytes(ix) if host_pool else None
    refs = gs.check_build(w, ix, [0, 9, 10, 29, 30, 36], seed, 3, 4)
    ix.ice_build_timed(K, V)
    torch.cuda.synchronize()
    assert torch.equal(piped, ix.blob), "the pipelined build differs from the one-stream build"
    if host_pool:
        assert np.array_equal(pool_piped, host_pool_bytes(ix)), "host pools differ"
    # a decode right after a pipelined build on the same stream
    Q = synth.decode_queries(w, 4, gen).cuda()
    with torch.cuda.stream(s):
        ix.ice_build(K, V)
        r = ix.ice_decode(Q, 256, 16)
    torch.cuda.synchronize()
    out = gs.run_decode(ix, Q, 256, 16)
    assert np.array_equal(r[0].cpu().numpy(), out["sel"]) and np.array_equal(r[1].cpu().numpy(), out["uni"])
    gs.compare_decode(ix, refs, out)


def test_pipelined_ranges_on_two_streams():
    """Two ranges of 20 heads (each pipelined over ranges of its own) built at
    the same time on two streams share the handle's one second stream; the
    index equals a one-stream build bit for bit."""
    from ann_retrieval_amd.api import IceIndex
    H, N, d, seed = 40, 2400, 128, 33
    say(f"pipelined ranges on two streams H={H} N={N} d={d} bf16")
    w, gen = synth.clustered_kv(H, N, d, 24, "bf16", seed, device="cpu")
    K, V = w.K.cuda(), w.V.cuda()
    ix = IceIndex(H, 4, d, "bf16", N + 8, seed=seed, max_budget=256)
    ix.ice_build_timed(K, V)
    torch.cuda.synchronize()
    one = ix.blob.clone()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(2):
        for i, h0 in enumerate((0, 20)):
            ix.ice_build_heads(K[h0:h0 + 20], V[h0:h0 + 20], h0, stream=streams[i])
        torch.cuda.synchronize()
        assert torch.equal(one, ix.blob), "concurrent pipelined range builds differ from the one-stream build"


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_reuse_layout_across_layers(dtype, d):
    """Heads 2, 3 (a second layer) take the layout of heads 0, 1 and their own
    rows: the structure equals the source's bit for bit, the lift and the page
    pool are their own, and select + attend match the oracle's reused index."""
    import gpu_support as gs
    from ann_retrieval_amd.api import IceIndex
    from oracle import icecache as ic
    H, N = 4, 1800
    say(f"reuse across layers H={H} N={N} d={d} {dtype}")
    w, gen = synth.clustered_kv(H, N, d, 16, dtype, 25, device="cpu")
    K, V = w.K.cuda(), w.V.cuda()
    ix = IceIndex(H, 2, d, dtype, N + 8, seed=25, max_budget=128)
    ix.ice_build_heads(K[:2], V[:2], 0)
    ix.ice_build_reuse(K[2:], V[2:], 2, 0)
    torch.cuda.synchronize()
    refs = gs.check_build(w, ix, [0, 1], 25, 3, 4)
    for h in (2, 3):
        g, s = gs.read_head(ix, h), gs.read_head(ix, h - 2)
        assert np.array_equal(g.lev, s.lev) and g.L_top == s.L_top and g.n_top == s.n_top
        assert all(np.array_equal(a, b) for a, b in zip(g.parent, s.parent))
        for ta, tb in zip(g.tables, s.tables):
            assert np.array_equal(ta["tok"], tb["tok"])
        ref = ic.build_head_reuse(gs.to64(w.K[h]), gs.to64(w.V[h]), refs[h - 2], h)
        assert abs(g.stats["M2"] - ref.M2) <= 1e-12 * max(ref.M2, 1e-300)
        assert np.allclose(g.e, ref.e, rtol=2e-6, atol=2e-6 * np.sqrt(ref.M2))
        assert g.stats["near_ties"] == 0 and g.stats["splits"] == 0
        P = len(g.tables[0]["pages"])
        nd = np.int16 if dtype == "bf16" else np.int32
        kp = ix.export(h, L.ICE_EXP_PAGE_K, 0, np_dtype=nd).reshape(-1, 16, d)[:P]
        vp = ix.export(h, L.ICE_EXP_PAGE_V, 0, np_dtype=nd).reshape(-1, 16, d)[:P]
        tok = g.tables[0]["tok"]
        valid = tok >= 0
        assert np.array_equal(kp[valid], gs.raw_rows(w.K[h])[tok[valid]])
        assert np.array_equal(vp[valid], gs.raw_rows(w.V[h])[tok[valid]])
        refs[h] = ref
    for _ in range(2):
        gs.check_decode(w, ix, refs, synth.decode_queries(w, 2, gen), 128, 8)
    # the source must be built and hold the same count; ranges must not overlap
    with pytest.raises(L.IceError):
        ix.ice_build_reuse(K[1:3], V[1:3], 1, 0)


def test_reused_head_inserts_are_bounded_by_its_tables():
    """A head built by reuse holds its source's promotion levels for the
    tokens it was built with and its own draws after them, so its level
    counts can outgrow tables sized from either head's own draws. With seed
    1, two heads, 2 levels and capacity 4096, a reuse at 2048 tokens would
    hold 262 level-1 points at token 3992 against 261 slots (the prediction
    is worked from the oracle's draws in test_abi.py): inserts up to token
    3991 succeed and stay within the tables, the insert of token 3992 is
    refused with ICE_ERR_CAPACITY and changes nothing."""
    import gpu_support as gs
    from ann_retrieval_amd.api import IceIndex
    H, N, d, cap, seed = 2, 2048, 64, 4096, 1
    say(f"reuse then insert to capacity H={H} N={N} cap={cap} levels=2 seed={seed}")
    w, gen = synth.clustered_kv(H, N, d, 8, "f32", seed, device="cpu")
    ix = IceIndex(H, 2, d, "f32", cap, 2, 4, seed, max_budget=64)
    ix.ice_build_heads(w.K[:1].cuda(), w.V[:1].cuda(), 0)
    ix.ice_build_reuse(w.K[1:].cuda(), w.V[1:].cuda(), 1, 0)
    torch.cuda.synchronize()
    g0 = torch.Generator().manual_seed(3)
    limit = 3992
    t = N
    while t < limit:
        n = min(256, limit - t)
        k = torch.randn(H, n, d, generator=g0).cuda()
        ix.ice_insert(k, k)
        t += n
    torch.cuda.synchronize()
    assert ix.n_tokens() == limit
    for h in range(H):
        st = ix.stats(h)
        assert st["overflow"] == 0 and st["n_tokens"] == limit
        gs.check_table_structure(gs.read_head(ix, h), ix.capacity)
    assert ix.stats(1)["n_top"] == 261
    before = gs.read_head(ix, 1)
    k = torch.randn(H, 1, d, generator=g0).cuda()
    with pytest.raises(L.IceError) as e:
        ix.ice_insert(k, k)
    assert e.value.code == L.ICE_ERR_CAPACITY
    after = gs.read_head(ix, 1)
    assert ix.n_tokens() == limit and after.n_top == before.n_top
    assert after.tables[0]["pages"] == before.tables[0]["pages"]
