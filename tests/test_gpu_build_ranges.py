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
    Q = synth.decode_queries(w, 4, gen).cuda()
    r1 = full.ice_decode(Q, 256, 16)
    r2 = part.ice_decode(Q, 256, 16)
    torch.cuda.synchronize()
    for x, y in zip(r1[:3], r2[:3]):
        assert torch.equal(x, y)
    # the fused step's attention sums pages in the order its waves take them
    den = r1[3].abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    assert float(((r1[3] - r2[3]).abs() / den).max()) <= 1e-5
    # a range build must keep the index's token count
    with pytest.raises(L.IceError):
        part.ice_build_heads(K[:2, :N - 1], V[:2, :N - 1], 0)
