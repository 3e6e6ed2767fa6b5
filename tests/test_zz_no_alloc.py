"""The allocation-free build (ice_build_noalloc, the library's fixed device
scratch instead of a caller workspace) against ice_build, through the C ABI:
two calls in a row on one index, the second with fewer tokens, each compared
bit for bit with ice_build on the same input; and the size limit. Every case
prints its name and shape before it touches the GPU."""
import numpy as np
import pytest
import torch

from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import say  # noqa: E402

def same_index(a, b, H, d, elt):
    """Every array the build defines, over the part it defines (the rest of
    the blob is whatever memory the allocator handed out)."""
    for h in range(H):
        sa, sb = a.stats(h), b.stats(h)
        assert sa == sb, f"head {h} header"
        n, n_top, (p0, p1) = sa["n_tokens"], sa["n_top"], sa["n_pages"][:2]
        row = 16 * d * elt
        for what, lv, nbytes in [(L.ICE_EXP_LEVEL, 0, n), (L.ICE_EXP_LIFT, 0, 4 * n), (L.ICE_EXP_PARENT, 0, 4 * n),
                                 (L.ICE_EXP_PARENT, 1, 4 * n), (L.ICE_EXP_PAGE_TOK, 0, 64 * p0),
                                 (L.ICE_EXP_PAGE_TOK, 1, 64 * p1), (L.ICE_EXP_PAGE_CNT, 0, 4 * p0),
                                 (L.ICE_EXP_PAGE_NEXT, 0, 4 * p0), (L.ICE_EXP_PAGE_OWNER, 0, 4 * p0),
                                 (L.ICE_EXP_OWNER_FIRST, 0, None), (L.ICE_EXP_OWNER_RUN, 0, None),
                                 (L.ICE_EXP_OWNER_COUNT, 0, None), (L.ICE_EXP_TOP, 0, 4 * n_top),
                                 (L.ICE_EXP_PAGE_K, 0, row * p0), (L.ICE_EXP_PAGE_K, 1, row * p1),
                                 (L.ICE_EXP_PAGE_V, 0, row * p0)]:
            x = a.export(h, what, lv, np_dtype=np.uint8)[:nbytes]
            y = b.export(h, what, lv, np_dtype=np.uint8)[:nbytes]
            assert np.array_equal(x, y), f"head {h} export {what} level {lv}"


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_noalloc_build_equals_build_twice(dtype, d):
    from ann_retrieval_amd.api import IceIndex
    H, N1, N2, cap, seed = 8, 6000, 2500, 6016, 31
    say(f"noalloc build H={H} N={N1} then {N2} d={d} {dtype}")
    w, gen = synth.clustered_kv(H, N1, d, 48, dtype, seed, device="cpu")
    K, V = w.K.cuda(), w.V.cuda()
    a = IceIndex(H, 4, d, dtype, cap, seed=seed, max_budget=128)
    b = IceIndex(H, 4, d, dtype, cap, seed=seed, max_budget=128)
    for n in (N1, N2):
        Kn, Vn = K[:, :n].contiguous(), V[:, :n].contiguous()
        a.ice_build_noalloc(Kn, Vn)
        b.ice_build(Kn, Vn)
        torch.cuda.synchronize()
        same_index(a, b, H, d, 2 if dtype == "bf16" else 4)
        Q = synth.decode_queries(w, 4, gen).cuda()
        ra, rb = a.ice_decode(Q, 128, 8), b.ice_decode(Q, 128, 8)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(ra, rb))
        say(f"noalloc build of {n} tokens equals ice_build")


def test_noalloc_rejects_builds_beyond_its_scratch():
    from ann_retrieval_amd.api import IceIndex
    say("noalloc size limit: 8 heads x 200k tokens")
    ix = IceIndex(8, 4, 128, "bf16", 200000, seed=0, max_budget=64)
    K = torch.zeros(8, 16, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.IceError) as e:
        ix.ice_build_noalloc(K, K)
    assert e.value.code == L.ICE_ERR_CAPACITY
    assert ix.n_tokens() == 0
