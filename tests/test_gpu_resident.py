"""Resident (sink and window) tokens and dense heads, GPU against the oracle
through the C ABI: the fused decode kernel with resident pages, the separate
select and attend kernels with dense heads, fp32 and bf16, clearing, and
rebuilds keeping both settings. Every case prints its name and shape before
it touches the GPU.
"""
import numpy as np
import pytest
import torch

import gpu_support as gs
from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import build_case, check_build, say  # noqa: E402


def _decode(ix, Q, budget, beam):
    """ice_decode, with the selection's trace from ice_select for the replay."""
    Qd = Q.cuda()
    sel, uni, nuni, O, lse = ix.ice_decode(Qd, budget, beam)
    s2, u2, n2, tr = ix.ice_select(Qd, budget, beam, trace=True)
    torch.cuda.synchronize()
    assert torch.equal(sel, s2) and torch.equal(uni, u2) and torch.equal(nuni, n2)
    return dict(Q=Q.cpu(), budget=budget, beam=beam, scale=None, sel=sel.cpu().numpy(), uni=uni.cpu().numpy(),
                nuni=nuni.cpu().numpy(), tr=tr.cpu().numpy(), O=O.cpu().double().numpy(),
                lse=lse.cpu().double().numpy())


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", d=128, G=4, budget=256, beam=16, n_res=70, cap=96),    # the fused decode kernel
    dict(dtype="bf16", d=64, G=2, budget=64, beam=4, n_res=16, cap=16),       # one full resident page
    dict(dtype="f32", d=64, G=1, budget=64, beam=4, n_res=37, cap=40),        # fp32 kernels
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_resident_tokens(case):
    w, gen, ix = build_case(3, 2500, case["d"], case["dtype"], 24, 21, G=case["G"], budget=case["budget"],
                            resident=case["cap"])
    refs = check_build(w, ix, [0, 1, 2], 21, 3, 4)
    Kr, Vr = synth.resident_tokens(w, case["n_res"], gen)
    say(f"resident n={case['n_res']} {case}")
    ix.set_resident(Kr.cuda(), Vr.cuda())
    for h in range(3):
        assert ix.stats(h)["n_resident"] == case["n_res"]
    for _ in range(2):
        Q = synth.decode_queries(w, case["G"], gen)
        gs.compare_decode(ix, refs, _decode(ix, Q, case["budget"], case["beam"]), resident=(Kr, Vr))
        # the attend call on its own attends the resident tokens too
        out = gs.run_decode(ix, Q, case["budget"], case["beam"])
        gs.compare_decode(ix, refs, out, resident=(Kr, Vr))
    # clearing returns to the pages alone
    say("resident cleared")
    ix.set_resident(None, None)
    Q = synth.decode_queries(w, case["G"], gen)
    gs.compare_decode(ix, refs, _decode(ix, Q, case["budget"], case["beam"]))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_dense_heads(dtype, d):
    w, gen, ix = build_case(4, 1800, d, dtype, 16, 22, G=2, budget=128, resident=32)
    refs = check_build(w, ix, [0, 1, 2, 3], 22, 3, 4)
    Kr, Vr = synth.resident_tokens(w, 20, gen)
    say(f"dense heads 1 and 3, resident 20, {dtype} d={d}")
    ix.set_dense([False, True, False, True])
    ix.set_resident(Kr.cuda(), Vr.cuda())
    assert [ix.stats(h)["dense"] for h in range(4)] == [0, 1, 0, 1]
    for _ in range(2):
        Q = synth.decode_queries(w, 2, gen)
        gs.compare_decode(ix, refs, _decode(ix, Q, 128, 8), resident=(Kr, Vr), dense={1, 3})
    # a rebuild keeps the dense flags and the resident tokens
    say("rebuild keeps dense flags and resident tokens")
    ix.ice_build(w.K.cuda(), w.V.cuda())
    torch.cuda.synchronize()
    assert [ix.stats(h)["dense"] for h in range(4)] == [0, 1, 0, 1]
    assert all(ix.stats(h)["n_resident"] == 20 for h in range(4))
    Q = synth.decode_queries(w, 2, gen)
    gs.compare_decode(ix, refs, _decode(ix, Q, 128, 8), resident=(Kr, Vr), dense={1, 3})
    ix.set_dense(None)
    Q = synth.decode_queries(w, 2, gen)
    gs.compare_decode(ix, refs, _decode(ix, Q, 128, 8), resident=(Kr, Vr))


def test_resident_argument_errors():
    w, gen, ix = build_case(2, 300, 64, "bf16", 8, 23, G=2, budget=64, resident=20)
    Kr, Vr = synth.resident_tokens(w, 21, gen)
    say("resident argument errors")
    with pytest.raises(L.IceError):
        ix.set_resident(Kr.cuda(), Vr.cuda())          # more than params.resident
    with pytest.raises(ValueError):
        ix.set_dense([True])                           # wrong length
    assert ix.stats(0)["n_resident"] == 0



def test_pipelined_rebuild_keeps_resident_and_dense():
    """A rebuild of 24 heads runs as the two-stream pipeline over 3 ranges; it
    keeps every head's resident tokens and dense flag like the one-stream
    rebuild, and the heads at the ranges' edges decode as the oracle does."""
    H, N, G = 24, 2000, 4
    w, gen, ix = build_case(H, N, 128, "bf16", 16, 23, G=G, budget=128, resident=48)
    heads = [0, 7, 8, 15, 16, 23]
    refs = check_build(w, ix, heads, 23, 3, 4)
    Kr, Vr = synth.resident_tokens(w, 40, gen)
    dense = [h % 5 == 3 for h in range(H)]
    say(f"pipelined rebuild H={H}: resident 40, dense heads {[h for h in range(H) if dense[h]]}")
    ix.set_dense(dense)
    ix.set_resident(Kr.cuda(), Vr.cuda())
    ix.ice_build(w.K.cuda(), w.V.cuda())
    torch.cuda.synchronize()
    assert [bool(ix.stats(h)["dense"]) for h in range(H)] == dense
    assert all(ix.stats(h)["n_resident"] == 40 for h in range(H))
    Q = synth.decode_queries(w, G, gen)
    out = gs.run_decode(ix, Q, 128, 8)
    gs.compare_decode(ix, {h: refs[h] for h in heads}, out, resident=(Kr, Vr),
                      dense={h for h in heads if dense[h]})
