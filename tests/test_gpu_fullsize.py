"""GPU vs oracle parity at the benchmark workloads' full sizes, in the launch
configuration bench.py times (all heads in one select and one attend launch).

The oracle cannot redo every head at these sizes in seconds, so each case
builds and decodes every head on the GPU and compares sampled heads with the
oracle one by one. Every head's outputs are also checked for properties that
hold at any size: selected pages exist and are distinct, the union is the
sorted set of the group's selections, attention outputs are finite.
"""
import numpy as np
import pytest
import torch

import bench
import gpu_support as gs
from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth
from gpu_support import check_build, compare_decode, run_decode, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from ann_retrieval_amd.api import IceIndex  # noqa: E402

DEV = torch.device("cuda", 0)


def check_all_heads(ix, out):
    """Properties of every head's select and attend outputs."""
    sel, uni, nuni, O = out["sel"], out["uni"], out["nuni"], out["O"]
    H = sel.shape[0]
    n_pages = np.array([ix.stats(h)["n_pages"][0] for h in range(H)])
    for h in range(H):
        s = sel[h]
        for g in range(s.shape[0]):
            ids = s[g][s[g] >= 0]
            assert len(set(ids.tolist())) == len(ids), f"head {h} q {g}: a page selected twice"
            assert np.all(ids < n_pages[h]) and np.all(s[g][len(ids):] == -1)
        want = sorted(set(int(x) for x in s.ravel() if x >= 0))
        assert int(nuni[h]) == len(want) and list(uni[h, :len(want)]) == want
        assert np.all(uni[h, len(want):] == -1)
    assert np.isfinite(O).all()
    say(f"all {H} heads: outputs well formed")


def test_ctx36k_sampled_heads():
    """The benchmark's 36k-token workload: 256 heads x 36,000 tokens, G=4,
    d=128 bf16, rotated 512-component mixtures, one build and decode steps at
    budgets 256 and 64; heads 0, 137 and 255 against the oracle."""
    H, G, N, d, dtype, C, rotate, _ = bench.WORKLOADS["ctx36k"]
    say(f"ctx36k H={H} G={G} N={N} d={d} {dtype}")
    w, gen = synth.clustered_kv(H, N, d, C, dtype, 0, device=DEV, rotate=rotate)
    ix = IceIndex(H, G, d, dtype, N + 60, seed=0, max_budget=256, device=DEV)
    ix.ice_build(w.K, w.V)
    torch.cuda.synchronize()
    refs = check_build(w, ix, [0, 137, 255], 0, 3, 4)
    for budget in (256, 64):
        Q = synth.decode_queries(w, G, gen, device=DEV)
        out = run_decode(ix, Q, budget, budget // 16)
        compare_decode(ix, refs, out)
        check_all_heads(ix, out)
        # the fused decode step, in the benchmark's launch configuration
        s1, u1, n1, O1, l1 = ix.ice_decode(Q, budget, budget // 16)
        torch.cuda.synchronize()
        assert np.array_equal(s1.cpu().numpy(), out["sel"]) and np.array_equal(u1.cpu().numpy(), out["uni"])
        O1 = O1.cpu().double().numpy()
        den = np.abs(out["O"]).max(axis=-1, keepdims=True)
        assert float((np.abs(O1 - out["O"]) / np.maximum(den, 1e-30)).max()) <= 1e-5
        say(f"ctx36k budget {budget}: fused decode equals select + attend")


def test_llama_layer_decode_with_inserts():
    """One Llama-shaped layer (8 KV heads x 4 query heads, 32,768 tokens,
    d=128 bf16), 128 decode steps of select + attend then one insert per KV
    head; heads 0 and 5 replayed by the oracle insert by insert, with
    decode checks at steps 0, 64 and 127 and the final layout compared."""
    H, G, N, d, dtype, C, rotate, _ = bench.WORKLOADS["llama-layer"]
    steps, checks = 128, (0, 64, 127)
    say(f"llama layer H={H} G={G} N={N} + {steps} steps")
    w, gen = synth.clustered_kv(H, N, d, C, dtype, 0, device=DEV, rotate=rotate)
    ix = IceIndex(H, G, d, dtype, N + steps, seed=0, max_budget=256, device=DEV)
    ix.ice_build(w.K, w.V)
    torch.cuda.synchronize()
    heads = [0, 5]
    refs = check_build(w, ix, heads, 0, 3, 4)
    outs, ks, vs = {}, [], []
    for s in range(steps):
        Q = synth.decode_queries(w, G, gen, device=DEV)
        if s in checks:
            outs[s] = run_decode(ix, Q, 256, 16)
            check_all_heads(ix, outs[s])
        else:
            _, uni, nuni = ix.ice_select(Q, 256, 16)
            ix.ice_attend(Q, uni, nuni)
        k, v = synth.new_tokens(w, gen, device=DEV)
        ix.ice_insert(k, v)
        ks.append(k)
        vs.append(v)
    torch.cuda.synchronize()
    Kn, Vn = torch.cat(ks, 1).cpu(), torch.cat(vs, 1).cpu()
    for h in heads:
        g = gs.read_head(ix, h)
        ref = refs[h]
        for s in range(steps):
            if s in checks:
                compare_decode(ix, {h: ref}, outs[s])
            gs.replay_inserts(ref, g, Kn[h, s:s + 1], Vn[h, s:s + 1], h, 0, 3, 4)
        gs.check_table_structure(g, ix.capacity)
        gs.compare_layout(ref, g, ix.capacity)
        assert g.n == N + steps
        assert g.stats["splits"] == ref.splits and g.stats["clamps"] == ref.clamps
    say("llama layer: inserts replayed, layouts equal")


@pytest.mark.parametrize("depth", [0.1, 0.3, 0.5, 0.7, 0.9])
def test_needle_100k(depth):
    """Needle workload: 8 KV heads x 4 query heads, 100,000 tokens, d=128
    bf16, 1024-component background, a 16-token span with cosine 0.9 to query
    head 0's query, budget 64. Head 0 is checked against the oracle at depth
    0.5; at every depth the coverage of the needle by query head 0's pages is
    reported, with the smallest beam that reaches it."""
    H, G, N, d = 8, 4, 100000, 128
    say(f"needle depth={depth} H={H} N={N}")
    w, Q, start = synth.needle_workload(H, G, N, d, 1024, depth, seed=0, device=DEV)
    ix = IceIndex(H, G, d, "bf16", N, seed=0, max_budget=64, device=DEV)
    ix.ice_build(w.K, w.V)
    torch.cuda.synchronize()
    out = run_decode(ix, Q, 64, 4)
    check_all_heads(ix, out)
    if depth == 0.5:
        refs = check_build(w, ix, [0], 0, 3, 4)
        compare_decode(ix, refs, out)
    needle = set(range(start, start + 16))
    covered = []
    for h in range(H):
        tok = ix.export(h, L.ICE_EXP_PAGE_TOK, 0).reshape(-1, 16)
        hit = {int(t) for p in out["sel"][h, 0] if p >= 0 for t in tok[p] if t in needle}
        first_beam = None
        for beam in (4, 8, 16, 32, 64, 128, 256):
            sel = ix.ice_select(Q, 64, beam)[0].cpu().numpy()
            if any(t in needle for p in sel[h, 0] if p >= 0 for t in tok[p]):
                first_beam = beam
                break
        covered.append((len(hit), first_beam))
    say(f"needle depth={depth}: tokens covered per head (beam 4) and smallest beam reaching it: {covered}")


def test_qwen_shaped_long_generation():
    """Qwen3-32B-shaped long generation: 512 heads (64 layers x 8 KV heads),
    8 query heads each, 8,192-token prompt, 4,096 steps of select + attend at
    budget 256 then one insert per head, queries and new keys walking between
    mixture centres so pages split. Heads 0 and 300 are replayed by the oracle
    through step 1,023 with decode checks at steps 0, 512 and 1,023; every head
    is checked for structure and counts after all 4,096 steps."""
    H, G, N, d, C = 512, 8, 8192, 128, 512
    steps, replayed, checks = 4096, 1024, (0, 512, 1023)
    say(f"qwen-shaped H={H} G={G} N={N} + {steps} steps")
    w, gen = synth.clustered_kv(H, N, d, C, "bf16", 0, device=DEV)
    ix = IceIndex(H, G, d, "bf16", N + steps, seed=0, max_budget=256, device=DEV)
    ix.ice_build(w.K, w.V)
    torch.cuda.synchronize()
    heads = [0, 300]
    refs = check_build(w, ix, heads, 0, 3, 4)
    walk = synth.QueryWalk(w, G, gen, device=DEV)
    outs, ks, vs = {}, [], []
    for s in range(steps):
        Q, k, v = walk.step()
        if s in checks:
            outs[s] = run_decode(ix, Q, 256, 16)
            check_all_heads(ix, outs[s])
        else:
            _, uni, nuni = ix.ice_select(Q, 256, 16)
            ix.ice_attend(Q, uni, nuni)
        ix.ice_insert(k, v)
        if s < replayed:
            ks.append(k[heads].cpu())
            vs.append(v[heads].cpu())
        if s % 1024 == 1023:
            torch.cuda.synchronize()
            say(f"step {s + 1} of {steps}")
    torch.cuda.synchronize()
    Kn, Vn = torch.cat(ks, 1), torch.cat(vs, 1)
    for i, h in enumerate(heads):
        g = gs.read_head(ix, h)
        ref = refs[h]
        for s in range(replayed):
            if s in checks:
                compare_decode(ix, {h: ref}, outs[s])
            gs.replay_inserts(ref, g, Kn[i, s:s + 1], Vn[i, s:s + 1], h, 0, 3, 4)
        say(f"head {h}: {replayed} inserts replayed, {ref.splits} splits")
    splits = 0
    for h in range(H):
        st = ix.stats(h)
        assert st["n_tokens"] == N + steps and st["overflow"] == 0
        splits += st["splits"]
    for h in heads:
        g = gs.read_head(ix, h)
        gs.check_table_structure(g, ix.capacity)
        members = sorted(t for p in g.tables[0]["pages"] for t in p)
        assert members == list(range(N + steps)), "every token in exactly one page"
    assert splits > 0
    say(f"qwen-shaped: {splits} page splits over {H} heads")
