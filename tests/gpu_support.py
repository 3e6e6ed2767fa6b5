"""Helpers of the GPU parity tests: read a head's layout out of the library,
rebuild the oracle's view of the same head, and compare the two under the
near-tie protocol.

Comparison protocol (near-tie band 1e-4 relative, from the method's parity
contract):

* promotion levels, the top list and page ids must match exactly;
* a parent may differ from the oracle's only when the GPU's choice is within
  the band of the best lifted distance (``|D_gpu - D1| <= 1e-4 * max(D_gpu, D1)``,
  in either direction, so a GPU parent that beats the oracle's fails); such
  choices are counted, and the oracle then continues with the GPU's choice;
* inside an owner, slots may differ only between tokens whose distances to the
  owner are within the band (counted);
* a selection cut may keep a different set only through near-tied items
  (counted); the oracle then continues from the GPU's kept set, so ``sel`` and
  ``uni`` must match exactly afterwards;
* attention: max_i |o_gpu - o_ref| / max_i |o_ref| per (head, query head)
  within 2e-3 for bf16 K/V and 1e-5 for fp32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

from oracle import icecache as ic
from ann_retrieval_amd import _lib as L
from ann_retrieval_amd import synth

BAND = ic.NEAR_TIE_REL
ATOL = {"bf16": 2e-3, "f32": 1e-5}


def to64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().double().numpy()


@dataclasses.dataclass
class GpuHead:
    n: int
    L_top: int
    n_top: int
    lev: np.ndarray
    e: np.ndarray
    parent: list
    tables: list          # per table: dict(pages, owner, first, next, cnt)
    top: list
    stats: dict


def read_head(ix, h: int) -> GpuHead:
    st = ix.stats(h)
    n, Lt = st["n_tokens"], st["top_level"]
    lev = ix.export(h, L.ICE_EXP_LEVEL, np_dtype=np.int8)[:n].astype(np.int64)
    e = ix.export(h, L.ICE_EXP_LIFT, np_dtype=np.float32)[:n].astype(np.float64)
    ntab = max(1, ix.levels - 1)
    parent = [ix.export(h, L.ICE_EXP_PARENT, l)[:n].astype(np.int64) for l in range(min(Lt, ntab))]
    tables = []
    for l in range(ntab):
        P = st["n_pages"][l]
        tok = ix.export(h, L.ICE_EXP_PAGE_TOK, l).reshape(-1, L.ICE_PAGE_CAP)[:P]
        cnt = ix.export(h, L.ICE_EXP_PAGE_CNT, l)[:P]
        tables.append(dict(
            tok=tok, cnt=cnt, pages=[[int(x) for x in tok[p, :cnt[p]]] for p in range(P)],
            next=ix.export(h, L.ICE_EXP_PAGE_NEXT, l)[:P], owner=ix.export(h, L.ICE_EXP_PAGE_OWNER, l)[:P],
            first=ix.export(h, L.ICE_EXP_OWNER_FIRST, l), tail=ix.export(h, L.ICE_EXP_OWNER_TAIL, l),
            run=ix.export(h, L.ICE_EXP_OWNER_RUN, l), count=ix.export(h, L.ICE_EXP_OWNER_COUNT, l)))
    top = [int(x) for x in ix.export(h, L.ICE_EXP_TOP)[:st["n_top"]]] if st["n_top"] > 0 else []
    return GpuHead(n=n, L_top=Lt, n_top=st["n_top"], lev=lev, e=e, parent=parent, tables=tables, top=top,
                   stats=st)


def owner_chain(tab: dict, owner_slot: int) -> list:
    out, p = [], int(tab["first"][owner_slot])
    while p >= 0:
        out.append(p)
        p = int(tab["next"][p])
    return out


def check_table_structure(g: GpuHead, cap: int):
    """Chains, owners and counts of every table are self-consistent."""
    for l, tab in enumerate(g.tables):
        P = len(tab["pages"])
        seen = np.zeros(P, dtype=np.int64)
        owners = set(int(o) for o in tab["owner"])
        for o in owners:
            slot = cap if o == ic.ROOT else o
            chain = owner_chain(tab, slot)
            assert chain, f"table {l}: owner {o} has no chain"
            assert int(tab["tail"][slot]) == chain[-1]
            # the owner's member count, and its contiguous run of pages from first[]
            assert int(tab["count"][slot]) == int(sum(tab["cnt"][p] for p in chain))
            run = int(tab["run"][slot])
            assert 1 <= run <= len(chain) and chain[:run] == list(range(chain[0], chain[0] + run))
            for i, p in enumerate(chain):
                seen[p] += 1
                assert int(tab["owner"][p]) == o
                assert 1 <= tab["cnt"][p] <= L.ICE_PAGE_CAP
                if i + 1 < len(chain):
                    assert tab["cnt"][p] == L.ICE_PAGE_CAP, "only an owner's last page may be partly filled"
        assert np.all(seen == 1), f"table {l}: a page is on no chain or on two"
        for p in range(P):
            assert np.all(tab["tok"][p, tab["cnt"][p]:] == -1)


def validate_parents(ref: ic.HeadIndex, g: GpuHead):
    """Compares parents level by level. Returns (parents to replay, near-tie count)."""
    X = ref.X()
    replay, ties = [], 0
    for l in range(ref.L_top):
        po, pg = ref.parent[l], g.parent[l]
        par = po.copy()
        diff = np.nonzero(po != pg)[0]
        for i in diff:
            i = int(i)
            assert ref.lev[i] == l, f"level {l}: token {i} (level {ref.lev[i]}) has parent {pg[i]} != {po[i]}"
            j = int(pg[i])
            assert 0 <= j < ref.n and ref.lev[j] >= l + 1, f"level {l}: parent {j} of {i} is not a level-{l+1} point"
            dg = float(((X[i] - X[j]) ** 2).sum())
            d1 = float(ref.dist[l][i])
            assert abs(dg - d1) <= BAND * max(dg, d1), (f"level {l}: token {i} parent {j} (D={dg:.9g}) vs oracle "
                                                       f"{po[i]} (D={d1:.9g}) outside the near-tie band")
            par[i] = j
            ties += 1
        replay.append(par)
    return replay, ties


def oracle_replay(K64, V64, h, seed, levels, plog2, replay_parents):
    return ic.build_head(K64, V64, h, seed, levels, plog2, 16, parents=replay_parents)


def compare_layout(ref: ic.HeadIndex, g: GpuHead, cap: int) -> int:
    """Exact page ids / owners / top list; slot differences only between
    near-equal distances. Returns the number of such slot differences."""
    assert g.L_top == ref.L_top
    assert g.top == ref.top
    swaps = 0
    tab = g.tables[0]
    assert len(tab["pages"]) == len(ref.pages), f"{len(tab['pages'])} pages vs oracle {len(ref.pages)}"
    assert [int(o) for o in tab["owner"]] == [int(o) for o in ref.page_owner]
    for owner, pids in ref.owner_pages.items():
        slot = cap if owner == ic.ROOT else owner
        assert owner_chain(tab, slot) == list(pids), f"owner {owner}: page chain differs"
        seq_o = [t for p in pids for t in ref.pages[p]]
        seq_g = [t for p in pids for t in tab["pages"][p]]
        assert sorted(seq_o) == sorted(seq_g), f"owner {owner}: different members"
        if seq_o != seq_g:
            d = ref.dist[0] if ref.L_top >= 1 else None
            for a, b in zip(seq_o, seq_g):
                if a != b:
                    assert d is not None, "root pages must be in token order"
                    da, db = float(d[a]), float(d[b])
                    assert abs(da - db) <= BAND * max(da, db), f"owner {owner}: slot order {a} vs {b} not a near-tie"
                    swaps += 1
    for l in range(1, ref.L_top):
        tl = g.tables[l]
        for owner, kids in ref.children[l].items():
            got = [t for p in owner_chain(tl, owner) for t in tl["pages"][p]]
            assert sorted(got) == sorted(kids), f"level {l} owner {owner}: different children"
            if got != kids:
                for a, b in zip(kids, got):
                    if a != b:
                        da, db = float(ref.dist[l][a]), float(ref.dist[l][b])
                        assert abs(da - db) <= BAND * max(da, db)
                        swaps += 1
    return swaps


def adopt_gpu_slots(ref: ic.HeadIndex, g: GpuHead):
    """After compare_layout accepted near-tie slot swaps, take the GPU's slots
    so the selection and attention checks see the same page contents."""
    ref.pages = [list(p) for p in g.tables[0]["pages"]]
    for l in range(1, ref.L_top):
        tl = g.tables[l]
        for owner in list(ref.children[l].keys()):
            ref.children[l][owner] = [t for p in owner_chain(tl, owner) for t in tl["pages"][p]]


def compare_selection(ref: ic.HeadIndex, q64, budget, beam, sel_g, trace_g):
    """Oracle select, continuing from the GPU's kept sets where they differ by
    near-ties only. Returns 1 if any cut needed that, else 0."""
    n_cuts = ref.L_top if ref.n > 0 else 0
    got = [int(x) for x in sel_g if x >= 0]
    kept_g = [[int(x) for x in trace_g[c] if x >= 0] for c in range(n_cuts)]
    free = ic.select(ref, q64, budget, beam)
    if free["kept"] == kept_g and free["sel"] == got:
        return 0
    r = ic.select(ref, q64, budget, beam, forced=kept_g + [None])
    assert r["admissible"], f"kept sets {kept_g} vs oracle {free['kept']} beyond the near-tie band"
    if got != r["sel"]:
        r2 = ic.select(ref, q64, budget, beam, forced=kept_g + [got])
        assert r2["admissible"], f"sel {got} vs oracle {r['sel']} beyond the near-tie band"
    return 1


def attn_error(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    den = np.abs(o_ref).max()
    return float(np.abs(o_gpu - o_ref).max() / den) if den > 0 else float(np.abs(o_gpu).max())


# ---- whole-case helpers ----------------------------------------------------

def say(*a):
    print("[case]", *a, flush=True)


def build_case(H, N, d, dtype, C, seed, G=4, levels=3, plog2=4, capacity=None, budget=256, rotate=False,
               resident=0):
    from ann_retrieval_amd.api import IceIndex
    say(f"build H={H} N={N} d={d} {dtype} C={C} seed={seed} G={G} L={levels} p=2^-{plog2} resident={resident}")
    w, gen = synth.clustered_kv(H, N, d, C, dtype, seed, device="cpu", rotate=rotate)
    ix = IceIndex(H, G, d, dtype, capacity or max(N, 1), levels, plog2, seed, max_budget=budget, resident=resident)
    ix.ice_build(w.K.cuda(), w.V.cuda())
    torch.cuda.synchronize()
    return w, gen, ix


def raw_rows(x: torch.Tensor) -> np.ndarray:
    """Raw bits of rows, for bit-exact copies."""
    return (x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)).cpu().numpy()


def check_build(w, ix, heads, seed, levels, plog2, check_pool=True):
    """Levels exact, lift close, parents within the band, layout exact (near-tie
    slot swaps counted), page pool rows bit-exact. Returns oracle indexes."""
    refs, ties, swaps = {}, 0, 0
    for h in heads:
        g = read_head(ix, h)
        K64, V64 = to64(w.K[h]), to64(w.V[h])
        ref = ic.build_head(K64, V64, h, seed, levels, plog2)
        assert g.n == ref.n
        assert np.array_equal(g.lev, ref.lev), "promotion levels differ"
        assert g.L_top == ref.L_top and g.n_top == len(ref.top)
        assert abs(g.stats["M2"] - ref.M2) <= 1e-12 * max(ref.M2, 1e-300)
        if ref.n:
            assert np.allclose(g.e, ref.e, rtol=2e-6, atol=2e-6 * math.sqrt(ref.M2) + 1e-30)
        assert g.stats["overflow"] == 0
        check_table_structure(g, ix.capacity)
        replay, t = validate_parents(ref, g)
        if t:
            ref = oracle_replay(K64, V64, h, seed, levels, plog2, replay)
        ties += t
        s = compare_layout(ref, g, ix.capacity)
        if s:
            adopt_gpu_slots(ref, g)
        swaps += s
        if check_pool and ref.n:
            P = len(g.tables[0]["pages"])
            kp = ix.export(h, L.ICE_EXP_PAGE_K, 0, np_dtype=np.int16 if ix.dtype == "bf16" else np.int32)
            vp = ix.export(h, L.ICE_EXP_PAGE_V, 0, np_dtype=np.int16 if ix.dtype == "bf16" else np.int32)
            kp = kp.reshape(-1, 16, ix.d)[:P]
            vp = vp.reshape(-1, 16, ix.d)[:P]
            Kr, Vr = raw_rows(w.K[h]), raw_rows(w.V[h])
            tok = g.tables[0]["tok"]
            valid = tok >= 0
            assert np.array_equal(kp[valid], Kr[tok[valid]]) and np.array_equal(vp[valid], Vr[tok[valid]])
            assert not kp[~valid].any() and not vp[~valid].any()
        refs[h] = ref
    say(f"build parity ok: heads={len(heads)} parent near-ties={ties} slot swaps={swaps}")
    return refs


def run_decode(ix, Q, budget, beam, scale=None):
    """One select + attend through the library; host copies of every output."""
    say(f"decode budget={budget} beam={beam} Q={tuple(Q.shape)}")
    Qd = Q if Q.is_cuda else Q.cuda()
    sel, uni, nuni, tr = ix.ice_select(Qd, budget, beam, trace=True)
    O, lse = ix.ice_attend(Qd, uni, nuni, scale)
    torch.cuda.synchronize()
    return dict(Q=Q.cpu(), budget=budget, beam=beam, scale=scale, sel=sel.cpu().numpy(), uni=uni.cpu().numpy(),
                nuni=nuni.cpu().numpy(), tr=tr.cpu().numpy(), O=O.cpu().double().numpy(),
                lse=lse.cpu().double().numpy())


def check_decode(w, ix, refs, Q, budget, beam, scale=None):
    out = run_decode(ix, Q, budget, beam, scale)
    compare_decode(ix, refs, out)
    return out["sel"], out["uni"], out["nuni"]


def compare_decode(ix, refs, out, resident=None, dense=()):
    """Selections of the heads in `refs` exact after tie-tolerant replay, the
    union exact, attention within the dtype's tolerance. resident: optional
    (K_r, V_r) host tensors [H, n, d] attended beside the pages; dense: heads
    whose attention covers every indexed token."""
    Q, budget, beam, scale = out["Q"], out["budget"], out["beam"], out["scale"]
    sel, uni, nuni, tr, O, lse = out["sel"], out["uni"], out["nuni"], out["tr"], out["O"], out["lse"]
    scale = 1.0 / math.sqrt(ix.d) if scale is None else scale
    ties, worst = 0, 0.0
    for h, ref in refs.items():
        for g in range(ix.G):
            q64 = to64(Q[h, g])
            ties += compare_selection(ref, q64, budget, beam, sel[h, g], tr[h, g])
        # union: ascending unique pages of the group, -1 padded
        want = sorted(set(int(x) for x in sel[h].ravel() if x >= 0))
        assert int(nuni[h]) == len(want)
        assert list(uni[h, :len(want)]) == want and np.all(uni[h, len(want):] == -1)
        res = None if resident is None else (to64(resident[0][h]), to64(resident[1][h]))
        for g in range(ix.G):
            o_ref, lse_ref = ic.attend(ref, to64(Q[h, g]), want, scale, resident=res, dense=h in dense)
            if lse_ref > -np.inf:
                err = attn_error(O[h, g], o_ref)
                worst = max(worst, err)
                assert err <= ATOL[ix.dtype], f"head {h} q {g}: attention error {err:.3g}"
                assert abs(lse[h, g] - lse_ref) <= 1e-4 * max(1.0, abs(lse_ref))
            else:
                assert np.all(O[h, g] == 0) and lse[h, g] == -np.inf
    for h in refs:
        assert ix.stats(h)["sync_timeouts"] == 0, "a selection barrier wait hit its spin limit"
    say(f"decode parity ok: heads={len(refs)} selection near-ties={ties} worst attention error={worst:.3g}")
    return ties, worst


def decode_against_select_attend(ix, refs, Q, budget, beam, tag=""):
    """One ice_decode step: selections and unions equal ice_select's exactly,
    attention equals ice_attend's up to the order of fp32 sums, a second call
    gives the same bits, and the step matches the oracle (tie-tolerant)."""
    say(f"decode vs select+attend {tag} budget={budget} beam={beam} Q={tuple(Q.shape)}")
    s1, u1, n1, O1, l1 = ix.ice_decode(Q, budget, beam)
    r2 = ix.ice_decode(Q, budget, beam)
    s2, u2, n2 = ix.ice_select(Q, budget, beam)
    O2, l2 = ix.ice_attend(Q, u2, n2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(u1, u2) and torch.equal(n1, n2)
    for x, y in zip((s1, u1, n1, O1, l1), r2):
        assert torch.equal(x, y), "two decode calls differ"
    den = O2.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    assert float(((O1 - O2).abs() / den).max()) <= 1e-5
    fin = torch.isfinite(l2)
    assert torch.equal(fin, torch.isfinite(l1))
    if fin.any():
        assert float((l1[fin] - l2[fin]).abs().max()) <= 1e-5 * max(1.0, float(l2[fin].abs().max()))
    out = run_decode(ix, Q, budget, beam)
    out["O"], out["lse"] = O1.cpu().double().numpy(), l1.cpu().double().numpy()
    compare_decode(ix, refs, out)
    return out


def replay_inserts(ref, g, k, v, h, seed, levels, plog2, resplit=False):
    """Applies inserted tokens (rows of k, v) to the oracle index `ref`,
    accepting the GPU's parent choice (from the GPU head `g`) only inside the
    near-tie band of the oracle's nearest point at that moment."""
    for j in range(k.shape[0]):
        t = ref.n
        lam = min(ref.L_top, int(ic.draw_levels(seed, h, t, 1, levels, plog2)[0]))
        override = None
        if lam < ref.L_top:
            cand = np.nonzero(ref.lev >= lam + 1)[0]
            x = np.concatenate([to64(k[j]), [ic.lift_one(to64(k[j]), ref.M2)[0]]])
            jj, D1, D2 = ic.nearest(x[None, :], ic.lifted(ref.K[cand], ref.e[cand]))
            gp = int(g.parent[lam][t])
            if gp != int(cand[jj[0]]):
                dg = float(((ic.lifted(ref.K[gp:gp + 1], ref.e[gp:gp + 1])[0] - x) ** 2).sum())
                assert abs(dg - D1[0]) <= BAND * max(dg, D1[0]), f"insert parent of {t} outside the band"
                override = gp
        ic.insert(ref, to64(k[j]), to64(v[j]), parent_override=override, resplit=resplit)


