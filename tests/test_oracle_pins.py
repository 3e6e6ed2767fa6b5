"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each check is tied to something other than the oracle's own formulas: the
generator's published outputs, closed-form identities, hand-worked cases from
``tests/golden/`` (every file states the passage of the pages it follows and
how the expected values were worked out), brute force on tiny inputs, or an
independent library routine. The last section plants mistakes in the oracle
and shows that one of the pins catches each of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import icecache as ic

from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed=0):
    return np.random.default_rng(seed)


def _clustered(n, d, c, seed):
    r = _rng(seed)
    cent = r.standard_normal((c, d))
    m = r.integers(0, c, n)
    K = cent[m] + 0.3 * r.standard_normal((n, d))
    V = r.standard_normal((n, d))
    return K, V, cent


# --------------------------------------------------------------------------
# promotion draws
# --------------------------------------------------------------------------

def check_splitmix_reference():
    g = _golden("splitmix64_reference.json")
    out = ic.splitmix64_outputs(g["seed"], len(g["outputs"]))
    return [int(x) for x in out] == [int(s) for s in g["outputs"]]


def test_splitmix64_published_outputs():
    assert check_splitmix_reference()


def test_ctz64_closed_form():
    xs = [0, 1, 2, 3, 12, 1 << 40, 1 << 63, (1 << 64) - 1, 0x8000000000000001, 96]
    want = [64, 0, 1, 0, 2, 40, 63, 0, 0, 5]
    assert list(ic.ctz64(np.array(xs, dtype=np.uint64))) == want


def check_level_distribution():
    n = 1 << 16
    lev = ic.draw_levels(7, 3, 0, n, levels=3, promote_log2=4)
    ok = True
    for l, p in ((1, 1 / 16), (2, 1 / 256)):
        cnt = int((lev >= l).sum())
        mu, sd = n * p, math.sqrt(n * p * (1 - p))
        ok &= abs(cnt - mu) <= 5 * sd
    return ok and lev.max() <= 2 and lev.min() >= 0


def test_level_counts_binomial():
    # [A §三] promotion is random with a smaller subset each level; p = 1/16 per level.
    assert check_level_distribution()


def test_levels_deterministic_and_counter_based():
    a = ic.draw_levels(0, 5, 0, 1000, 3, 4)
    b = ic.draw_levels(0, 5, 0, 1000, 3, 4)
    assert np.array_equal(a, b)
    # token t draws the same level whether drawn in a batch or alone (inserts)
    tail = ic.draw_levels(0, 5, 700, 300, 3, 4)
    assert np.array_equal(a[700:], tail)
    # heads use different streams
    assert not np.array_equal(a, ic.draw_levels(0, 6, 0, 1000, 3, 4))


# --------------------------------------------------------------------------
# lift
# --------------------------------------------------------------------------

def test_lift_puts_every_build_key_on_the_sphere():
    K, _, _ = _clustered(500, 16, 8, 1)
    n2, M2, e = ic.lift(K)
    X = ic.lifted(K, e)
    assert np.allclose((X * X).sum(1), M2, rtol=1e-12, atol=0)
    assert e[np.argmax(n2)] == 0.0          # M^2 kept as the norm itself


def test_lifted_query_distance_identity():
    # [A §六] with TQ(q) = [q, 0]: |TQ(q) - TK(k)|^2 = |q|^2 + M^2 - 2 q.k
    r = _rng(2)
    K = r.standard_normal((200, 8))
    q = r.standard_normal(8)
    n2, M2, e = ic.lift(K)
    X = ic.lifted(K, e)
    direct = ((np.concatenate([q, [0.0]])[None, :] - X) ** 2).sum(1)
    closed = q @ q + M2 - 2 * K @ q
    assert np.allclose(direct, closed, rtol=1e-12, atol=1e-12)
    # so the nearest lifted key is the maximum inner product key
    assert int(np.argmin(direct)) == int(np.argmax(K @ q))


# --------------------------------------------------------------------------
# parents
# --------------------------------------------------------------------------

def check_parent_golden():
    ok = True
    for case in _golden("lift_parent_cases.json")["cases"]:
        K = np.array(case["keys"], dtype=np.float64)
        lev = np.array(case["levels"])
        idx = ic.build_head(K, np.zeros_like(K), 0, 0, lev=lev)
        ok &= list(idx.parent[0]) == case["parent0"]
        if "M2" in case:
            ok &= abs(idx.M2 - case["M2"]) < 1e-15
            ok &= np.allclose(idx.e, case["e"], rtol=1e-14, atol=1e-15)
        if "dist0" in case:
            ok &= np.allclose(idx.dist[0], case["dist0"], rtol=1e-12, atol=1e-15)
        if "near_tie" in case:
            flags = ic.is_near_tie(idx.dist[0], idx.second[0])
            ok &= list(map(bool, flags)) == case["near_tie"]
    return bool(ok)


def test_parent_hand_cases():
    assert check_parent_golden()


def test_parent_brute_force_tiny():
    # brute force on tiny inputs: itertools double loop over every pair
    for seed in range(4):
        r = _rng(10 + seed)
        n, d = 48, 3
        K = r.standard_normal((n, d)) * r.uniform(0.5, 2.0, (n, 1))
        lev = r.integers(0, 3, n)
        lev[r.integers(0, n)] = 2
        idx = ic.build_head(K, K, 0, 0, lev=lev)
        X = idx.X()
        for l in range(idx.L_top):
            for i in range(n):
                if lev[i] < l:
                    continue
                if lev[i] >= l + 1:
                    assert idx.parent[l][i] == i
                    continue
                best, bj = None, None
                for j in itertools.chain(range(n)):
                    if lev[j] < l + 1:
                        continue
                    dd = sum((X[i, c] - X[j, c]) ** 2 for c in range(d + 1))
                    if best is None or dd < best:
                        best, bj = dd, j
                assert idx.parent[l][i] == bj
                assert abs(idx.dist[l][i] - best) <= 1e-12 * max(1.0, best)


# --------------------------------------------------------------------------
# pack
# --------------------------------------------------------------------------

def _pack_case_index():
    c = _golden("pack_insert_select_cases.json")["pack"]
    K = np.array(c["keys"], dtype=np.float64)
    V = np.arange(K.size, dtype=np.float64).reshape(K.shape)
    return ic.build_head(K, V, 0, 0, lev=np.array(c["levels"]), page_cap=c["page_cap"]), c


def check_pack_golden():
    idx, c = _pack_case_index()
    return (idx.pages == c["pages"] and idx.page_owner == c["page_owner"]
            and {str(k): v for k, v in idx.owner_pages.items()} == c["owner_pages"] and idx.top == c["top"])


def test_pack_hand_case():
    assert check_pack_golden()


def check_layout_invariants(idx, ordered=True):
    n, cap = idx.n, idx.page_cap
    seen = np.zeros(n, dtype=np.int64)
    for pg, toks in enumerate(idx.pages):
        if not (1 <= len(toks) <= cap):
            return False
        own = idx.page_owner[pg]
        for t in toks:
            seen[t] += 1
            expect = ic.ROOT if idx.L_top == 0 else (t if idx.lev[t] >= 1 else idx.parent[0][t])
            if expect != own:
                return False
    if not np.all(seen == 1):
        return False
    n1 = int((idx.lev >= 1).sum())
    counts = {}
    for pg, own in enumerate(idx.page_owner):
        counts.setdefault(own, 0)
        counts[own] += len(idx.pages[pg])
    for own, pgs in idx.owner_pages.items():
        if len(pgs) != math.ceil(counts.get(own, 0) / cap):
            return False
        # every page but the owner's last is full
        if any(len(idx.pages[p]) != cap for p in pgs[:-1]):
            return False
        if ordered and idx.L_top >= 1:
            dmax = -np.inf
            for p in pgs:
                ds = [idx.dist[0][t] for t in idx.pages[p]]
                if min(ds) < dmax:
                    return False
                dmax = max(ds)
    if len(idx.pages) > n / cap + max(1, n1):
        return False
    return True


@pytest.mark.parametrize("n,d,c,seed", [(2048, 16, 32, 0), (777, 8, 5, 1), (300, 4, 300, 2)])
def test_pack_invariants(n, d, c, seed):
    K, V, _ = _clustered(n, d, c, seed)
    idx = ic.build_head(K, V, 0, seed)
    assert check_layout_invariants(idx)
    # page ids follow the owners in ascending token order
    owners = [o for o in idx.page_owner]
    assert owners == sorted(owners)
    # every upper-level child list holds exactly its owner's children
    for l, lists in idx.children.items():
        allk = sorted(t for v in lists.values() for t in v)
        assert allk == sorted(np.nonzero(idx.lev >= l)[0].tolist())


def test_no_promoted_point_gives_token_order_pages():
    K, V, _ = _clustered(40, 4, 3, 3)
    idx = ic.build_head(K, V, 0, 0, lev=np.zeros(40, dtype=np.int64))
    assert idx.L_top == 0
    assert idx.pages == [list(range(0, 16)), list(range(16, 32)), list(range(32, 40))]
    assert idx.page_owner == [ic.ROOT] * 3


def test_empty_and_single_token_builds():
    idx = ic.build_head(np.zeros((0, 4)), np.zeros((0, 4)), 0, 0)
    assert idx.pages == [] and idx.L_top == 0 and idx.M2 == 0.0
    r = ic.select(idx, np.ones(4), 64, 4)
    assert r["sel"] == []
    o, lse = ic.attend(idx, np.ones(4), [], 0.5)
    assert np.all(o == 0) and lse == -np.inf
    one = ic.build_head(np.ones((1, 4)), np.ones((1, 4)), 0, 0)
    assert one.pages == [[0]] and one.e[0] == 0.0


# --------------------------------------------------------------------------
# insert
# --------------------------------------------------------------------------

def check_insert_golden():
    idx, _ = _pack_case_index()
    c = _golden("pack_insert_select_cases.json")["insert"]
    for tok in c["tokens"]:
        assert idx.n == tok["t"]
        ic.insert(idx, np.array(tok["key"]), np.zeros(2), lev_override=tok["level"])
    return (idx.pages == c["pages"] and idx.page_owner == c["page_owner"]
            and {str(k): v for k, v in idx.owner_pages.items()} == c["owner_pages"]
            and idx.top == c["top"] and idx.splits == c["splits"])


def test_insert_hand_case():
    assert check_insert_golden()


def test_insert_invariants_and_parents_at_insert_time():
    K, V, cent = _clustered(1500, 8, 16, 4)
    idx = ic.build_head(K, V, 2, 4)
    before = [list(p) for p in idx.pages]
    r = _rng(5)
    for step in range(400):
        m = r.integers(0, len(cent))
        k = cent[m] + 0.3 * r.standard_normal(8)
        cand = np.nonzero(idx.lev >= 1)[0]
        Xc = idx.X()[cand]
        lam, p = ic.insert(idx, k, r.standard_normal(8))
        t = idx.n - 1
        if lam < idx.L_top:
            # brute force over the points of level lam+1 present at insertion time
            cand = np.nonzero(idx.lev[:t] >= lam + 1)[0]
            x = idx.X()[t]
            dd = ((idx.X()[cand] - x) ** 2).sum(1)
            assert p == cand[np.nonzero(dd == dd.min())[0][0]]
    assert check_layout_invariants(idx, ordered=False)
    # resident tokens never move: old pages are prefixes of the new ones
    for a, b in zip(before, idx.pages):
        assert b[:len(a)] == a
    assert idx.splits > 0


def test_insert_into_empty_index_and_clamp():
    idx = ic.build_head(np.zeros((0, 3)), np.zeros((0, 3)), 0, 0)
    for i in range(20):
        ic.insert(idx, np.ones(3) * (i + 1), np.zeros(3))
    assert idx.pages == [list(range(16)), list(range(16, 20))]
    assert idx.clamps == 20                     # M^2 = 0: every new key is clamped
    K = np.eye(3)
    idx = ic.build_head(K, K, 0, 0, lev=np.array([1, 1, 0]))
    ic.insert(idx, np.array([2.0, 0.0, 0.0]), np.zeros(3), lev_override=0)
    assert idx.clamps == 1 and idx.e[-1] == 0.0
    ic.insert(idx, np.array([0.5, 0.0, 0.0]), np.zeros(3), lev_override=0)
    assert idx.clamps == 1 and abs(idx.e[-1] - math.sqrt(0.75)) < 1e-15


# --------------------------------------------------------------------------
# replay entry points: a given parent instead of the search's own choice
# --------------------------------------------------------------------------
# The GPU parity tests hand the oracle the GPU's parent wherever the two best
# parents are near-tied (build_head(parents=...), insert(parent_override=...)).
# These pins fix what those two paths compute: a hand-worked case where the
# given parent is the runner-up, and the identity with the free search when
# the given parents are the search's own.

def _replay_case():
    c = _golden("replay_case.json")
    K = np.array(c["keys"], dtype=np.float64)
    return c, K


def _num(x):
    return np.inf if x == "inf" else float(x)


def check_replay_golden():
    c, K = _replay_case()
    lev = np.array(c["levels"])
    cap = c["page_cap"]
    ok = True
    free = ic.build_head(K, K, 0, 0, lev=lev, page_cap=cap)
    f = c["free"]
    ok &= free.parent[0].tolist() == f["parent0"]
    ok &= np.allclose(free.dist[0], f["dist0"], rtol=0, atol=1e-9)
    ok &= np.allclose(free.second[0], [_num(x) for x in f["second0"]], rtol=0, atol=1e-9)
    ok &= free.pages == f["pages"] and {str(k): v for k, v in free.owner_pages.items()} == f["owner_pages"]
    fb = c["forced_build"]
    forced = ic.build_head(K, K, 0, 0, lev=lev, page_cap=cap, parents=[np.array(fb["parents0"])])
    ok &= forced.parent[0].tolist() == fb["parent0"]
    ok &= np.allclose(forced.dist[0], fb["dist0"], rtol=0, atol=1e-9)
    ok &= forced.pages == fb["pages"] and {str(k): v for k, v in forced.owner_pages.items()} == fb["owner_pages"]
    ins = c["insert"]
    for mode, override in (("free", None), ("forced", ins["forced"]["parent"])):
        idx = ic.build_head(K, K, 0, 0, lev=lev, page_cap=cap)
        lam, p = ic.insert(idx, np.array(ins["key"], np.float64), np.zeros(2), lev_override=ins["level"],
                           parent_override=override)
        w = ins[mode]
        ok &= lam == ins["level"] and p == w["parent"] and abs(idx.dist[0][5] - w["dist"]) <= 1e-9
        ok &= idx.pages == w["pages"] and {str(k): v for k, v in idx.owner_pages.items()} == w["owner_pages"]
        ok &= idx.splits == w["splits"]
    return bool(ok)


def test_replay_hand_case_runner_up():
    assert check_replay_golden()


def test_replay_build_with_own_parents_is_the_free_build():
    for n, d, c, seed, levels in [(1500, 8, 16, 21, 3), (700, 4, 40, 22, 4), (300, 16, 5, 23, 2)]:
        K, V, _ = _clustered(n, d, c, seed)
        free = ic.build_head(K, V, 3, seed, levels)
        given = [free.parent[l].copy() for l in range(free.L_top)]
        rep = ic.build_head(K, V, 3, seed, levels, parents=given)
        assert rep.pages == free.pages and rep.page_owner == free.page_owner
        assert rep.owner_pages == free.owner_pages and rep.children == free.children and rep.top == free.top
        for l in range(free.L_top):
            assert np.array_equal(rep.parent[l], free.parent[l])
            # the replay recomputes D as a direct sum of squares, as the free search does
            m = free.parent[l] >= 0
            assert np.array_equal(rep.dist[l][m], free.dist[l][m])


def test_replay_insert_with_own_choice_is_the_free_insert():
    K, V, cent = _clustered(1500, 8, 16, 24)
    a = ic.build_head(K, V, 2, 24)
    b = ic.build_head(K, V, 2, 24)
    r = _rng(25)
    for step in range(400):
        k = cent[r.integers(0, len(cent))] + 0.3 * r.standard_normal(8)
        v = r.standard_normal(8)
        lam, p = ic.insert(a, k, v)
        lam_b, p_b = ic.insert(b, k, v, parent_override=p)
        assert (lam, p) == (lam_b, p_b)
    assert a.pages == b.pages and a.owner_pages == b.owner_pages and a.top == b.top
    assert a.children == b.children and a.splits == b.splits and a.splits > 0
    for l in range(a.L_top):
        assert np.array_equal(a.parent[l], b.parent[l])
        m = a.parent[l] >= 0
        assert np.array_equal(a.dist[l][m], b.dist[l][m])


def test_planted_replay_ignoring_the_given_parent_is_caught(monkeypatch):
    # a replay that silently keeps the search's own parent fails the hand case
    real = ic.build_head

    def ignoring(K, V, head, seed, levels=3, promote_log2=4, page_cap=16, lev=None, parents=None, pdci=None):
        return real(K, V, head, seed, levels, promote_log2, page_cap, lev=lev, parents=None, pdci=pdci)
    monkeypatch.setattr(ic, "build_head", ignoring)
    assert not check_replay_golden()


def test_planted_insert_ignoring_the_override_is_caught(monkeypatch):
    real = ic.insert

    def ignoring(idx, k, v, lev_override=None, parent_override=None, resplit=False):
        return real(idx, k, v, lev_override=lev_override, parent_override=None, resplit=resplit)
    monkeypatch.setattr(ic, "insert", ignoring)
    assert not check_replay_golden()


# --------------------------------------------------------------------------
# insert with the re-sort split
# --------------------------------------------------------------------------

def check_resplit_golden():
    """Runs the hand-worked re-sort case in both split modes; True when every
    checkpoint's pages are the hand-worked ones."""
    c = _golden("resplit_case.json")
    ok = True
    for mode in ("resplit", "append"):
        K = np.array(c["keys"])
        nb = len(c["build_levels"])
        idx = ic.build_head(K[:nb], np.zeros((nb, 2)), 0, 0, lev=np.array(c["build_levels"]))
        for t in c["inserts"]:
            ic.insert(idx, K[t], np.zeros(2), lev_override=0, resplit=mode == "resplit")
            want = c["after"].get(str(t))
            if want is not None:
                ok &= idx.pages == want[mode]
        ok &= idx.splits == c["splits"] and idx.owner_pages[0] == [0, 1, 2]
    return bool(ok)


def test_resplit_hand_case():
    assert check_resplit_golden()


def _chain_sequences(idx):
    return {o: [t for p in ps for t in idx.pages[p]] for o, ps in idx.owner_pages.items()}


@pytest.mark.parametrize("seed", [6, 7])
def test_resplit_is_a_sorted_prefix_of_the_append_order(seed):
    """Closed form against the append split on the same inputs: same page
    ids, owners, chains and counts; per owner, the members present at its
    last split (the first 16*(pages-1)+1 of the append order) appear sorted
    by (distance to the owner, token id), then the later arrivals in arrival
    order. An owner whose pages never split since the build has a sorted
    prefix already (the build packs that way), so the form holds for it too."""
    K, V, cent = _clustered(1200, 8, 12, seed)
    a = ic.build_head(K, V, 1, seed)
    b = ic.build_head(K, V, 1, seed)
    r = _rng(seed + 100)
    for _ in range(900):
        m = r.integers(0, len(cent))
        k = cent[m] + 0.3 * r.standard_normal(8)
        v = r.standard_normal(8)
        ra = ic.insert(a, k, v)
        rb = ic.insert(b, k, v, resplit=True)
        assert ra == rb
    assert a.splits == b.splits > 20
    assert a.page_owner == b.page_owner and a.owner_pages == b.owner_pages
    assert [len(p) for p in a.pages] == [len(p) for p in b.pages]
    sa, sb = _chain_sequences(a), _chain_sequences(b)
    n_sorted = 0
    for o, seq in sa.items():
        s = 16 * (len(a.owner_pages[o]) - 1) + 1
        head = sorted(seq[:s], key=lambda t: (float(np.sum((b.X()[t] - b.X()[o]) ** 2)), t))
        assert sb[o] == head + seq[s:], f"owner {o}"
        n_sorted += head != seq[:s]
    assert n_sorted > 5


def test_resplit_limits_keep_the_append_split(monkeypatch):
    """The virtual root never re-sorts (its pages are token-order runs), and
    an owner over RESPLIT_MAX members splits by appending."""
    r = _rng(8)
    K = r.standard_normal((40, 4))
    a = ic.build_head(K, K, 0, 0, lev=np.zeros(40, dtype=np.int64))
    for i in range(30):
        ic.insert(a, r.standard_normal(4), np.zeros(4), lev_override=0, resplit=True)
    assert a.pages == [list(range(s, min(s + 16, 70))) for s in range(0, 70, 16)]
    c = _golden("resplit_case.json")
    Kc = np.array(c["keys"])
    monkeypatch.setattr(ic, "RESPLIT_MAX", 16)
    idx = ic.build_head(Kc[:16], np.zeros((16, 2)), 0, 0, lev=np.array(c["build_levels"]))
    ic.insert(idx, Kc[16], np.zeros(2), lev_override=0, resplit=True)
    assert idx.pages == c["after"]["16"]["append"]
    monkeypatch.setattr(ic, "RESPLIT_MAX", 17)
    idx = ic.build_head(Kc[:16], np.zeros((16, 2)), 0, 0, lev=np.array(c["build_levels"]))
    ic.insert(idx, Kc[16], np.zeros(2), lev_override=0, resplit=True)
    assert idx.pages == c["after"]["16"]["resplit"]


# --------------------------------------------------------------------------
# P-DCI parents
# --------------------------------------------------------------------------

from oracle import pdci as pd  # noqa: E402


def _dirs(r, rows, d):
    u = r.standard_normal((rows, d))
    return (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32).astype(np.float64)


def test_pdci_hand_case_projection_misleads():
    """Keys A=(0.1, 2), B=(0.5, 0) at level 1, C=(0, 0) at level 0; M^2 =
    |A|^2 = 4.01, so e_A = 0, e_B = sqrt(3.76), e_C = sqrt(4.01). Lifted
    D(C,A) = 0.01 + 4 + 4.01 = 8.02 and D(C,B) = 0.25 + (2.00250 - 1.93907)^2
    = 0.2540, so B is the exact parent. One simple index projecting on the
    first key coordinate puts A (|0.1 - 0| = 0.1) before B (0.5): with one
    visit P-DCI returns A, with two it ranks both and returns B."""
    K = np.array([[0.1, 2.0], [0.5, 0.0], [0.0, 0.0]])
    lev = np.array([1, 1, 0])
    dirs = np.array([[1.0, 0.0, 0.0]])
    ex = ic.build_head(K, K, 0, 0, levels=2, lev=lev)
    assert ex.parent[0][2] == 1 and abs(ex.dist[0][2] - 0.2540) < 1e-4
    one = ic.build_head(K, K, 0, 0, levels=2, lev=lev, pdci=pd.Pdci(dirs, 1, 1, 1, 1))
    assert one.parent[0][2] == 0 and abs(one.dist[0][2] - 8.02) < 1e-9
    two = ic.build_head(K, K, 0, 0, levels=2, lev=lev, pdci=pd.Pdci(dirs, 1, 1, 2, 2))
    assert two.parent[0][2] == 1 and np.isfinite(two.second[0][2])


def test_pdci_with_unbounded_budgets_is_the_exact_search():
    K, V, _ = _clustered(700, 6, 8, 12)
    r = _rng(13)
    n = 700
    cfg = pd.Pdci(_dirs(r, 4, 7), m=2, l=2, visits=2 * n, cands=n)
    a = ic.build_head(K, V, 0, 12, pdci=cfg)
    b = ic.build_head(K, V, 0, 12)
    for l in range(b.L_top):
        assert np.array_equal(a.parent[l], b.parent[l])
    assert a.pages == b.pages


def _visit_rank_candidates(qkey, keys, cfg):
    """Closed form of one query's candidates: every (point, simple index) pair
    is visited in ascending (|key - query key|, simple index, point) order, so
    a point completes at the largest visit rank of its l pairs; a composite
    index keeps the points completing within its visit budget (at least the
    first), in completion order, at most cands."""
    n = keys.shape[0]
    out = []
    for j in range(cfg.m):
        cols = range(j * cfg.l, (j + 1) * cfg.l)
        pairs = sorted((abs(keys[c, col] - qkey[col]), i, c) for i, col in enumerate(cols) for c in range(n))
        rank = {}
        for r_, (_, i, c) in enumerate(pairs):
            rank[(c, i)] = r_
        done = sorted((max(rank[(c, i)] for i in range(cfg.l)), c) for c in range(n))
        keep = [c for rk, c in done if rk < cfg.visits] or [done[0][1]]
        out.extend(keep[:cfg.cands])
    return out


@pytest.mark.parametrize("m,l,visits,cands", [(1, 1, 5, 3), (1, 2, 40, 6), (2, 2, 25, 4), (3, 3, 90, 8),
                                              (1, 3, 3, 5)])
def test_pdci_candidates_follow_the_visit_order(m, l, visits, cands):
    r = _rng(20 + m + l)
    keys = r.standard_normal((60, m * l))
    for _ in range(20):
        q = r.standard_normal(m * l)
        cfg = pd.Pdci(np.zeros((m * l, 1)), m, l, visits, cands)
        assert pd.candidates(q, keys, cfg) == _visit_rank_candidates(q, keys, cfg)


# --------------------------------------------------------------------------
# select and union
# --------------------------------------------------------------------------

def check_select_golden():
    g = _golden("pack_insert_select_cases.json")
    idx, _ = _pack_case_index()
    ok = True
    for qc in g["select"][0]["queries"]:
        r = ic.select(idx, np.array(qc["q"]), qc["budget"], qc["beam"])
        ok &= r["sel"] == qc["sel"]
    c = g["select"][1]
    K = np.array(c["keys"])
    idx3 = ic.build_head(K, np.zeros_like(K), 0, 0, lev=np.array(c["levels"]))
    ok &= idx3.pages == c["pages"]
    ok &= {str(k): v for k, v in idx3.children[1].items()} == c["children1"]
    for qc in c["queries"]:
        r = ic.select(idx3, np.array(qc["q"]), qc["budget"], qc["beam"])
        ok &= r["sel"] == qc["sel"] and r["kept"] == qc["kept"]
    return bool(ok)


def test_select_hand_cases():
    assert check_select_golden()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_full_beam_is_brute_force_page_ranking(seed):
    # beam >= every point: the descent keeps everything and the result is a
    # plain sort of all pages by their best token score
    K, V, cent = _clustered(1200, 8, 12, seed)
    idx = ic.build_head(K, V, 1, seed)
    r = _rng(100 + seed)
    for _ in range(5):
        q = cent[r.integers(0, len(cent))] + 0.3 * r.standard_normal(8)
        for budget in (16, 64, 128):
            got = ic.select(idx, q, budget, beam=idx.n)["sel"]
            scores = [max(float(K[t] @ q) for t in toks) for toks in idx.pages]
            want = sorted(range(len(scores)), key=lambda p: (-scores[p], p))[:budget // 16]
            assert got == want
            best_tok = int(np.argmax(K @ q))
            assert any(best_tok in idx.pages[p] for p in got)


def test_select_forced_cut_admissibility():
    ids, sc = [3, 1, 2], [1.0, 0.5, 0.49999999]
    kept, tie, ok = ic._cut(ids, sc, 1, 1.0, 1.0)
    assert kept == [3] and not tie and ok
    kept, tie, ok = ic._cut([1, 2], [0.5, 0.5 - 1e-9], 1, 1.0, 1.0, forced=[2])
    assert ok and tie                       # a near-tie may go either way
    kept, tie, ok = ic._cut([1, 2], [0.9, 0.1], 1, 1.0, 1.0, forced=[2])
    assert not ok                           # a clear inversion may not


def test_gqa_union_is_sorted_set_union():
    assert ic.gqa_union([[5, 2, -1], [2, 9], [], [7, 5]]) == [2, 5, 7, 9]


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def check_attention_golden():
    ok = True
    for c in _golden("attention_cases.json")["cases"]:
        K = np.array(c["keys"])
        idx = ic.build_head(K, np.array(c["values"]), 0, 0, lev=np.zeros(len(K), dtype=np.int64))
        o, lse = ic.attend(idx, np.array(c["q"]), list(range(len(idx.pages))), c["scale"])
        ok &= np.allclose(o, c["o"], rtol=0, atol=1e-14) and abs(lse - c["lse"]) < 1e-14
    return bool(ok)


def test_attention_hand_cases():
    assert check_attention_golden()


def test_attention_all_pages_equals_dense_sdpa():
    K, V, cent = _clustered(700, 16, 10, 6)
    idx = ic.build_head(K, V, 0, 6)
    r = _rng(7)
    q = cent[3] + 0.3 * r.standard_normal(16)
    o, lse = ic.attend(idx, q, list(range(len(idx.pages))), 1 / math.sqrt(16))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None, :], torch.tensor(K)[None, None], torch.tensor(V)[None, None])
    assert np.allclose(o, ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)
    assert abs(lse - float(torch.logsumexp(torch.tensor(K @ q / 4.0), 0))) < 1e-12


def test_attention_split_combine_identity():
    K, V, cent = _clustered(900, 8, 10, 8)
    idx = ic.build_head(K, V, 0, 8)
    q = cent[0]
    pages = list(range(len(idx.pages)))
    o, lse = ic.attend(idx, q, pages, 0.3)
    a, la = ic.attend(idx, q, pages[::2], 0.3)
    b, lb = ic.attend(idx, q, pages[1::2], 0.3)
    m = max(la, lb)
    wa, wb = math.exp(la - m), math.exp(lb - m)
    assert np.allclose(o, (wa * a + wb * b) / (wa + wb), rtol=1e-12, atol=1e-12)
    assert abs(lse - (m + math.log(wa + wb))) < 1e-12
    # page order does not matter
    o2, _ = ic.attend(idx, q, pages[::-1], 0.3)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-14)


def test_attention_resident_only_equals_sdpa():
    """Resident tokens with no selected page: plain softmax attention over them."""
    r = _rng(11)
    K, V, _ = _clustered(300, 16, 6, 12)
    idx = ic.build_head(K, V, 0, 12)
    Kr, Vr = r.standard_normal((37, 16)), r.standard_normal((37, 16))
    q = r.standard_normal(16)
    o, lse = ic.attend(idx, q, [], 0.25, resident=(Kr, Vr))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None, :], torch.tensor(Kr)[None, None], torch.tensor(Vr)[None, None], scale=0.25)
    assert np.allclose(o, ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)
    assert abs(lse - float(torch.logsumexp(torch.tensor(Kr @ q * 0.25), 0))) < 1e-12


def test_attention_with_resident_combines_two_softmaxes():
    """Pages plus resident tokens = the lse-weighted merge of the two parts."""
    r = _rng(12)
    K, V, cent = _clustered(800, 8, 10, 13)
    idx = ic.build_head(K, V, 0, 13)
    Kr, Vr = r.standard_normal((20, 8)), r.standard_normal((20, 8))
    q = cent[2]
    pages = list(range(0, len(idx.pages), 3))
    o, lse = ic.attend(idx, q, pages, 0.4, resident=(Kr, Vr))
    a, la = ic.attend(idx, q, pages, 0.4)
    b, lb = ic.attend(idx, q, [], 0.4, resident=(Kr, Vr))
    m = max(la, lb)
    wa, wb = math.exp(la - m), math.exp(lb - m)
    assert np.allclose(o, (wa * a + wb * b) / (wa + wb), rtol=1e-12, atol=1e-12)
    assert abs(lse - (m + math.log(wa + wb))) < 1e-12


def test_attention_dense_head_ignores_the_selection():
    """A dense head attends every indexed token, whatever pages are passed."""
    K, V, cent = _clustered(500, 16, 8, 14)
    idx = ic.build_head(K, V, 0, 14)
    q = cent[1]
    o, lse = ic.attend(idx, q, [0], 0.25, dense=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None, :], torch.tensor(K)[None, None], torch.tensor(V)[None, None], scale=0.25)
    assert np.allclose(o, ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)
    assert abs(lse - float(torch.logsumexp(torch.tensor(K @ q * 0.25), 0))) < 1e-12


def test_reuse_keeps_the_structure_and_lifts_its_own_keys():
    K, V, cent = _clustered(900, 16, 10, 15)
    src = ic.build_head(K, V, 0, 15)
    r = _rng(16)
    K2, V2 = K + 0.1 * r.standard_normal(K.shape), r.standard_normal(V.shape)
    idx = ic.build_head_reuse(K2, V2, src, 1)
    assert idx.pages == src.pages and idx.top == src.top and np.array_equal(idx.lev, src.lev)
    assert all(np.array_equal(a, b) for a, b in zip(idx.parent, src.parent))
    # its own lift: the largest key has e = 0 and every lifted norm is M
    assert idx.M2 == float((K2 * K2).sum(1).max())
    assert np.allclose((idx.X() ** 2).sum(1), idx.M2, rtol=1e-12)
    # attention reads its own rows
    q = cent[4]
    o, _ = ic.attend(idx, q, [0, 1], 0.25)
    toks = idx.pages[0] + idx.pages[1]
    w = np.exp(K2[toks] @ q * 0.25 - (K2[toks] @ q * 0.25).max())
    assert np.allclose(o, (w @ V2[toks]) / w.sum(), rtol=1e-12, atol=1e-12)
    # with the same keys the reused index selects exactly as its source
    same = ic.build_head_reuse(K, V, src, 1)
    for g in range(4):
        qq = cent[g] + 0.2 * r.standard_normal(16)
        assert ic.select(same, qq, 64, 4)["sel"] == ic.select(src, qq, 64, 4)["sel"]


# --------------------------------------------------------------------------
# planted mistakes: each must break at least one pin above
# --------------------------------------------------------------------------

def test_planted_lift_without_extra_coordinate_is_caught(monkeypatch):
    def bad_lift(K):
        n2, M2, e = _orig_lift(K)
        return n2, M2, np.zeros_like(e)
    monkeypatch.setattr(ic, "lift", bad_lift)
    assert not check_parent_golden()


def test_planted_wrong_promotion_shift_is_caught(monkeypatch):
    orig = ic.splitmix64_mix

    def bad_mix(z):
        z = np.atleast_1d(np.asarray(z, dtype=np.uint64))
        z = (z ^ (z >> np.uint64(31))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))
    monkeypatch.setattr(ic, "splitmix64_mix", bad_mix)
    assert not check_splitmix_reference()
    monkeypatch.setattr(ic, "splitmix64_mix", orig)
    assert check_splitmix_reference()


def test_planted_pack_in_token_order_is_caught(monkeypatch):
    orig_pack = ic.pack

    def bad_pack(lev, L_top, parent, dist, page_cap):
        flat = [np.zeros_like(d0) for d0 in dist]
        return orig_pack(lev, L_top, parent, flat, page_cap)
    monkeypatch.setattr(ic, "pack", bad_pack)
    assert not check_pack_golden()


def test_planted_page_score_mean_is_caught(monkeypatch):
    orig_max = np.max

    class FakeNp:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def max(x, *a, **k):
            return np.mean(x)
    monkeypatch.setattr(ic, "np", FakeNp())
    try:
        assert not check_select_golden()
    finally:
        monkeypatch.setattr(ic, "np", np)
    assert orig_max is np.max


def test_planted_attention_scale_dropped_is_caught(monkeypatch):
    orig = ic.attend

    def bad_attend(idx, q, pages, scale):
        return orig(idx, q, pages, 1.0)
    monkeypatch.setattr(ic, "attend", bad_attend)
    assert not check_attention_golden()


def test_planted_resplit_sorted_descending_is_caught(monkeypatch):
    class FakeNp:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def lexsort(keys, *a, **k):
            return np.lexsort(keys, *a, **k)[::-1]
    monkeypatch.setattr(ic, "np", FakeNp())
    try:
        assert not check_resplit_golden()
    finally:
        monkeypatch.setattr(ic, "np", np)
    assert check_resplit_golden()


_orig_lift = ic.lift
