"""IceCache hot path written out plainly, in fp64 NumPy.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library. It shares
no code, table or constant generator with the HIP path; the promotion hash is
implemented here from the published SplitMix64 definition and independently
in HIP.

Sources, cited by page and section:

* [A] "IceCache" article on aitangshan.cn (arXiv 2604.10539, ICLR 2026):
  section 二 (pages of 16 tokens, semantic instead of sequential pages),
  section 三 (DCI tree: lift, random promotion, nearest parent, same parent =
  same page, incremental insert), section 四 (bulk loading), section 六
  (TK/TQ transform, GQA union; sink and window tokens stay resident on the
  GPU, only the tokens in between are indexed).
* [N] papernotes.org notes "IceCache: Memory-Efficient KV-cache Management for
  Long-Sequence LLMs": "Overall framework" (index / page selection / bulk
  load), key design 1 (semantic pages, the sparse-attention weight formula),
  key design 2 (M-DCI: promotion, parents, top-down search, incremental insert,
  page split), key design 3 (per-head selection, GQA union); the
  limitations section (the first two layers are left out of retrieval, their
  attention being dense).

Where the pages leave a step open, the reading taken is marked ``[reading]``;
each one is listed in the design notes. Every function here is pinned by
``tests/test_oracle_pins.py`` against hand-worked cases (``tests/golden/``),
closed forms, library routines or brute force. Nothing here is "parity
unpinned".

Conventions: a head's tokens are numbered 0..n-1 in arrival order. Level 0
holds every token. ``lev[t]`` is the highest level token t belongs to. A page
is an ordered list of at most ``page_cap`` token ids; page ids are dense
0,1,2,... per head. ``ROOT`` (-1) is the virtual owner used when no token was
promoted at build.
"""
from __future__ import annotations

import dataclasses

import numpy as np

ROOT = -1
NEAR_TIE_REL = 1e-4

# --------------------------------------------------------------------------
# Promotion draws [A §三 "random promotion"; N key design 2]
# --------------------------------------------------------------------------
# [reading] The pages give no generator. Each head draws from SplitMix64
# (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
# OOPSLA 2014; constants of Vigna's public splitmix64.c). The stream of head h
# is seeded with ``seed + h * 2**40``; token t takes output number t of that
# stream. Counter based, so inserted tokens (t = their position) draw exactly
# as built ones do.

_U64 = np.uint64
_MASK = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def splitmix64_mix(z) -> np.ndarray:
    """SplitMix64 output function applied to the state word(s) ``z``."""
    z = np.atleast_1d(np.asarray(z, dtype=np.uint64))
    z = (z ^ (z >> _U64(30))) * _U64(_MIX1)
    z = (z ^ (z >> _U64(27))) * _U64(_MIX2)
    return z ^ (z >> _U64(31))


def splitmix64_outputs(seed: int, n: int, first: int = 0) -> np.ndarray:
    """Outputs ``first .. first+n-1`` of SplitMix64 seeded with ``seed``.

    The generator adds the golden gamma to its state before each output, so
    output i is ``mix(seed + (i+1) * gamma)`` (mod 2**64).
    """
    i = np.arange(first, first + n, dtype=np.uint64)
    state = _U64(seed & _MASK) + (i + _U64(1)) * _U64(_GOLDEN_GAMMA)
    return splitmix64_mix(state)


def head_stream_seed(seed: int, head: int) -> int:
    return (int(seed) + (int(head) << 40)) & _MASK


def ctz64(x) -> np.ndarray:
    """Number of trailing zero bits of each 64-bit word; 64 for zero."""
    x = np.atleast_1d(np.asarray(x, dtype=np.uint64))
    out = np.zeros(x.shape, dtype=np.int64)
    for k in range(64):
        low_bits = _U64((1 << (k + 1)) - 1)
        out += ((x & low_bits) == 0)
    return out


def draw_levels(seed: int, head: int, first: int, n: int, levels: int, promote_log2: int) -> np.ndarray:
    """Promotion level of tokens ``first .. first+n-1`` of one head.

    [A §三] every token starts at the bottom; a random part is promoted one
    level, and a smaller random part of *that* part once more. A token is
    promoted past level l with probability 2**-promote_log2 independently per
    level, i.e. ``level = floor(ctz(z) / promote_log2)`` capped at
    ``levels-1``. Nesting (level l+1 inside level l) holds by construction.
    """
    z = splitmix64_outputs(head_stream_seed(seed, head), n, first)
    return np.minimum(levels - 1, ctz64(z) // promote_log2).astype(np.int64)


# --------------------------------------------------------------------------
# Lift: inner product -> Euclidean distance [A §三, §六 "TK and TQ"]
# --------------------------------------------------------------------------
# [reading] TK/TQ are named but not printed. The pages say they normalise and
# add one dimension so that inner-product similarity becomes Euclidean
# distance. Keys: TK(k) = [k, sqrt(M^2 - |k|^2)] with M^2 the largest squared
# key norm of the build; queries: TQ(q) = [q, 0]. The positive scale of the
# pages' normalisation changes no ranking and is left out. M^2 is kept as the
# squared norm itself, so the largest key's extra coordinate is exactly 0. Keys
# inserted later use the build's M^2; a larger key gets 0 (a counted clamp).

def lift(K: np.ndarray):
    """Returns (|k|^2 per token, M^2, extra coordinate e per token)."""
    K = np.asarray(K, dtype=np.float64)
    n2 = (K * K).sum(axis=1)
    M2 = float(n2.max()) if n2.size else 0.0
    e = np.sqrt(np.maximum(0.0, M2 - n2))
    return n2, M2, e


def lift_one(k: np.ndarray, M2: float):
    """Lift of a key inserted after the build: (e, clamped?)."""
    n2 = float(np.dot(k, k))
    return float(np.sqrt(max(0.0, M2 - n2))), n2 > M2


def lifted(K: np.ndarray, e: np.ndarray) -> np.ndarray:
    return np.concatenate([np.asarray(K, np.float64), np.asarray(e, np.float64)[:, None]], axis=1)


# --------------------------------------------------------------------------
# Nearest parent [A §三 "parent = most similar word one level up"; N key design 2]
# --------------------------------------------------------------------------
# [reading] "most similar" is the smallest lifted squared Euclidean distance
# D(i,j) = |TK(k_i) - TK(k_j)|^2 (the lift exists to make this the measure).
# Equal distances go to the lower token id. D1/D2 are the best and second
# best distances; a point is a near-tie when D2 - D1 < 1e-4 * D2.

def _sq_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Squared Euclidean distance of row vector ``a`` to each row of ``b``."""
    diff = b - a[None, :]
    return (diff * diff).sum(axis=1)


def nearest(Xc: np.ndarray, Xp: np.ndarray, chunk: int = 1024):
    """For each row of Xc: index of the nearest row of Xp, D1 and D2.

    Candidates are ranked with the expansion |a|^2 + |b|^2 - 2 a.b (an fp64
    matmul). Rows whose best candidates lie within a rounding band (1e-9
    relative) of each other are re-ranked over that band with the direct sum
    of squared differences, so the choice is the brute-force argmin with the
    lowest index winning exact ties. D1 and D2 (best and runner-up distance)
    are then recomputed directly as sums of squared differences.
    """
    Xc = np.asarray(Xc, np.float64)
    Xp = np.asarray(Xp, np.float64)
    n_c, n_p = Xc.shape[0], Xp.shape[0]
    if n_p == 0:
        raise ValueError("no candidate parents")
    j_out = np.empty(n_c, dtype=np.int64)
    d1 = np.empty(n_c)
    d2 = np.full(n_c, np.inf)
    nc2 = (Xc * Xc).sum(axis=1)
    np2 = (Xp * Xp).sum(axis=1)
    for s in range(0, n_c, chunk):
        e = min(n_c, s + chunk)
        rows = np.arange(e - s)
        dexp = nc2[s:e, None] + np2[None, :] - 2.0 * (Xc[s:e] @ Xp.T)
        mn = dexp.min(axis=1)
        band = 1e-9 * (nc2[s:e] + np2.max()) + 1e-300
        j = dexp.argmin(axis=1)                 # first occurrence = lowest index
        close = dexp <= (mn + band)[:, None]
        for r in np.nonzero(close.sum(axis=1) > 1)[0]:
            c = np.nonzero(close[r])[0]
            dd = _sq_dist(Xc[s + r], Xp[c])
            j[r] = c[np.nonzero(dd == dd.min())[0][0]]
        j_out[s:e] = j
        diff = Xc[s:e] - Xp[j]
        d1[s:e] = (diff * diff).sum(axis=1)
        if n_p > 1:
            dexp[rows, j] = np.inf
            j2 = dexp.argmin(axis=1)
            diff = Xc[s:e] - Xp[j2]
            d2[s:e] = (diff * diff).sum(axis=1)
    return j_out, d1, d2


def is_near_tie(D1, D2) -> np.ndarray:
    D1 = np.asarray(D1, np.float64)
    D2 = np.asarray(D2, np.float64)
    with np.errstate(invalid="ignore"):
        return np.isfinite(D2) & ((D2 - D1) < NEAR_TIE_REL * D2)


def assign_parents(X: np.ndarray, lev: np.ndarray, L_top: int, pdci=None):
    """Parent of every point at every level below the top.

    ``pdci`` (an ``oracle.pdci.Pdci``) replaces the exact nearest point by the
    one P-DCI finds; its keys use the lift coordinate rounded to fp32.

    Returns lists indexed by level l = 0 .. L_top-1 of arrays over tokens:
    ``parent[l][t]`` (token id of the level-(l+1) owner, -1 if t is not a
    level-l point), ``dist[l][t]`` (D to that owner; 0 for a point that is
    itself at level l+1) and ``second[l][t]`` (runner-up distance).
    """
    n = X.shape[0]
    parent, dist, second = [], [], []
    for l in range(L_top):
        par = np.full(n, -1, dtype=np.int64)
        dst = np.full(n, np.nan)
        sec = np.full(n, np.inf)
        cand = np.nonzero(lev >= l + 1)[0]
        child = np.nonzero(lev == l)[0]
        par[cand] = cand            # a point of level l+1 is its own parent
        dst[cand] = 0.0
        if child.size and pdci is not None:
            from oracle import pdci as _pdci
            X32 = X.copy()
            X32[:, -1] = X32[:, -1].astype(np.float32)
            j, D1, D2 = _pdci.nearest_pdci(X[child], X32[child], X[cand], X32[cand], pdci)
            par[child] = cand[j]
            dst[child] = D1
            sec[child] = D2
        elif child.size:
            j, D1, D2 = nearest(X[child], X[cand])
            par[child] = cand[j]
            dst[child] = D1
            sec[child] = D2
        parent.append(par)
        dist.append(dst)
        second.append(sec)
    return parent, dist, second


# --------------------------------------------------------------------------
# Index state of one head
# --------------------------------------------------------------------------

@dataclasses.dataclass
class HeadIndex:
    head: int
    seed: int
    levels: int
    promote_log2: int
    page_cap: int
    K: np.ndarray                  # [n, d] fp64
    V: np.ndarray                  # [n, d] fp64
    n2: np.ndarray                 # [n]
    e: np.ndarray                  # [n] lift coordinate
    M2: float
    lev: np.ndarray                # [n] level used by the index (capped at L_top)
    L_top: int
    parent: list                   # per level l < L_top: [n] owner token (-1 = not a level-l point)
    dist: list                     # per level: [n] D to owner
    second: list                   # per level: [n] runner-up D
    pages: list                    # level-0 pages: list of token-id lists
    page_owner: list               # owner token (or ROOT) of each page
    owner_pages: dict              # owner -> ordered page ids
    children: dict                 # level l in 1..L_top-1 -> {owner: ordered level-l points}
    top: list                      # level-L_top points in order
    clamps: int = 0
    splits: int = 0
    insert_ties: int = 0
    # spare-capacity buffers behind the per-token arrays, so that a long run
    # of inserts appends in amortised constant time (storage only)
    _spare: dict = dataclasses.field(default_factory=dict, repr=False, compare=False)

    @property
    def n(self) -> int:
        return self.K.shape[0]

    @property
    def d(self) -> int:
        return self.K.shape[1]

    def X(self) -> np.ndarray:
        return lifted(self.K, self.e)

    def _append(self, name: str, arr: np.ndarray, x) -> np.ndarray:
        """``arr`` with ``x`` appended along axis 0, as a view of a buffer
        with room to spare (the values are exactly those of np.append)."""
        buf, view = self._spare.get(name, (None, None))
        n = arr.shape[0]
        if view is not arr or buf.shape[0] <= n:
            buf = np.empty((max(2 * n, 64),) + arr.shape[1:], dtype=arr.dtype)
            buf[:n] = arr
        buf[n] = x
        out = buf[:n + 1]
        self._spare[name] = (buf, out)
        return out


def pack(lev: np.ndarray, L_top: int, parent: list, dist: list, page_cap: int):
    """Pages and child lists from parent links [A §三; N key design 1, 2].

    [A §三] tokens that share a parent are stored in the same page; [N] each
    node maps to one physical page. [reading] A node with more children than
    fit one page is cut into several pages: walk the level-1 owners in
    ascending token id, order each owner's level-0 points (itself included,
    D = 0) by (D to the owner, token id) and cut them into consecutive runs of
    ``page_cap``; page ids follow that walk. Upper levels keep, per owner,
    the same (D, token id) order of its level-l points. With no promoted
    point a virtual root owns every token and pages are token-order runs.
    """
    n = lev.shape[0]
    pages, page_owner, owner_pages = [], [], {}
    children = {}
    if L_top == 0:
        groups = [(ROOT, list(range(n)))]
    else:
        groups = []
        for p in np.nonzero(lev >= 1)[0]:
            groups.append((int(p), None))
        # members of every owner, ordered by (D, token id): one pass collecting
        # the level-0 points of each owner, then a sort per owner.
        members = {int(p): [] for p, _ in groups}
        for t in range(n):
            members[int(parent[0][t])].append(t)
        groups = [(p, sorted(members[p], key=lambda t: (dist[0][t], t))) for p, _ in groups]
    for owner, toks in groups:
        ids = []
        for s in range(0, len(toks), page_cap):
            ids.append(len(pages))
            pages.append(list(toks[s:s + page_cap]))
            page_owner.append(owner)
        owner_pages[owner] = ids
    for l in range(1, L_top):
        members = {int(p): [] for p in np.nonzero(lev >= l + 1)[0]}
        for t in np.nonzero(lev >= l)[0]:
            members[int(parent[l][t])].append(int(t))
        children[l] = {p: sorted(m, key=lambda t: (dist[l][t], t)) for p, m in members.items()}
    # with no promoted point the virtual root owns the pages and there is no
    # top level of points to search
    top = [int(t) for t in np.nonzero(lev >= L_top)[0]] if L_top >= 1 else []
    return pages, page_owner, owner_pages, children, top


def build_head(K, V, head: int, seed: int, levels: int = 3, promote_log2: int = 4,
               page_cap: int = 16, lev: np.ndarray | None = None, parents=None, pdci=None) -> HeadIndex:
    """Index of one head from its prefill keys and values [N "Overall framework" step 1].

    ``lev`` overrides the promotion draws and ``parents`` the nearest-parent
    search (hand-worked cases; tie-tolerant replay of another implementation's
    choices). ``parents`` is a list over levels of arrays giving, for every
    level-l point that is not itself at level l+1, its owner token. ``pdci``
    (an ``oracle.pdci.Pdci``) finds parents by P-DCI instead of exactly.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n = K.shape[0]
    n2, M2, e = lift(K)
    if lev is None:
        lev = draw_levels(seed, head, 0, n, levels, promote_log2)
    lev = np.asarray(lev, dtype=np.int64)
    L_top = int(lev.max()) if n else 0
    X = lifted(K, e)
    if parents is None:
        parent, dist, second = assign_parents(X, lev, L_top, pdci)
    else:
        parent, dist, second = [], [], []
        for l in range(L_top):
            par = np.full(n, -1, dtype=np.int64)
            dst = np.full(n, np.nan)
            cand = np.nonzero(lev >= l + 1)[0]
            child = np.nonzero(lev == l)[0]
            par[cand] = cand
            dst[cand] = 0.0
            given = np.asarray(parents[l], dtype=np.int64)
            par[child] = given[child]
            if child.size and not np.all(lev[par[child]] >= l + 1):
                raise ValueError("given parent is not a level-(l+1) point")
            for t in child:
                dst[t] = float(_sq_dist(X[t], X[par[t]:par[t] + 1])[0])
            parent.append(par)
            dist.append(dst)
            second.append(np.full(n, np.inf))
    pages, page_owner, owner_pages, children, top = pack(lev, L_top, parent, dist, page_cap)
    return HeadIndex(head=head, seed=seed, levels=levels, promote_log2=promote_log2, page_cap=page_cap,
                     K=K, V=V, n2=n2, e=e, M2=M2, lev=lev, L_top=L_top, parent=parent, dist=dist,
                     second=second, pages=pages, page_owner=page_owner, owner_pages=owner_pages,
                     children=children, top=top)


def build_head_reuse(K, V, src: HeadIndex, head: int) -> HeadIndex:
    """[A §五 IceCache(reuse); N key design 4 "page reuse"] one layer's index
    serving another layer's head.

    [reading] The pages name inter-layer index reuse without its steps. Here
    the head takes ``src``'s structure as it stands (levels, parents, which
    tokens share a page and in what order, the child lists, the top list) and
    keeps its own keys, values and lift (M and e), so its selection scores its
    own keys inside the shared structure. Both hold the same token count.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if K.shape[0] != src.n:
        raise ValueError("the reusing head must hold as many tokens as its source")
    n2, M2, e = lift(K)
    X = lifted(K, e)
    dist = []
    for l in range(src.L_top):
        par = src.parent[l]
        dst = np.full(src.n, np.nan)
        has = np.nonzero(par >= 0)[0]
        for t in has:
            dst[t] = float(_sq_dist(X[t], X[par[t]:par[t] + 1])[0])
        dist.append(dst)
    return HeadIndex(head=head, seed=src.seed, levels=src.levels, promote_log2=src.promote_log2,
                     page_cap=src.page_cap, K=K, V=V, n2=n2, e=e, M2=M2, lev=src.lev.copy(), L_top=src.L_top,
                     parent=[p.copy() for p in src.parent], dist=dist,
                     second=[np.full(src.n, np.inf) for _ in range(src.L_top)],
                     pages=[list(p) for p in src.pages], page_owner=list(src.page_owner),
                     owner_pages={o: list(ps) for o, ps in src.owner_pages.items()},
                     children={l: {o: list(c) for o, c in ch.items()} for l, ch in src.children.items()},
                     top=list(src.top))


# --------------------------------------------------------------------------
# Incremental insert [A §三 "no rebuild"; N key design 2 "split on overflow"]
# --------------------------------------------------------------------------
# [reading] A new token t (next position) draws its level like any token,
# capped at the build's top level L_top. Below its level it is its own
# parent. At its level (if below the top) its parent is the nearest point of
# the *current* next level. No token already placed re-parents. At level 0
# it joins its owner's last page if that page has room; otherwise a new page
# (next free id) is split off, becomes the owner's last page and takes t
# (append split: placed tokens keep their slots). A promoted token opens its
# own first page. Upper-level child lists grow in arrival order. The re-sort
# split (``resplit``) is described at ``insert``; it touches level-0 pages
# only, the one level whose page boundaries decide what is selected and
# attended (upper levels are scored token by token).

RESPLIT_MAX = 1024   # [reading] owners with more members keep the append split


def insert(idx: HeadIndex, k, v, lev_override: int | None = None, parent_override: int | None = None,
           resplit: bool = False):
    """One new token (module notes above).

    ``resplit`` selects the other reading of the notes' split of an
    overflowing node [N key design 2]: when the owner's last page is full,
    a new page is still appended to its chain, and then the owner's members,
    the new token included, are re-sorted as the build packs them (lifted
    distance to the owner, the owner itself at 0, ties by token id) and
    re-cut into the owner's pages in chain order, so the new page ends up
    holding the farthest member. Page ids, chains and counts are those of
    the append split; only which member sits in which page and slot
    changes. [reading] Only owners that are tokens (not the virtual root,
    whose pages are token-order runs) with at most RESPLIT_MAX members
    re-sort; the others split by appending.
    """
    k = np.asarray(k, np.float64).reshape(-1)
    v = np.asarray(v, np.float64).reshape(-1)
    t = idx.n
    if lev_override is None:
        drawn = int(draw_levels(idx.seed, idx.head, t, 1, idx.levels, idx.promote_log2)[0])
    else:
        drawn = int(lev_override)
    lam = min(idx.L_top, drawn)
    e_t, clamped = lift_one(k, idx.M2)
    x = np.concatenate([k, [e_t]])
    p = None
    if lam < idx.L_top:
        cand = np.nonzero(idx.lev >= lam + 1)[0]
        if parent_override is None:
            j, D1, D2 = nearest(x[None, :], lifted(idx.K[cand], idx.e[cand]))
            p = int(cand[j[0]])
            if is_near_tie(D1, D2)[0]:
                idx.insert_ties += 1
            dp = float(D1[0])
        else:
            p = int(parent_override)
            if idx.lev[p] < lam + 1:
                raise ValueError("given parent is not a point of the next level")
            dp = float(_sq_dist(x, lifted(idx.K[p:p + 1], idx.e[p:p + 1]))[0])
    # grow token arrays
    idx.K = idx._append("K", idx.K, k)
    idx.V = idx._append("V", idx.V, v)
    idx.n2 = idx._append("n2", idx.n2, float(np.dot(k, k)))
    idx.e = idx._append("e", idx.e, e_t)
    idx.lev = idx._append("lev", idx.lev, lam)
    idx.clamps += int(clamped)
    for l in range(idx.L_top):
        par = idx._append(f"parent{l}", idx.parent[l], -1)
        dst = idx._append(f"dist{l}", idx.dist[l], np.nan)
        sec = idx._append(f"second{l}", idx.second[l], np.inf)
        if l < lam:
            par[t], dst[t] = t, 0.0
        elif l == lam:
            par[t], dst[t] = p, dp
        idx.parent[l], idx.dist[l], idx.second[l] = par, dst, sec
    # level-0 placement
    if idx.L_top == 0:
        owner0 = ROOT
    else:
        owner0 = t if lam >= 1 else p
    if owner0 == t or owner0 not in idx.owner_pages or not idx.owner_pages[owner0]:
        idx.owner_pages[owner0] = [len(idx.pages)]
        idx.pages.append([t])
        idx.page_owner.append(owner0)
    else:
        tail = idx.owner_pages[owner0][-1]
        if len(idx.pages[tail]) < idx.page_cap:
            idx.pages[tail].append(t)
        else:
            idx.owner_pages[owner0].append(len(idx.pages))
            idx.pages.append([t])
            idx.page_owner.append(owner0)
            idx.splits += 1
            members = [u for pg in idx.owner_pages[owner0] for u in idx.pages[pg]]
            if resplit and owner0 != ROOT and len(members) <= RESPLIT_MAX:
                # the build's packing key: D to the owner (0 for the owner
                # itself), then token id
                mem = np.asarray(members, dtype=np.int64)
                mem = mem[np.lexsort((mem, idx.dist[0][mem]))]
                for i, pg in enumerate(idx.owner_pages[owner0]):
                    idx.pages[pg] = [int(u) for u in mem[i * idx.page_cap:(i + 1) * idx.page_cap]]
    for l in range(1, idx.L_top):
        if lam > l:
            idx.children[l][t] = [t]
        elif lam == l:
            idx.children[l][p].append(t)
    if idx.L_top >= 1 and lam == idx.L_top:
        idx.top.append(t)
    return lam, p


# --------------------------------------------------------------------------
# Page selection [N key design 2 "top-down search", key design 3; A §六]
# --------------------------------------------------------------------------
# [reading] Beam descent: score the top level, keep the B best; at each lower
# level >= 1 score the children of the kept points and keep the B best; at
# level 0 the candidates are all pages of the kept level-1 points. "Find the
# k nearest points" is read as B = k by default (B is a parameter). Ranking
# by the lifted query distance |TQ(q) - TK(k)|^2 = |q|^2 + M^2 - 2 q.k is the
# same as ranking by q.k descending, which is what is computed. A page's
# score is the best q.k over its tokens [N "core idea": choosing the top-k
# pages approximates choosing the top-k tokens]. Budget T tokens = T/page_cap
# pages, whether or not a page is full. Ties go to the lower token / page id.

def _lifted_q_dist(s, q2: float, M2: float):
    return q2 + M2 - 2.0 * np.asarray(s, np.float64)


def _near_tied(sa: float, sb: float, q2: float, M2: float) -> bool:
    da, db = _lifted_q_dist(sa, q2, M2), _lifted_q_dist(sb, q2, M2)
    return bool(abs(da - db) <= NEAR_TIE_REL * max(abs(da), abs(db)))


def _cut(ids, scores, keep: int, q2: float, M2: float, forced=None):
    """Keep the ``keep`` best ids by (score desc, id asc).

    Returns (kept ids in rank order, tie?, admissible?). ``tie`` says the
    last kept and first dropped items are near-tied. With ``forced`` (the
    other implementation's kept list) the cut continues from it, after
    checking that every rank inversion it contains is a near-tie.
    """
    ids = np.asarray(ids, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float64)
    order = np.lexsort((ids, -scores))
    kept = ids[order[:keep]]
    tie = bool(len(order) > keep and keep > 0 and
               _near_tied(scores[order[keep - 1]], scores[order[keep]], q2, M2))
    if forced is None:
        return [int(x) for x in kept], tie, True
    forced = [int(x) for x in forced]
    sc = {int(i): float(s) for i, s in zip(ids, scores)}
    ok = (len(forced) == min(keep, len(ids)) and len(set(forced)) == len(forced)
          and all(f in sc for f in forced))
    if ok:
        fs = set(forced)
        # a dropped item may beat a kept one only when the two are near-tied
        for i, s in sc.items():
            if i in fs:
                continue
            for f in forced:
                if sc[f] < s and not _near_tied(sc[f], s, q2, M2):
                    ok = False
        # rank order inside the kept list: inversions only between near-ties
        for a, b in zip(forced, forced[1:]):
            if sc[a] < sc[b] and not _near_tied(sc[a], sc[b], q2, M2):
                ok = False
    return forced, tie, ok


def select(idx: HeadIndex, q, budget_tokens: int, beam: int, forced=None):
    """Top-k pages of one head for one query.

    Returns a dict: ``sel`` (page ids in rank order), ``kept`` (kept point
    lists per cut, top level first), ``ties`` (cuts that were near-tied) and
    ``admissible`` (False if a forced cut broke the ranking beyond the band).
    ``forced`` optionally holds the other implementation's kept lists in the
    same shape as ``kept`` followed by its ``sel``; the descent then
    continues from those.
    """
    q = np.asarray(q, np.float64).reshape(-1)
    q2 = float(np.dot(q, q))
    k_pages = budget_tokens // idx.page_cap
    ties, ok_all, kept_trace = 0, True, []
    cut_no = 0

    def take(ids, scores, keep):
        nonlocal ties, ok_all, cut_no
        f = None if forced is None else forced[cut_no]
        cut_no += 1
        out, tie, ok = _cut(ids, scores, keep, q2, idx.M2, f)
        ties += int(tie)
        ok_all &= ok
        return out

    if idx.n == 0:
        return dict(sel=[], kept=[], ties=0, admissible=True)
    if idx.L_top == 0:
        cand_pages = list(idx.owner_pages.get(ROOT, []))
    else:
        pts = np.asarray(idx.top, dtype=np.int64)
        kept = take(pts, idx.K[pts] @ q, beam)
        kept_trace.append(kept)
        for l in range(idx.L_top - 1, 0, -1):
            cand = [c for p in kept for c in idx.children[l][p]]
            cand = np.asarray(cand, dtype=np.int64)
            kept = take(cand, idx.K[cand] @ q, beam)
            kept_trace.append(kept)
        cand_pages = [pg for p in kept for pg in idx.owner_pages.get(p, [])]
    pscore = [float(np.max(idx.K[idx.pages[pg]] @ q)) for pg in cand_pages]
    sel = take(cand_pages, pscore, k_pages)
    return dict(sel=sel, kept=kept_trace, ties=ties, admissible=ok_all)


def gqa_union(sel_lists) -> list:
    """[N key design 3; A §六] pages of one KV group = union of its query heads' pages.

    [reading] The union is listed in ascending page id.
    """
    out = set()
    for s in sel_lists:
        out.update(int(p) for p in s if p >= 0)
    return sorted(out)


# --------------------------------------------------------------------------
# Sparse attention [N key design 1, attention weight formula]
# --------------------------------------------------------------------------
# a_j = s_j exp(q.k_j / sqrt(d)) / sum_j' s_j' exp(q.k_j' / sqrt(d)) with s the
# selection mask: a softmax over the tokens of the selected pages only.
# [reading] the caller passes the scale (1/sqrt(d) in the formula); the result
# also returns the log-sum-exp of the scaled logits.

def attend(idx: HeadIndex, q, pages, scale: float, resident=None, dense: bool = False):
    """[N key design 1] softmax attention over the tokens of ``pages``.

    [A §六] ``resident`` = (K_r, V_r), the head's sink and window tokens kept
    beside the index, join the same softmax. [N limitations] a ``dense`` head
    attends every indexed token instead of the selected pages. [reading] The
    resident tokens are given by the caller as plain rows; they are never
    indexed or selected.
    """
    q = np.asarray(q, np.float64).reshape(-1)
    if dense:
        pages = range(len(idx.pages))
    toks = np.asarray([t for pg in pages for t in idx.pages[pg]], dtype=np.int64)
    Kx, Vx = idx.K[toks], idx.V[toks]
    if resident is not None:
        Kx = np.concatenate([Kx, np.asarray(resident[0], np.float64).reshape(-1, idx.d)])
        Vx = np.concatenate([Vx, np.asarray(resident[1], np.float64).reshape(-1, idx.d)])
    if Kx.shape[0] == 0:
        return np.zeros(idx.d), -np.inf
    logits = (Kx @ q) * scale
    m = logits.max()
    w = np.exp(logits - m)
    l = w.sum()
    return (w @ Vx) / l, float(m + np.log(l))


# --------------------------------------------------------------------------
# Whole-batch helpers (H independent heads)
# --------------------------------------------------------------------------

def build_all(K, V, seed: int, levels: int = 3, promote_log2: int = 4, page_cap: int = 16,
              heads=None) -> list:
    """One index per head; ``heads`` selects a subset of head numbers."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    hs = range(K.shape[0]) if heads is None else heads
    return [build_head(K[h], V[h], h, seed, levels, promote_log2, page_cap) for h in hs]


def select_all(idxs: list, Q, budget_tokens: int, beam: int):
    """Q [H,G,d] -> (sel [H,G,k] with -1 padding, union per head, tie count)."""
    Q = np.asarray(Q, np.float64)
    H, G = Q.shape[0], Q.shape[1]
    k = budget_tokens // idxs[0].page_cap if idxs else 0
    sel = np.full((H, G, k), -1, dtype=np.int64)
    unis, ties = [], 0
    for h in range(H):
        lists = []
        for g in range(G):
            r = select(idxs[h], Q[h, g], budget_tokens, beam)
            sel[h, g, :len(r["sel"])] = r["sel"]
            lists.append(r["sel"])
            ties += r["ties"]
        unis.append(gqa_union(lists))
    return sel, unis, ties


def attend_all(idxs: list, Q, unis, scale: float):
    Q = np.asarray(Q, np.float64)
    H, G, d = Q.shape
    O = np.zeros((H, G, d))
    lse = np.full((H, G), -np.inf)
    for h in range(H):
        for g in range(G):
            O[h, g], lse[h, g] = attend(idxs[h], Q[h, g], unis[h], scale)
    return O, lse
