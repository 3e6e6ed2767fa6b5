"""Prioritized DCI nearest-parent search, written out plainly in fp64 NumPy.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and by ``oracle.icecache``
when a build asks for it, never by the library. It shares no code with the
HIP path.

Sources: the papernotes.org notes "IceCache: Memory-Efficient KV-cache
Management for Long-Sequence LLMs", key design 2 (M-DCI sits on Prioritized
Dynamic Continuous Indexing: no space partitioning, several indices that
each project the points onto a random direction and order them by how far
their projection lies from the query's, a priority queue expanding the
closest first), and the aitangshan.cn IceCache article, section 3, which
names P-DCI as the prior work the tree builds on. The structure of the
indices follows the published method (Li and Malik, "Fast k-Nearest
Neighbour Search via Prioritized DCI", ICML 2017): m composite indices of l
simple indices each; a composite index yields a point as a candidate once
all of its l simple indices have visited it; it stops after ``visits`` visits
or ``cands`` candidates; the candidates of all composite indices are ranked
by their true distance.

[reading] The pages print neither the parameters nor the queue's tie rules:
- directions are inputs (rows of ``dirs``, simple index i of composite j is
  row j*l + i), shared by every level and head;
- a simple index is walked outward from the query's position in its sorted
  keys (sorted by key, then point), one neighbour per step on either side; the
  queue of a composite index pops the walker front with the smallest
  |key - query key|, ties by simple index, then point;
- projections use the lift coordinate as the index stores it (rounded to
  fp32), so both implementations order identical values; the final ranking
  uses the fp64 lifted distance like the exact search, ties to the lower
  token id, near-ties as there.
"""
from __future__ import annotations

import dataclasses
import heapq

import numpy as np


@dataclasses.dataclass
class Pdci:
    dirs: np.ndarray    # [m*l, d+1] projection directions (fp32 values)
    m: int              # composite indices
    l: int              # simple indices per composite index
    visits: int         # visits per composite index at most
    cands: int          # candidates per composite index at most


def project(X32: np.ndarray, dirs: np.ndarray) -> np.ndarray:
    """Keys of every point in every simple index: [n, m*l], fp64."""
    return np.asarray(X32, np.float64) @ np.asarray(dirs, np.float64).T


def candidates(qkey: np.ndarray, keys: np.ndarray, cfg: Pdci) -> list:
    """Candidate point indices for one query: for each composite index, the
    points completed (visited by all its simple indices) in visit order, as
    many as its budgets allow; composite indices in order, repeats kept.

    qkey: [m*l] the query's keys; keys: [n, m*l] the points' keys.
    """
    n = keys.shape[0]
    out = []
    for j in range(cfg.m):
        heap = []
        orders = []
        for i in range(cfg.l):
            col = keys[:, j * cfg.l + i]
            order = np.lexsort((np.arange(n), col))       # by key, then point
            orders.append((order, col[order]))
            pos = int(np.searchsorted(col[order], qkey[j * cfg.l + i], side="left"))
            for side, p in ((-1, pos - 1), (1, pos)):
                if 0 <= p < n:
                    c = int(order[p])
                    heapq.heappush(heap, (abs(col[c] - qkey[j * cfg.l + i]), i, c, side, p))
        seen = {}
        found = []
        visits = 0
        # [reading] the visit budget ends a walk only once it has a candidate,
        # so every composite index yields at least one
        while heap and len(found) < cfg.cands and (visits < cfg.visits or not found):
            _, i, c, side, p = heapq.heappop(heap)
            visits += 1
            seen[c] = seen.get(c, 0) + 1
            if seen[c] == cfg.l:
                found.append(c)
            order, sk = orders[i]
            p += side
            if 0 <= p < n:
                c2 = int(order[p])
                heapq.heappush(heap, (abs(sk[p] - qkey[j * cfg.l + i]), i, c2, side, p))
        out.extend(found)
    return out


def nearest_pdci(Xc_child: np.ndarray, Kc_child: np.ndarray, Xc: np.ndarray, Kc: np.ndarray, cfg: Pdci):
    """For each child row: (index into the candidate rows, D1, D2) found by
    P-DCI. Xc_child / Xc: fp64 lifted rows for the distances; Kc_child / Kc:
    the same rows with the lift coordinate rounded to fp32, for the keys.
    D2 is the runner-up among the distinct candidates (inf if only one)."""
    nq = Xc_child.shape[0]
    keys = project(Kc, cfg.dirs)
    qkeys = project(Kc_child, cfg.dirs)
    idx = np.zeros(nq, dtype=np.int64)
    D1 = np.full(nq, np.inf)
    D2 = np.full(nq, np.inf)
    for r in range(nq):
        cs = sorted(set(candidates(qkeys[r], keys, cfg)))
        diff = Xc[cs] - Xc_child[r][None, :]
        d = (diff * diff).sum(axis=1)
        o = np.lexsort((np.asarray(cs), d))
        idx[r] = cs[o[0]]
        D1[r] = d[o[0]]
        if len(cs) > 1:
            D2[r] = d[o[1]]
    return idx, D1, D2
