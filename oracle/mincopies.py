"""Oracle: brute-force minimum number of redundant expert copies (test infrastructure, tiny inputs).

The pages call their planner a near-optimal online integer program but do not
state its objective ([P1] abstract; [P2] "Core technique").  The reading used
here: a copy is an (expert e, rank d != home(e)) pair that carries at least one
of e's pairs; minimise the number of copies subject to every rank holding
exactly P pairs and every expert's T_e pairs being placed; optionally also
subject to a slot cap (every rank receives at most B distinct non-home
experts, so that none is read directly from its home row).

Method: try every set of allowed non-home edges, smallest sets first, and test
each with a max-flow (source -> expert, capacity T_e; expert -> its home rank
and -> each chosen rank, unbounded; rank -> sink, capacity P).  The first size
with a flow of N is the minimum.  Exponential; meant for R <= 4, E <= 16.
"""
from __future__ import annotations

from itertools import combinations

import numpy as np
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import maximum_flow


def _feasible(T, R, P, home, edges) -> bool:
    E = len(T)
    N = int(np.sum(T))
    src, sink = E + R, E + R + 1
    rows, cols, caps = [], [], []

    def add(a, b, c):
        rows.append(a)
        cols.append(b)
        caps.append(int(c))

    for e in range(E):
        if T[e] > 0:
            add(src, e, T[e])
            add(e, E + home[e], N)
    for (e, d) in edges:
        add(e, E + d, N)
    for r in range(R):
        add(E + r, sink, P)
    n = E + R + 2
    g = csr_matrix((np.array(caps, dtype=np.int32), (np.array(rows), np.array(cols))), shape=(n, n))
    return maximum_flow(g, src, sink).flow_value == N


def lower_bound(T, R, P) -> int:
    """Every overloaded rank needs an outgoing copy and every underloaded rank an incoming one."""
    E = len(T)
    per = E // R
    load = np.array([np.sum(T[r * per:(r + 1) * per]) for r in range(R)])
    return int(max(np.sum(load > P), np.sum(load < P)))


def min_copies(T, R: int, P: int, max_size: int | None = None, slot_cap: int | None = None):
    """Smallest number of non-home (expert, rank) placements that balances every rank to exactly P.

    With ``slot_cap`` = B, only placements in which every rank receives at most B distinct non-home
    experts count (each one then fits a prefetch slot: no direct reads); returns None when no such
    placement exists.
    """
    T = np.asarray(T, dtype=np.int64)
    E = len(T)
    per = E // R
    home = [e // per for e in range(E)]
    assert int(T.sum()) == R * P
    cand = [(e, d) for e in range(E) if T[e] > 0 for d in range(R) if d != home[e]]
    top = len(cand) if max_size is None else max_size
    for size in range(0, top + 1):
        for edges in combinations(cand, size):
            if slot_cap is not None and max(np.bincount([d for _, d in edges], minlength=R)) > slot_cap:
                continue
            if _feasible(T, R, P, home, edges):
                return size
    if slot_cap is not None:
        return None
    raise RuntimeError("no balancing placement within the size limit")
