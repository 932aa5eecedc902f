"""Oracle: expert histogram, maxvio, and the home-first prefix-sum planner (test infrastructure).

Everything is numpy int64 / Python float64, written for readability, not speed.

What the pages fix:
  * maxvio = max_e(T_e / Tbar) - 1, T_e the number of (token, k) pairs routed
    to expert e, Tbar the mean under perfect balance ([P2] "Core problem";
    [P3] paragraph two).
  * Every rank receives exactly S*K pairs whatever the skew, by planning a few
    redundant experts from the current router output ([P1] section 2; [P2]
    "Core technique"; [P3] paragraph three).
  * Rows [0,E) of the per-rank weight tensor are the home experts, E/R per
    rank; rows [E,E+B) are the rank's prefetch slots; a rank that needs more
    remote experts than it has slots reads their home rows directly; the
    planner emits cu_seqlens over the E+B rows ([P2] "Memory contract and
    weight layout").

Readings where the pages leave a step open (each one is listed in the design
notes of the repository):
  * home(e) = e // (E/R): contiguous blocks of E/R experts per rank.
  * Canonical pair order is (expert, src rank, token, k); the flat pair id
    q = (src*S + token)*K + k is already in (src, token, k) order, so the order
    inside one expert is ascending q.
  * Home-first ("prefix" planner): rank r walks its home experts in ascending
    order and keeps the first P = S*K pairs of that list; the rest overflow.
  * Fewest copies ("mincopy" planner, the pages' planner minimises the
    redundant experts it creates but does not print its program): an
    overloaded rank sends its excess L_r - P out of as few of its experts as
    possible -- its home experts largest first (equal counts: lower id first),
    each overflowing in turn until the excess is covered -- and keeps the first
    keep_e pairs of every expert.  Everything after the keep counts is the
    same for both planners.
  * The overflow list is every overflow pair in ascending (expert, order); the
    deficits D_r = max(0, P - L_r) of underloaded ranks are filled from it in
    rank order, each deficit taking one contiguous cut.
  * On a receiving rank the distinct experts of its cut, in ascending expert
    order, take slots j = 0, 1, ...; an expert with j >= B is read directly
    from its home row (group g = e).
  * cu_seqlens is stored as [R, E+B+1] with a leading zero; groups g < E come
    before the slot groups; rows inside a group keep the canonical order.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Plan:
    expert_counts: np.ndarray  # [E] int64, T_e
    maxvio: float
    cu_seqlens: np.ndarray  # [R, E+B+1] int64
    slot_expert: np.ndarray  # [R, B] int64, -1 = unused slot
    dest_idx: np.ndarray  # [R, S, K] int64, global row in the [R*S*K, .] buffer
    src_of_row: np.ndarray  # [R*S*K] int64, flat pair id that lands on each row
    stats: np.ndarray  # [4] int64: copies, slotted, direct_read, invalid_ids
    # intermediate quantities, kept for tests
    keep: np.ndarray  # [E]
    over: np.ndarray  # [E]
    load: np.ndarray  # [R] L_r, pairs whose home is r
    deficit: np.ndarray  # [R]
    flows: dict  # (expert, dest rank) -> pairs moved


def home_rank(e, E: int, R: int):
    """Owner of expert e: ranks hold contiguous blocks of E/R experts."""
    return e // (E // R)


def histogram(topk_idx: np.ndarray, E: int) -> np.ndarray:
    """T_e: how many (token, k) pairs chose expert e."""
    return np.bincount(np.asarray(topk_idx).reshape(-1).astype(np.int64), minlength=E)[:E]


def maxvio(counts: np.ndarray, n_pairs: int) -> float:
    """max_e(T_e / Tbar) - 1 with Tbar = N / E, evaluated as (E * max T) / N - 1 in float64.

    With no pairs at all (N = 0) the ratio is 0/0; the reading used here is that an
    empty routing has no imbalance, maxvio = 0.
    """
    if n_pairs == 0:
        return 0.0
    E = len(counts)
    return float(E * int(np.max(counts))) / float(n_pairs) - 1.0


def stable_order(ids: np.ndarray) -> np.ndarray:
    """ord(q): number of earlier pairs (smaller flat id) that chose the same expert."""
    ids = np.asarray(ids, dtype=np.int64)
    perm = np.argsort(ids, kind="stable")
    sorted_ids = ids[perm]
    first = np.searchsorted(sorted_ids, sorted_ids, side="left")
    out = np.empty_like(ids)
    out[perm] = np.arange(len(ids)) - first
    return out


PLANNERS = ("prefix", "mincopy")


def keep_counts(T: np.ndarray, R: int, P: int, planner: str = "prefix"):
    """How many of each expert's pairs stay on its home rank, and L_r, the pairs whose expert lives on r.

    prefix:  rank r walks its home experts in ascending order and keeps the first P pairs of that list.
    mincopy: a rank with L_r > P must send out L_r - P pairs; it takes its home experts largest first
             (equal counts: lower id first) and overflows each of them in turn, as much as is still
             needed, so the excess leaves through the fewest experts; the last one may keep some pairs.
    """
    E = len(T)
    per = E // R
    keep = np.zeros(E, dtype=np.int64)
    load = np.zeros(R, dtype=np.int64)
    for r in range(R):
        experts = list(range(r * per, (r + 1) * per))
        load[r] = sum(int(T[e]) for e in experts)
        if planner == "prefix":
            before = 0  # pairs of r's lower-numbered home experts
            for e in experts:
                keep[e] = min(max(P - before, 0), T[e])
                before += T[e]
        elif planner == "mincopy":
            excess = load[r] - P
            for e in experts:
                keep[e] = T[e]
            for e in sorted(experts, key=lambda e: (-T[e], e)):
                if excess <= 0:
                    break
                moved = min(int(T[e]), excess)
                keep[e] = T[e] - moved
                excess -= moved
        else:
            raise ValueError(f"unknown planner {planner!r}")
    return keep, load


def plan(topk_idx: np.ndarray, E: int, B: int, planner: str = "prefix") -> Plan:
    """Balanced plan for router output ``topk_idx`` [R, S, K]: the home-first prefix planner, or with
    planner="mincopy" the planner that sends each rank's excess out of the fewest experts."""
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    R, S, K = topk_idx.shape
    assert E % R == 0 and B >= 0
    per = E // R
    P = S * K
    N = R * P
    ids = topk_idx.reshape(-1)
    assert ids.min() >= 0 and ids.max() < E

    # Step 1: histogram and skew.
    T = histogram(ids, E)
    mv = maxvio(T, N)

    # Step 2: canonical order inside each expert.
    order = stable_order(ids)

    # Step 3: keep counts (which of each expert's pairs stay home: the first keep_e of its canonical
    # list).  L_r = pairs whose expert lives on r.
    keep, load = keep_counts(T, R, P, planner)
    over = T - keep

    # Step 4: the overflow list (ascending expert, then order) and the deficits.
    ov_start = np.concatenate([[0], np.cumsum(over)[:-1]])
    deficit = np.maximum(0, P - load)
    def_start = np.concatenate([[0], np.cumsum(deficit)[:-1]])
    assert over.sum() == deficit.sum()  # sum_r L_r = R*P

    # Step 5: contiguous cut of the overflow list into the deficits, in rank order.
    flows = {}
    for e in range(E):
        a0, a1 = ov_start[e], ov_start[e] + over[e]
        for d in range(R):
            b0, b1 = def_start[d], def_start[d] + deficit[d]
            amount = min(a1, b1) - max(a0, b0)
            if amount > 0:
                flows[(e, d)] = int(amount)

    # Step 6: slots on each receiving rank, experts in ascending order.
    slot_expert = -np.ones((R, B), dtype=np.int64)
    group_of = {}  # (e, d) -> group row on rank d
    copies = slotted = direct = 0
    for d in range(R):
        received = sorted(e for (e, dd) in flows if dd == d)
        for j, e in enumerate(received):
            copies += 1
            if j < B:
                slot_expert[d, j] = e
                group_of[(e, d)] = E + j
                slotted += 1
            else:
                group_of[(e, d)] = e  # read the home row directly
                direct += 1

    # Step 7: group sizes and cu_seqlens per rank.
    cnt = np.zeros((R, E + B), dtype=np.int64)
    for e in range(E):
        cnt[home_rank(e, E, R), e] += keep[e]
    for (e, d), amount in flows.items():
        cnt[d, group_of[(e, d)]] += amount
    cu = np.zeros((R, E + B + 1), dtype=np.int64)
    cu[:, 1:] = np.cumsum(cnt, axis=1)

    # Step 8: destination row of every pair (array form of one rule per pair).
    #   kept pair:     rank home(e), group e, position ord
    #   overflow pair: list position v = OvStart_e + ord - keep_e; the rank d whose
    #                  deficit interval holds v; the group chosen in step 6; the
    #                  position inside that (e, d) cut.
    group = -np.ones((R, E), dtype=np.int64)
    for (e, d), g in group_of.items():
        group[d, e] = g
    kept = order < keep[ids]
    v = ov_start[ids] + order - keep[ids]
    d_over = np.searchsorted(def_start + deficit, v, side="right")
    d_over = np.where(kept, 0, d_over)
    assert np.all(kept | ((def_start[d_over] <= v) & (v < def_start[d_over] + deficit[d_over])))
    d = np.where(kept, home_rank(ids, E, R), d_over)
    g = np.where(kept, ids, group[d_over, ids])
    pos = np.where(kept, order, v - np.maximum(ov_start[ids], def_start[d_over]))
    assert np.all(g >= 0)
    dest = d * P + cu[d, g] + pos
    src_of_row = np.empty(N, dtype=np.int64)
    src_of_row[dest] = np.arange(N)

    stats = np.array([copies, slotted, direct, 0], dtype=np.int64)
    return Plan(T, mv, cu, slot_expert, dest.reshape(R, S, K), src_of_row, stats,
                keep, over, load, deficit, flows)

