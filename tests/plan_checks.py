"""Checks shared by the planner tests (CPU and GPU): invariants any correct plan satisfies,
and a list-based simulation of the home-first planner for tiny inputs.

Neither helper calls the oracle or the HIP library; they take plans as plain arrays.
"""
from __future__ import annotations

import numpy as np


def check_plan_invariants(topk_idx, E, B, cu, slot_expert, dest_idx, src_of_row=None, stats=None,
                          planner="prefix"):
    """Invariants from the pages and the planner reading; raises AssertionError on the first violation.

    planner="prefix": every rank keeps the first min(P, L_r) pairs of its canonical home list.
    planner="mincopy": every expert keeps a canonical prefix of its pairs, and an overloaded rank's
    overflow leaves through its home experts largest first (equal counts: lower id first): in that
    order the experts are wholly overflowed, then at most one partly, then kept whole.
    """
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    R, S, K = topk_idx.shape
    P, N, per = S * K, R * S * K, E // R
    ids = topk_idx.reshape(-1)
    cu = np.asarray(cu, dtype=np.int64)
    slot_expert = np.asarray(slot_expert, dtype=np.int64)
    dest = np.asarray(dest_idx, dtype=np.int64).reshape(-1)
    assert cu.shape == (R, E + B + 1)
    # exact S*K pairs per rank, monotone group boundaries
    assert np.all(cu[:, 0] == 0) and np.all(cu[:, -1] == P), "every rank must hold exactly S*K pairs"
    assert np.all(np.diff(cu, axis=1) >= 0)
    # destinations form a bijection onto [0, N)
    assert dest.min() >= 0 and dest.max() < N
    assert len(np.unique(dest)) == N, "dest_idx must be a permutation of the rows"
    inv = np.empty(N, dtype=np.int64)
    inv[dest] = np.arange(N)
    if src_of_row is not None:
        assert np.array_equal(np.asarray(src_of_row, dtype=np.int64), inv)
    # every row's expert matches its group; rows inside a group keep canonical order
    copies = {}
    for r in range(R):
        for g in range(E + B):
            a, b = r * P + cu[r, g], r * P + cu[r, g + 1]
            if b == a:
                continue
            qs = inv[a:b]
            assert np.all(np.diff(qs) > 0), "rows in a group keep canonical (src, token, k) order"
            es = ids[qs]
            if g < E:
                assert np.all(es == g), "home-row group g holds only expert g"
                if g // per != r:
                    copies.setdefault(r, []).append((g, "direct"))
            else:
                e = slot_expert[r, g - E]
                assert e >= 0, "a non-empty slot group needs a slot expert"
                assert np.all(es == e)
                assert e // per != r, "a slot never holds a home expert of its own rank"
                copies.setdefault(r, []).append((e, "slot"))
    for r in range(R):
        used = [e for e in slot_expert[r] if e >= 0]
        assert len(used) == len(set(used)), "at most one slot per (expert, rank)"
        # slots are used first and in ascending expert order; direct reads only past B
        js = [j for j in range(B) if slot_expert[r, j] >= 0]
        assert js == list(range(len(js))), "slots fill from j = 0"
        assert used == sorted(used)
        lst = copies.get(r, [])
        n_direct = sum(1 for _, kind in lst if kind == "direct")
        if n_direct:
            assert len(js) == B, "direct reads only once all B slots are taken"
            slot_es = [e for e, k in lst if k == "slot"]
            if slot_es:
                assert max(slot_es) < min(e for e, k in lst if k == "direct"), "slots go to the lowest experts"
    if planner == "prefix":  # home-first: rank r keeps the first min(P, L_r) pairs of its canonical home list
        for r in range(R):
            home_pairs = [q for e in range(r * per, (r + 1) * per) for q in np.nonzero(ids == e)[0]]
            kept = [q for q in home_pairs if dest[q] // P == r]
            assert kept == home_pairs[:min(P, len(home_pairs))], "home-first prefix property"
    else:
        assert planner == "mincopy"
        for r in range(R):
            experts = list(range(r * per, (r + 1) * per))
            T = {e: int(np.sum(ids == e)) for e in experts}
            kept_n = {}
            for e in experts:
                qs = list(np.nonzero(ids == e)[0])
                kept = [q for q in qs if dest[q] // P == r]
                assert kept == qs[:len(kept)], "every expert keeps a canonical prefix of its pairs"
                kept_n[e] = len(kept)
            assert sum(kept_n.values()) == min(P, sum(T.values())), "an overloaded rank keeps exactly P"
            order = sorted(experts, key=lambda e: (-T[e], e))
            state = [0 if kept_n[e] == 0 and T[e] > 0 else (2 if kept_n[e] == T[e] else 1) for e in order]
            assert state == sorted(state) and state.count(1) <= 1, "overflow leaves through the largest experts"
    # contiguous cut: overflow pairs in canonical order go to non-decreasing ranks
    over = []
    for e in range(E):
        for q in np.nonzero(ids == e)[0]:
            if dest[q] // P != e // per:
                over.append(dest[q] // P)
    assert over == sorted(over), "overflow list is cut contiguously, in rank order"
    if stats is not None:
        n_copies = sum(len(v) for v in copies.values())
        n_direct = sum(1 for v in copies.values() for _, k in v if k == "direct")
        assert list(np.asarray(stats)[:3]) == [n_copies, n_copies - n_direct, n_direct]
    return True


def list_plan(topk_idx, E, B, planner="prefix"):
    """Builds every rank's buffer by moving pair ids between Python lists.

    Rank r lists its home experts' pairs (ascending expert, then ascending pair
    id) and keeps the first P (planner="mincopy": it strips its excess from the
    tails of its experts' lists, the longest list first, equal lengths lower
    expert first); the leftovers of all ranks, in rank order and ascending
    expert within a rank, are handed to the ranks below P in rank order; each
    receiving rank gives its arrived experts slots in ascending order (home-row
    groups past B).  Returns (cu [R,E+B+1], slot_expert [R,B], dest [R,S,K]).
    """
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    R, S, K = topk_idx.shape
    P, N, per = S * K, R * S * K, E // R
    ids = [int(x) for x in topk_idx.reshape(-1)]
    kept, overflow, load = {}, [], {}
    for r in range(R):
        mine = [(e, q) for e in range(r * per, (r + 1) * per) for q in range(N) if ids[q] == e]
        load[r] = len(mine)
        if planner == "prefix":
            kept[r], overflow = mine[:P], overflow + mine[P:]
            continue
        lists = {e: [(ee, q) for ee, q in mine if ee == e] for e in range(r * per, (r + 1) * per)}
        strip = {e: 0 for e in lists}
        excess = len(mine) - P
        for e in sorted(lists, key=lambda e: (-len(lists[e]), e)):
            strip[e] = max(0, min(len(lists[e]), excess))
            excess -= strip[e]
        kept[r] = [x for e in sorted(lists) for x in lists[e][:len(lists[e]) - strip[e]]]
        overflow = overflow + [x for e in sorted(lists) for x in lists[e][len(lists[e]) - strip[e]:]]
    received = {}
    for d in range(R):
        need = max(0, P - load[d])
        received[d], overflow = overflow[:need], overflow[need:]
    assert overflow == []
    cu = np.zeros((R, E + B + 1), dtype=np.int64)
    slot_expert = -np.ones((R, B), dtype=np.int64)
    dest = np.empty(N, dtype=np.int64)
    for d in range(R):
        arrived = sorted({e for e, _ in received[d]})
        slot = {e: j for j, e in enumerate(arrived)}
        groups = [[] for _ in range(E + B)]
        for e, q in kept[d]:
            groups[e].append(q)
        for e, q in received[d]:
            j = slot[e]
            if j < B:
                slot_expert[d, j] = e
                groups[E + j].append(q)
            else:
                groups[e].append(q)
        row = 0
        for g in range(E + B):
            for q in groups[g]:
                dest[q] = d * P + row
                row += 1
            cu[d, g + 1] = row
    return cu, slot_expert, dest.reshape(R, S, K)


def random_routing(rng, R, S, K, E, skew):
    """Tiny random routing with distinct experts per token and a tunable skew (test-only)."""
    w = np.exp(skew * rng.standard_normal(E))
    out = np.empty((R, S, K), dtype=np.int64)
    for r in range(R):
        for s in range(S):
            out[r, s] = rng.choice(E, size=K, replace=False, p=w / w.sum())
    return out
