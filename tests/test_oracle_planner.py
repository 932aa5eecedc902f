"""Pins the planner oracle to what the pages and arithmetic fix (CPU only).

Pins: hand-worked examples (tests/golden), maxvio closed forms, plan
invariants over 100 seeds, a list-based simulation of the same planner on tiny
inputs, the brute-force minimum copy count, and planted mistakes that each pin
must catch.
"""
import json
import os

import numpy as np
import pytest

from oracle import mincopies, planner
from tests.plan_checks import check_plan_invariants, list_plan, random_routing

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _check_example(g):
    p = planner.plan(np.array(g["topk_idx"]), g["E"], g["B"])
    assert p.expert_counts.tolist() == g["expert_counts"]
    assert abs(p.maxvio - g["maxvio_num"] / g["maxvio_den"]) < 1e-15
    assert p.cu_seqlens.tolist() == g["cu_seqlens"]
    assert p.slot_expert.tolist() == g["slot_expert"]
    assert p.dest_idx.tolist() == g["dest_idx"]
    assert p.stats.tolist() == g["stats"]
    return p


@pytest.mark.parametrize("name", ["plan_example1.json", "plan_example2.json"])
def test_hand_worked_examples(name):
    g = load(name)
    p = _check_example(g)
    check_plan_invariants(g["topk_idx"], g["E"], g["B"], p.cu_seqlens, p.slot_expert, p.dest_idx,
                          p.src_of_row, p.stats)
    assert mincopies.min_copies(p.expert_counts, g["R"], g["S"] * g["K"]) == g["min_copies"]


def routing_from_counts(counts, R, S, K):
    """Distinct-per-token routing with the given per-expert counts (each count <= R*S).

    Lists the ids in expert order and gives token t the ids at positions
    t, t + R*S, t + 2*R*S, ...
    """
    lst = np.repeat(np.arange(len(counts)), counts)
    T = R * S
    assert len(lst) == T * K and max(counts) <= T
    return np.stack([lst[k * T:(k + 1) * T] for k in range(K)], axis=1).reshape(R, S, K)


def test_example3_training_budget_exceeded():
    g = load("plan_example3_counts.json")
    idx = routing_from_counts(g["expert_counts"], g["R"], g["S"], g["K"])
    assert all(len(set(t)) == g["K"] for t in idx.reshape(-1, g["K"]).tolist())
    p = planner.plan(idx, g["E"], g["B"])
    assert p.expert_counts.tolist() == g["expert_counts"]
    assert p.maxvio == g["maxvio"]
    assert p.load.tolist() == g["load"]
    assert [e for e in range(g["E"]) if p.over[e] > 0] == g["overflow_experts"]
    assert p.slot_expert[3].tolist() == g["slot_expert_rank3"]
    assert p.stats.tolist() == g["stats"]
    check_plan_invariants(idx, g["E"], g["B"], p.cu_seqlens, p.slot_expert, p.dest_idx, p.src_of_row, p.stats)
    P = g["S"] * g["K"]
    assert mincopies.lower_bound(p.expert_counts, g["R"], P) == g["min_copies"]
    assert mincopies.min_copies(p.expert_counts, g["R"], P, max_size=3) == g["min_copies"]


@pytest.mark.parametrize("E,K", [(16, 2), (64, 6), (256, 8), (384, 8)])
def test_maxvio_closed_forms(E, K):
    # perfectly balanced counts -> 0
    T = 1000
    assert planner.maxvio(np.full(E, T), E * T) == 0.0
    # one expert picked by every token: T_max = #tokens = N/K -> E/K - 1
    tokens = 3 * E
    counts = np.full(E, (tokens * K - tokens) // (E - 1))
    counts[0] = tokens
    n = tokens * K
    assert planner.maxvio(counts, n) == float(E * tokens) / float(n) - 1.0
    assert abs(planner.maxvio(counts, n) - (E / K - 1)) < 1e-12


def test_maxvio_of_empty_routing_is_zero():
    assert planner.maxvio(np.zeros(8, dtype=np.int64), 0) == 0.0


def test_stable_order_brute_force():
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 7, size=300)
    want = [int(np.sum(ids[:q] == ids[q])) for q in range(len(ids))]
    assert planner.stable_order(ids).tolist() == want


def test_histogram_brute_force():
    rng = np.random.default_rng(6)
    idx = random_routing(rng, 3, 20, 3, 9, 1.0)
    T = planner.histogram(idx, 9)
    assert T.sum() == idx.size
    assert T.tolist() == [int(np.sum(idx == e)) for e in range(9)]


def _small_case(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.integers(1, 5))
    per = int(rng.integers(1, 5))
    E = R * per
    K = int(rng.integers(1, min(E, 4) + 1))
    S = int(rng.integers(1, 9))
    B = int(rng.integers(0, per + 3))
    skew = float(rng.uniform(0, 3))
    return random_routing(rng, R, S, K, E, skew), E, B


@pytest.mark.parametrize("seed", range(100))
def test_invariants_and_list_simulation(seed):
    idx, E, B = _small_case(seed)
    p = planner.plan(idx, E, B)
    check_plan_invariants(idx, E, B, p.cu_seqlens, p.slot_expert, p.dest_idx, p.src_of_row, p.stats)
    cu, slots, dest = list_plan(idx, E, B)
    assert np.array_equal(cu, p.cu_seqlens)
    assert np.array_equal(slots, p.slot_expert)
    assert np.array_equal(dest, p.dest_idx)


@pytest.mark.parametrize("seed", range(25))
def test_copies_at_least_brute_force_minimum(seed):
    rng = np.random.default_rng(2000 + seed)
    R = int(rng.integers(2, 5))
    per = int(rng.integers(1, 3))
    E = R * per
    K = int(rng.integers(1, min(E, 3) + 1))
    S = int(rng.integers(1, 6))
    idx = random_routing(rng, R, S, K, E, float(rng.uniform(0.5, 3)))
    p = planner.plan(idx, E, B=E)
    lb = mincopies.lower_bound(p.expert_counts, R, S * K)
    m = mincopies.min_copies(p.expert_counts, R, S * K)
    assert lb <= m <= p.stats[0]


def test_balanced_routing_needs_no_copies():
    # every rank's home experts receive exactly P pairs -> everything stays home
    R, S, K, E = 4, 8, 2, 8
    counts = np.full(E, R * S * K // E)
    idx = routing_from_counts(counts, R, S, K)
    p = planner.plan(idx, E, B=2)
    assert p.stats.tolist() == [0, 0, 0, 0]
    assert np.all(p.slot_expert == -1)
    per = E // R
    assert np.all(p.dest_idx.reshape(-1) // (S * K) == idx.reshape(-1) // per)


# ------------------------------------------------------------ planted mistakes


def test_pins_catch_reversed_order(monkeypatch):
    # last-come-first within each expert: in-range, but not the canonical order
    real = planner.stable_order

    def reversed_within_expert(ids):
        ids = np.asarray(ids, dtype=np.int64)
        return np.bincount(ids)[ids] - 1 - real(ids)

    monkeypatch.setattr(planner, "stable_order", reversed_within_expert)
    with pytest.raises(AssertionError):
        _check_example(load("plan_example1.json"))
    idx, E, B = _small_case(7)
    p = planner.plan(idx, E, B)
    with pytest.raises(AssertionError):
        check_plan_invariants(idx, E, B, p.cu_seqlens, p.slot_expert, p.dest_idx)


def test_pins_catch_wrong_tbar(monkeypatch):
    monkeypatch.setattr(planner, "maxvio", lambda c, n: float(int(np.max(c)) * n) / len(c) - 1.0)
    with pytest.raises(AssertionError):
        _check_example(load("plan_example1.json"))


def test_pins_catch_unbalanced_rank(monkeypatch):
    # a plan that gives one rank a row more than S*K must fail the invariants
    real = planner.plan

    def broken(topk_idx, E, B):
        p = real(topk_idx, E, B)
        p.cu_seqlens[0, -1] += 1
        return p

    monkeypatch.setattr(planner, "plan", broken)
    idx, E, B = _small_case(3)
    p = planner.plan(idx, E, B)
    with pytest.raises(AssertionError):
        check_plan_invariants(idx, E, B, p.cu_seqlens, p.slot_expert, p.dest_idx)


# ------------------------------------------------------------ the fewest-copies planner


def _check_mincopy_example(g):
    p = planner.plan(np.array(g["topk_idx"]), g["E"], g["B"], planner="mincopy")
    assert p.expert_counts.tolist() == g["expert_counts"]
    assert abs(p.maxvio - g["maxvio_num"] / g["maxvio_den"]) < 1e-15
    assert p.keep.tolist() == g["keep"]
    assert p.cu_seqlens.tolist() == g["cu_seqlens"]
    assert p.slot_expert.tolist() == g["slot_expert"]
    assert p.dest_idx.tolist() == g["dest_idx"]
    assert p.stats.tolist() == g["stats"]
    return p


@pytest.mark.parametrize("name", ["plan_example1_mincopy.json", "plan_example2_mincopy.json",
                                  "plan_example4_tie.json"])
def test_mincopy_hand_worked_examples(name):
    g = load(name)
    p = _check_mincopy_example(g)
    check_plan_invariants(g["topk_idx"], g["E"], g["B"], p.cu_seqlens, p.slot_expert, p.dest_idx, p.src_of_row,
                          p.stats, planner="mincopy")
    assert mincopies.min_copies(p.expert_counts, g["R"], g["S"] * g["K"]) == g["min_copies"] == p.stats[0]
    if "prefix_keep" in g:
        assert planner.plan(np.array(g["topk_idx"]), g["E"], g["B"]).keep.tolist() == g["prefix_keep"]


def test_mincopy_example3_reaches_the_minimum():
    g = load("plan_example3_counts.json")
    idx = routing_from_counts(g["expert_counts"], g["R"], g["S"], g["K"])
    p = planner.plan(idx, g["E"], g["B"], planner="mincopy")
    assert [e for e in range(g["E"]) if p.over[e] > 0] == g["mincopy"]["overflow_experts"]
    assert p.slot_expert[3].tolist() == g["mincopy"]["slot_expert_rank3"]
    assert p.stats.tolist() == g["mincopy"]["stats"]
    assert p.stats[0] == g["min_copies"]
    check_plan_invariants(idx, g["E"], g["B"], p.cu_seqlens, p.slot_expert, p.dest_idx, p.src_of_row, p.stats,
                          planner="mincopy")


@pytest.mark.parametrize("seed", range(100))
def test_mincopy_invariants_and_list_simulation(seed):
    idx, E, B = _small_case(seed)
    p = planner.plan(idx, E, B, planner="mincopy")
    check_plan_invariants(idx, E, B, p.cu_seqlens, p.slot_expert, p.dest_idx, p.src_of_row, p.stats,
                          planner="mincopy")
    cu, slots, dest = list_plan(idx, E, B, planner="mincopy")
    assert np.array_equal(cu, p.cu_seqlens)
    assert np.array_equal(slots, p.slot_expert)
    assert np.array_equal(dest, p.dest_idx)
    # the overflowing experts of an overloaded rank are as few as any choice allows: no smaller set of its
    # experts holds the excess (brute force over subsets)
    from itertools import combinations
    R = idx.shape[0]
    per = E // R
    for r in range(R):
        T = p.expert_counts[r * per:(r + 1) * per]
        x = int(T.sum()) - idx.shape[1] * idx.shape[2]
        n_over = int(np.sum(p.over[r * per:(r + 1) * per] > 0))
        if x <= 0:
            assert n_over == 0
            continue
        least = min(m for m in range(1, per + 1) for c in combinations(T.tolist(), m) if sum(c) >= x)
        assert n_over == least


def test_mincopy_never_above_prefix_and_never_below_the_minimum():
    for seed in range(60):
        idx, E, B = _small_case(seed)
        R, S, K = idx.shape
        a = planner.plan(idx, E, B)
        b = planner.plan(idx, E, B, planner="mincopy")
        assert b.stats[0] <= a.stats[0]
        if R >= 2 and E // R <= 2:
            assert mincopies.min_copies(b.expert_counts, R, S * K) <= b.stats[0]


def test_slot_capped_minimum():
    # example 2 (B = 1): two copies leave one for a direct read; one copy of expert 0 fits the slot
    g = load("plan_example2.json")
    T = np.array(g["expert_counts"])
    assert mincopies.min_copies(T, g["R"], g["S"] * g["K"], slot_cap=1) == 1
    # example 3 counts (ranks 0-2 over by 2 each, rank 3 short by 6): even one slot per rank allows the
    # minimum of 3 copies, as a chain -- expert 8 sends 2 pairs to rank 1, expert 4 sends 4 to rank 0,
    # expert 0 sends 6 to rank 3 -- while no slots at all (cap 0) admit no balanced placement
    g = load("plan_example3_counts.json")
    T = np.array(g["expert_counts"])
    P = g["S"] * g["K"]
    assert mincopies.min_copies(T, g["R"], P, max_size=3, slot_cap=3) == 3
    assert mincopies.min_copies(T, g["R"], P, max_size=3, slot_cap=1) == 3
    assert mincopies.min_copies(T, g["R"], P, max_size=3, slot_cap=0) is None
    per = g["E"] // g["R"]
    assert mincopies._feasible(T, g["R"], P, [e // per for e in range(g["E"])], [(8, 1), (4, 0), (0, 3)])


def test_planner_gap_report_matches_the_stored_table():
    # the distribution quoted in the design notes: copies of both planners against the brute-force minimum
    from tests import planner_gap
    with open(planner_gap.GOLDEN) as f:
        stored = json.load(f)
    n = 60  # a prefix of the stored cases keeps the CPU suite quick; the summary covers all of them
    for seed in range(n):
        assert planner_gap.measure(seed) == stored["cases"][seed], seed
    assert planner_gap.summary(stored["cases"]) == stored["summary"]
    s = stored["summary"]
    assert s["copies_total"]["min"] <= s["copies_total"]["mincopy"] <= s["copies_total"]["prefix"]
    for r in stored["cases"]:
        assert r["lower_bound"] <= r["min"] <= r["mincopy"][0] <= r["prefix"][0]
        assert r["min_capped"] is None or r["min_capped"] >= r["min"]


def test_pins_catch_reversed_tie_order(monkeypatch):
    # equal counts broken toward the higher id: example 4 then overflows expert 1
    real = planner.keep_counts

    def higher_id_first(T, R, P, name="prefix"):
        if name != "mincopy":
            return real(T, R, P, name)
        keep, load = real(T[::-1].copy(), R, P, name)  # mirror the expert order inside every rank
        return keep[::-1].copy(), load[::-1].copy()

    monkeypatch.setattr(planner, "keep_counts", higher_id_first)
    with pytest.raises(AssertionError):
        _check_mincopy_example(load("plan_example4_tie.json"))


def test_pins_catch_smallest_first(monkeypatch):
    def smallest_first(T, R, P, name="prefix"):
        E = len(T)
        per = E // R
        keep, load = T.copy(), np.zeros(R, dtype=np.int64)
        for r in range(R):
            ex = list(range(r * per, (r + 1) * per))
            load[r] = T[ex].sum()
            x = load[r] - P
            for e in sorted(ex, key=lambda e: (T[e], e)):
                m = max(0, min(int(T[e]), x))
                keep[e] -= m
                x -= m
        return keep, load

    monkeypatch.setattr(planner, "keep_counts", smallest_first)
    with pytest.raises(AssertionError):
        _check_mincopy_example(load("plan_example1_mincopy.json"))
    idx, E, B = _small_case(9)
    p = planner.plan(idx, E, B, planner="mincopy")
    with pytest.raises(AssertionError):
        for seed in range(40):
            idx, E, B = _small_case(seed)
            p = planner.plan(idx, E, B, planner="mincopy")
            check_plan_invariants(idx, E, B, p.cu_seqlens, p.slot_expert, p.dest_idx, p.src_of_row, p.stats,
                                  planner="mincopy")
