"""Copies made by the two planners against the brute-force minimum, over seeded tiny routings (CPU only).

For each case (R in 2..4 ranks, 1..2 home experts per rank, K in 1..3, S in 1..5 tokens per rank, a
random skew, training slot budget B = E/R) it records the redundant copies and direct reads of the
home-first prefix planner and of the fewest-copies planner, the smallest number of copies any balanced
placement needs (uncapped, and with every rank receiving at most B experts), and the lower bound
max(#overloaded ranks, #underloaded ranks).  Everything comes from oracle/; the routings from the
test-only generator.

    python -m tests.planner_gap            print the summary
    python -m tests.planner_gap --write    also store it in tests/golden/planner_gap.json
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

from oracle import mincopies, planner
from tests.plan_checks import random_routing

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "planner_gap.json")
N_CASES = 300


def case(seed):
    rng = np.random.default_rng(5000 + seed)
    R = int(rng.integers(2, 5))
    per = int(rng.integers(1, 3))
    E = R * per
    K = int(rng.integers(1, min(E, 3) + 1))
    S = int(rng.integers(1, 6))
    idx = random_routing(rng, R, S, K, E, float(rng.uniform(0.5, 3)))
    return idx, E, per  # B = per: the training budget E/R


def measure(seed):
    idx, E, B = case(seed)
    R, S, K = idx.shape
    P = S * K
    out = {}
    for name in planner.PLANNERS:
        p = planner.plan(idx, E, B, planner=name)
        out[name] = [int(p.stats[0]), int(p.stats[2])]
    T = planner.histogram(idx, E)
    top = max(out["prefix"][0], out["mincopy"][0])
    out["min"] = mincopies.min_copies(T, R, P)
    out["min_capped"] = mincopies.min_copies(T, R, P, max_size=top, slot_cap=B)
    out["lower_bound"] = mincopies.lower_bound(T, R, P)
    return out


def summary(rows):
    def hist(vals):
        h = {}
        for v in vals:
            h[str(v)] = h.get(str(v), 0) + 1
        return dict(sorted(h.items(), key=lambda kv: int(kv[0])))

    s = {"cases": len(rows),
         "copies_total": {"prefix": sum(r["prefix"][0] for r in rows), "mincopy": sum(r["mincopy"][0] for r in rows),
                          "min": sum(r["min"] for r in rows)},
         "direct_reads_total": {"prefix": sum(r["prefix"][1] for r in rows),
                                "mincopy": sum(r["mincopy"][1] for r in rows)},
         "gap_to_min_histogram": {"prefix": hist(r["prefix"][0] - r["min"] for r in rows),
                                  "mincopy": hist(r["mincopy"][0] - r["min"] for r in rows)},
         "cases_at_min": {"prefix": sum(r["prefix"][0] == r["min"] for r in rows),
                          "mincopy": sum(r["mincopy"][0] == r["min"] for r in rows)},
         "capped_min_exists": sum(r["min_capped"] is not None for r in rows),
         "mincopy_at_capped_min_without_direct_reads": sum(
             r["min_capped"] is not None and r["mincopy"][1] == 0 and r["mincopy"][0] == r["min_capped"] for r in rows)}
    return s


def table(n=N_CASES):
    rows = [measure(seed) for seed in range(n)]
    return {"source": "python -m tests.planner_gap --write (oracle/planner.py, oracle/mincopies.py)",
            "summary": summary(rows), "cases": rows}


if __name__ == "__main__":
    t = table()
    print(json.dumps(t["summary"], indent=1))
    if "--write" in sys.argv[1:]:
        with open(GOLDEN, "w") as f:
            json.dump(t, f, indent=0)
            f.write("\n")
