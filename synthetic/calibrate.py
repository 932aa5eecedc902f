"""Finds the skew alpha that puts a workload's measured maxvio near each sweep target.

Writes ``alpha_table.json`` beside this file.  Uses only the router generator
(no layer arithmetic).  Run:  python -m synthetic.calibrate [--seeds 0]
"""
from __future__ import annotations

import argparse
import json
import os

from .configs import WORKLOADS
from .router import measured_maxvio, router_output

TABLE = os.path.join(os.path.dirname(__file__), "alpha_table.json")


def maxvio_at(wl, seed, alpha):
    idx, _ = router_output(wl.R, wl.S, wl.E, wl.K, seed, alpha=alpha, zipf_s=wl.zipf_s)
    return measured_maxvio(idx, wl.E)


def calibrate(wl, seed, target, tol=0.05, iters=30):
    if target == 0.0:
        return 0.0, maxvio_at(wl, seed, 0.0)
    lo, hi = 0.0, 0.5
    while maxvio_at(wl, seed, hi) < target:
        hi *= 2.0
        if hi > 64:
            raise RuntimeError("target maxvio out of reach")
    best = (hi, maxvio_at(wl, seed, hi))
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        m = maxvio_at(wl, seed, mid)
        if abs(m - target) < abs(best[1] - target):
            best = (mid, m)
        if abs(m - target) <= tol:
            return mid, m
        if m < target:
            lo = mid
        else:
            hi = mid
    return best


def load_table():
    if os.path.exists(TABLE):
        with open(TABLE) as f:
            return json.load(f)
    return {}


def alpha_for(wl, seed, target):
    """Calibrated alpha for (workload, seed, target); bisects when the table has no entry."""
    key = f"{wl.name}/{seed}/{target}"
    tab = load_table()
    if key in tab:
        return tab[key]["alpha"]
    return calibrate(wl, seed, target)[0]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seeds", type=int, nargs="*", default=[0])
    args = ap.parse_args()
    tab = load_table()
    for name, wl in WORKLOADS.items():
        for seed in args.seeds:
            for tgt in wl.maxvio_targets:
                a, m = calibrate(wl, seed, tgt)
                tab[f"{name}/{seed}/{tgt}"] = {"alpha": a, "maxvio": m}
                print(name, seed, tgt, a, m, flush=True)
    with open(TABLE, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
