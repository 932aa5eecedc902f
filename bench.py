"""Benchmark of the balanced expert-parallel MoE layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
plan -> dispatch -> prefetch -> group GEMM -> combine -> wgrad -> reduce_grad,
with every input already resident in HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload mid|large|stress|tiny]
                    [--maxvio T] [--no-sweep] [--no-cpu-baseline]

Default workload: R8 E64 K6 S4096 H2048 H'1408 B8 (bf16 activations and
weights, fp32 gradients), routing skew calibrated to maxvio ~ 1; the sweep adds
maxvio ~ 0, 2, 3.  value = token-expert pairs per second through the whole
step; the JSON also carries plan+dispatch pairs/s, group-GEMM TFLOP/s and
reduce_grad GB/s, the dominant kernel's roofline and the CPU oracle's rate on
a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16

WORKLOAD_KEYS = {"tiny": "tiny_f32", "mid": "mid_fwd", "large": "large_fwd", "stress": "plan_stress"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mid", choices=sorted(WORKLOAD_KEYS))
    ap.add_argument("--maxvio", type=float, default=None, help="target maxvio of the headline point")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forward-only", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for counter runs: 1 warm-up + --steps steps of the whole path, then one plain 1 GiB "
                         "device copy whose FETCH_SIZE/WRITE_SIZE calibrate the traffic counters; prints no JSON")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def make_layer(wl, backward):
    import torch

    import load_balanced_dispatch_amd as m
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    return m.MoeLayer(wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp, dtype=dt, device="cuda", backward=backward,
                      src_of_row=False)


def load_inputs(L, wl, seed, alpha):
    """Seeded synthetic inputs, drawn on the device, copied into the layer's static buffers."""
    import torch

    from synthetic.router import TAG_DY, TAG_W, TAG_X, normal_tensor, router_output
    idx, gates = router_output(wl.R, wl.S, wl.E, wl.K, seed, alpha=alpha, zipf_s=wl.zipf_s)
    L.topk_idx.copy_(torch.as_tensor(idx))
    L.gates.copy_(torch.as_tensor(gates))
    L.X.copy_(normal_tensor((wl.R, wl.S, wl.H), 1.0, wl.dtype, seed, TAG_X, "cuda", slices=wl.R))
    if wl.Hp is not None:
        L.W_home.copy_(normal_tensor((wl.E, wl.H, wl.Hp), wl.H ** -0.5, wl.dtype, seed, TAG_W, "cuda", slices=wl.E))
        if hasattr(L, "dY"):
            L.dY.copy_(normal_tensor((wl.N, wl.Hp), 1.0, wl.dtype, seed, TAG_DY, "cuda", slices=wl.R))
            L.dW_home.zero_()
            L.dW_slots.zero_()
    torch.cuda.synchronize()
    return idx, gates


STAGES = ("plan", "dispatch", "prefetch", "group_gemm", "combine", "wgrad", "reduce_grad")


def stage_calls(L, backward):
    calls = [("plan", L.plan), ("dispatch", L.dispatch)]
    if L.Hp is not None:
        calls += [("prefetch", L.prefetch), ("group_gemm", L.group_gemm), ("combine", L.combine)]
        if backward:
            calls += [("wgrad", L.wgrad), ("reduce_grad", L.reduce_grad)]
    return calls


def time_steps(L, backward, steps, warmup):
    """Headline timing: K whole steps between two device synchronisations, with HIP events around the
    dominant kernel's call on the same (current) stream."""
    import torch
    calls = stage_calls(L, backward)
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for name, f in calls:
            if name == "group_gemm":
                ev[s][0].record()
                f()
                ev[s][1].record()
            else:
                f()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gemm_ms = [a.elapsed_time(b) for a, b in ev] if L.Hp is not None else []
    return (t1 - t0) * 1e3 / steps, (sum(gemm_ms) / len(gemm_ms) if gemm_ms else None)


def time_stages(L, backward, reps=10):
    """Per-stage breakdown: events between consecutive calls of each step, averaged."""
    import torch
    calls = stage_calls(L, backward)
    acc = {n: 0.0 for n, _ in calls}
    for _ in range(2):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    for _ in range(reps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        evs[0].record()
        for i, (_, f) in enumerate(calls):
            f()
            evs[i + 1].record()
        torch.cuda.synchronize()
        for i, (n, _) in enumerate(calls):
            acc[n] += evs[i].elapsed_time(evs[i + 1])
    return {n: v / reps for n, v in acc.items()}


def algorithmic(wl, stats, slot_expert_np):
    """Algorithmic bytes / flops per launch of each stage (documented with the roofline model)."""
    import numpy as np
    b = 4 if wl.dtype == "f32" else 2
    N, T, H = wl.N, wl.R * wl.S, wl.H
    out = {
        "plan_bytes": 8 * N,
        "dispatch_bytes": T * H * b + N * H * b + 4 * N,
    }
    if wl.Hp is not None:
        Hp = wl.Hp
        copies_slotted = int(stats[1])
        out["prefetch_bytes"] = 2 * H * Hp * b * copies_slotted
        out["gemm_flops"] = 2 * N * H * Hp
        out["combine_bytes"] = N * Hp * b + T * Hp * 4 + 8 * N
        used = slot_expert_np[slot_expert_np >= 0]
        experts_with_copies = len(np.unique(used))
        out["reduce_grad_bytes"] = 4 * H * Hp * (2 * experts_with_copies + 2 * len(used))
        out["wgrad_flops"] = 2 * N * H * Hp
    return out


def cpu_baseline(wl, seed, alpha, tokens_per_rank):
    """The oracle as it stands, on a bounded sample: the same routing recipe with S' tokens per rank and
    the workload's full E, B, H, H'; pairs/s = sampled pairs / oracle time of the whole step."""
    import numpy as np

    from oracle import layer as olayer
    from oracle import planner as oplanner
    from synthetic.router import router_output
    sw = wl.with_dims(S=tokens_per_rank)
    idx, gates = router_output(sw.R, sw.S, sw.E, sw.K, seed, alpha=alpha, zipf_s=sw.zipf_s)
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((sw.R, sw.S, sw.H))
    if sw.Hp is not None:  # inputs are drawn before the clock starts: only oracle work is timed
        W = rng.standard_normal((sw.E, sw.H, sw.Hp)) / np.sqrt(sw.H)
        dY = rng.standard_normal((sw.N, sw.Hp))
    t0 = time.perf_counter()
    p = oplanner.plan(idx, sw.E, sw.B)
    Xp = olayer.dispatch(X, p.dest_idx)
    if sw.Hp is not None:
        Ws = olayer.prefetch(W, p.slot_expert)
        Yp = olayer.group_gemm(Xp, W, Ws, p.cu_seqlens, sw.P)
        olayer.combine(Yp, p.dest_idx, gates)
        dWh = np.zeros_like(W)
        dWs = np.zeros((sw.R, sw.B, sw.H, sw.Hp))
        olayer.wgrad(Xp, dY, p.cu_seqlens, sw.P, dWh, dWs)
        olayer.reduce_grad(p.slot_expert, dWh, dWs)
    t = time.perf_counter() - t0
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": sw.N / t, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole step (plan, dispatch, prefetch, group GEMM, combine, wgrad, reduce_grad) on the same "
                      f"recipe with S={sw.S} tokens per rank ({sw.N} pairs), full E/B/H/H', float64; {t:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from synthetic import WORKLOADS
    from synthetic.calibrate import alpha_for
    from synthetic.router import measured_maxvio

    wl = WORKLOADS[WORKLOAD_KEYS[args.workload]]
    backward = wl.Hp is not None and not args.forward_only
    if args.workload == "mid":
        head_target = 1.0 if args.maxvio is None else args.maxvio
        sweep_targets = [0.0, 1.0, 2.0, 3.0]
    elif args.workload == "large":
        head_target = 1.0 if args.maxvio is None else args.maxvio
        sweep_targets = [0.5, 1.0, 2.0, 4.0]
    else:
        head_target = None
        sweep_targets = []

    def alpha_of(target):
        if wl.zipf_s is not None:
            return 0.0
        if target is None:
            return wl.alpha or 0.0
        key_wl = WORKLOADS["mid_bwd"] if (args.workload == "mid" and target == 2.0) else wl
        return alpha_for(key_wl, args.seed, target)

    log(f"workload {wl.description}; building buffers")
    L = make_layer(wl, backward)
    if args.profile_pass:
        load_inputs(L, wl, args.seed, alpha_of(head_target))
        for _ in range(1 + args.steps):
            for _, f in stage_calls(L, backward):
                f()
        torch.cuda.synchronize()
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)  # a plain copy kernel moving 1 GiB in and 1 GiB out
        torch.cuda.synchronize()
        log("profile pass done: stages", [n for n, _ in stage_calls(L, backward)], "then a 1 GiB copy")
        return
    results = {}
    points = [head_target] + ([t for t in sweep_targets if t != head_target] if not args.no_sweep else [])
    for tgt in points:
        alpha = alpha_of(tgt)
        idx, _ = load_inputs(L, wl, args.seed, alpha)
        ms, gemm_ms = time_steps(L, backward, args.steps if tgt == head_target else max(5, args.steps // 2),
                                 args.warmup)
        stages = time_stages(L, backward)
        torch.cuda.synchronize()
        stats = L.stats.cpu().numpy()
        slots = L.slot_expert.cpu().numpy()
        results[tgt] = dict(alpha=alpha, maxvio=float(L.maxvio.item()), ms=ms, gemm_ms=gemm_ms, stages=stages,
                            stats=stats.tolist(), slots=slots, maxvio_host=measured_maxvio(idx, wl.E))
        log(f"maxvio target {tgt}: measured {results[tgt]['maxvio']:.3f}, {ms:.3f} ms/step, stages {stages}")

    h = results[head_target]
    alg = algorithmic(wl, h["stats"], h["slots"])
    st = h["stages"]
    comp = {"plan_dispatch_pairs_per_s": wl.N / ((st["plan"] + st["dispatch"]) * 1e-3),
            "plan_ms": st["plan"], "dispatch_GBs": alg["dispatch_bytes"] / (st["dispatch"] * 1e-3) / 1e9}
    roofline = None
    if wl.Hp is not None:
        comp["group_gemm_tflops"] = alg["gemm_flops"] / (h["gemm_ms"] * 1e-3) / 1e12
        comp["combine_GBs"] = alg["combine_bytes"] / (st["combine"] * 1e-3) / 1e9
        comp["prefetch_GBs"] = alg["prefetch_bytes"] / (st["prefetch"] * 1e-3) / 1e9 if alg["prefetch_bytes"] else None
        if backward:
            comp["wgrad_tflops"] = alg["wgrad_flops"] / (st["wgrad"] * 1e-3) / 1e12
            comp["reduce_grad_GBs"] = (alg["reduce_grad_bytes"] / (st["reduce_grad"] * 1e-3) / 1e9
                                       if alg["reduce_grad_bytes"] else None)
        ach = comp["group_gemm_tflops"]
        roofline = {"kernel": "ggemm_bf16 (moonep_group_gemm)", "bound": "mfma", "achieved": round(ach, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": None, "avg_launch_ms": round(h["gemm_ms"], 4),
                    "algorithmic_per_launch": f"{alg['gemm_flops']:.4g} FLOP (2*N*H*H')"}
    else:
        ach = comp["dispatch_GBs"]
        roofline = {"kernel": "dispatch_rows (moonep_dispatch)", "bound": "hbm", "achieved": round(ach, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, args.seed, h["alpha"], tokens_per_rank=max(1, min(wl.S, 640)))

    sweep = []
    for tgt in points:
        r = results[tgt]
        fwd = sum(r["stages"].get(n, 0.0) for n in ("plan", "dispatch", "prefetch", "group_gemm", "combine"))
        sweep.append({"maxvio_target": tgt, "maxvio": round(r["maxvio"], 4), "ms_per_step": round(r["ms"], 4),
                      "forward_ms": round(fwd, 4), "copies_slotted_direct": r["stats"][:3],
                      "stages_ms": {k: round(v, 4) for k, v in r["stages"].items()}})
    sweep.sort(key=lambda x: (x["maxvio_target"] is None, x["maxvio_target"]))
    line = {
        "metric": "token-expert pairs/s planned+dispatched; group-GEMM TFLOP/s; reduce_grad GB/s",
        "value": wl.N / (h["ms"] * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(h["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded router skew, N(0,1) activations, N(0,1/H) weights)",
        "config": {"workload": f"{wl.name}: {wl.description}; step = "
                               + ("forward + backward" if backward else "forward"),
                   "R": wl.R, "E": wl.E, "B": wl.B, "S": wl.S, "K": wl.K, "H": wl.H, "Hp": wl.Hp,
                   "pairs_per_step": wl.N, "maxvio_target": head_target, "maxvio": round(h["maxvio"], 4),
                   "copies_slotted_direct": h["stats"][:3]},
        "components": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in comp.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
