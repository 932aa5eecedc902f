"""Benchmark of the balanced expert-parallel MoE layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
plan -> prefetch -> dispatch -> group GEMM -> combine -> wgrad -> reduce_grad,
with every input already resident in HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload large|mid|stress|tiny]
                    [--maxvio T] [--no-sweep] [--no-extras] [--no-ffn] [--no-cpu-baseline]

Default workload: R8 E256 K8 S4096 H7168 H'2048 B32 (bf16 activations and
weights, fp32 gradients; the [288, 7168, 2048] weight tensor, 262144 pairs),
routing skew calibrated to maxvio ~ 1; the sweep adds maxvio ~ 0.5, 2, 4.
value = token-expert pairs planned and dispatched per second,
N / (plan time + dispatch time), at the headline point.  The JSON also carries
group-GEMM TFLOP/s and reduce_grad GB/s, every stage's roofline (the longest
stage's as `roofline`), the backward of the data path (combine backward,
dgrad, dispatch backward) as `next_rows`, the sweep and its flatness, the other
workloads timed after the headline one (`other_workloads`: the mid sweep with
the backward workload's point, the mid gated FFN, the routing-stress
plan + dispatch), and the CPU oracle's plan + dispatch rate on a bounded sample.

    python bench.py --stats-md run_kernel_stats.csv          (rocprofv3 summary -> markdown)
    python bench.py --traffic-md fetch.csv write.csv         (counter runs -> per-stage HBM bytes)
    python bench.py --mfma-md counters.csv                   (counter run -> GEMM MFMA utilisation)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_F32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector
N_CU, SIMDS_PER_CU, TOP_CLOCK_GHZ = 256, 4, 2.4  # MI355X compute units, SIMDs per CU, peak engine clock
MFMA_FLOP_PER_INST = 32768  # one v_mfma_f32_32x32x16_bf16, the only MFMA the GEMM kernels issue
MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES")

WORKLOAD_KEYS = {"tiny": "tiny_f32", "mid": "mid_fwd", "large": "large_fwd", "stress": "plan_stress"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large", choices=sorted(WORKLOAD_KEYS))
    ap.add_argument("--maxvio", type=float, default=None, help="target maxvio of the headline point")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forward-only", action="store_true")
    ap.add_argument("--no-ffn", action="store_true", help="skip the full gated expert FFN on the mid dims")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline workload (by default the large run is followed by the mid sweep "
                         "with the backward workload's point, the mid FFN and the routing-stress workload)")
    ap.add_argument("--stats-md", metavar="CSV",
                    help="print a markdown table of the library kernels in a rocprofv3 kernel_stats.csv; no GPU")
    ap.add_argument("--traffic-md", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the per-stage HBM traffic summary of two --profile-pass counter runs "
                         "(FETCH_SIZE, WRITE_SIZE) for --workload/--maxvio; no GPU")
    ap.add_argument("--ffn-only", action="store_true",
                    help="time only the full gated expert FFN and print its object (not the bench line); with "
                         "--profile-pass, run its passes for counter runs instead")
    ap.add_argument("--ffn-stats-md", metavar="TRACE_CSV",
                    help="print per-call kernel times of an --ffn-only rocprofv3 kernel_trace.csv; no GPU")
    ap.add_argument("--ffn-traffic-md", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the per-call HBM traffic of two --ffn-only --profile-pass counter runs; no GPU")
    ap.add_argument("--mfma-md", metavar="COUNTER_CSV",
                    help="print the MFMA utilisation of the GEMM kernels from a --profile-pass counter run of "
                         + " ".join(MFMA_COUNTERS) + "; no GPU")
    ap.add_argument("--vendor-pass", action="store_true",
                    help="for counter runs: only the vendor BLAS GEMMs the GEMM stages are compared with (the "
                         "forward shape, then the weight-gradient shape, each 2 + R calls); prints no JSON")
    ap.add_argument("--vendor-mfma-md", metavar="COUNTER_CSV",
                    help="print the MFMA utilisation of the vendor GEMM kernels of a --vendor-pass counter run of "
                         + " ".join(MFMA_COUNTERS) + "; no GPU")
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
                      src_of_row=False, data_grad=backward)


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




def stage_calls(L, backward):
    if L.Hp is None:
        return [("plan", L.plan), ("dispatch", L.dispatch)]
    # prefetch needs only the plan; run before dispatch, it does not pay for the write-back of
    # dispatch's output, which the compute-bound GEMM absorbs instead
    calls = [("plan", L.plan), ("prefetch", L.prefetch), ("dispatch", L.dispatch), ("group_gemm", L.group_gemm),
             ("combine", L.combine)]
    if backward:
        calls += [("wgrad", L.wgrad), ("reduce_grad", L.reduce_grad)]
    return calls


def time_steps(L, backward, steps, warmup):
    """K whole steps between two device synchronisations (wall clock), with HIP events recorded between
    consecutive calls on the stream the kernels run on (torch's current stream), so every stage's average
    launch duration comes from the same timed region."""
    import torch
    calls = stage_calls(L, backward)
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        evs[s][0].record()
        for i, (_, f) in enumerate(calls):
            f()
            evs[s][i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = {n: sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)) / steps
              for i, (n, _) in enumerate(calls)}
    return (t1 - t0) * 1e3 / steps, stages


def next_calls(L):
    return [("combine_backward", L.combine_backward), ("dgrad", L.dgrad), ("dispatch_backward", L.dispatch_backward)]


def time_next_rows(L, steps, warmup):
    """The backward of the data path (combine backward -> dgrad -> dispatch backward) on the same
    workload: dout ~ N(0, 1) drawn once on the device, a forward pass for Yp, then K timed passes with
    HIP events between the calls, as for the step."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(7)
    L.dout.normal_(generator=g)
    L.forward()
    calls = next_calls(L)
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for s in range(steps):
        evs[s][0].record()
        for i, (_, f) in enumerate(calls):
            f()
            evs[s][i + 1].record()
    torch.cuda.synchronize()
    return {n: sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)) / steps
            for i, (n, _) in enumerate(calls)}


# Library kernel dispatches of each call of one full-FFN pass, in call order, and the stages those
# kernels belong to; labels each dispatch of an FFN-only profile with the call that launched it.
FFN_CALLS = [("plan", 4, ("plan",)), ("prefetch", 2, ("prefetch",)), ("dispatch", 1, ("dispatch",)),
             ("gemm_gate_up", 2, ("group_gemm",)), ("swiglu", 1, ("swiglu",)), ("gemm_down", 2, ("group_gemm",)),
             ("combine", 1, ("combine",)), ("combine_backward", 1, ("combine_backward",)),
             ("dgrad_down", 2, ("group_gemm", "dgrad")), ("wgrad_down", 2, ("wgrad",)),
             ("swiglu_backward", 1, ("swiglu_backward",)), ("dgrad_gate_up", 2, ("group_gemm", "dgrad")),
             ("wgrad_gate_up", 2, ("wgrad",)), ("dispatch_backward", 1, ("dispatch_backward",)),
             ("reduce_grad", 2, ("reduce_grad",))]
FFN_GEMM_FLOPS = {"gemm_gate_up": 4, "gemm_down": 2, "dgrad_down": 2, "wgrad_down": 2, "dgrad_gate_up": 4,
                  "wgrad_gate_up": 4}  # x N*H*H'
FFN_ACT_BYTES = {"swiglu": 3, "swiglu_backward": 5}  # x N*H'*b


def make_ffn(wl, seed, alpha):
    """A MoeFFN on the workload's dims with its inputs drawn, and its forward + backward call list."""
    import torch

    import load_balanced_dispatch_amd as m
    from synthetic.router import TAG_W, TAG_WD, TAG_X, normal_tensor, router_output
    R, E, B, S, K, H, Hp = wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp
    F = m.MoeFFN(R, E, B, S, K, H, Hp, backward=True)
    idx, gates = router_output(R, S, E, K, seed, alpha=alpha, zipf_s=wl.zipf_s)
    F.topk_idx.copy_(torch.as_tensor(idx))
    F.gates.copy_(torch.as_tensor(gates))
    F.X.copy_(normal_tensor((R, S, H), 1.0, "bf16", seed, TAG_X, "cuda", slices=R))
    F.W_gu_home.copy_(normal_tensor((E, H, 2 * Hp), H ** -0.5, "bf16", seed, TAG_W, "cuda", slices=E))
    F.W_down_home.copy_(normal_tensor((E, Hp, H), Hp ** -0.5, "bf16", seed, TAG_WD, "cuda", slices=E))
    F.dout.normal_(generator=torch.Generator(device="cuda").manual_seed(seed + 11))
    calls = F.forward_calls() + F.backward_calls()
    assert [n for n, _ in calls] == [c[0] for c in FFN_CALLS]
    return F, calls


def time_ffn(wl, seed, alpha, steps, warmup):
    """The full gated expert FFN (NEXT row) on the workload's dims: gate|up [E+B, H, 2H'], swiglu,
    down [E+B, H', H], forward then backward, every call bracketed by HIP events."""
    import torch

    R, E, B, S, K, H, Hp = wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp
    F, calls = make_ffn(wl, seed, alpha)
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for st in range(steps):
        evs[st][0].record()
        for i, (_, f) in enumerate(calls):
            f()
            evs[st][i + 1].record()
    torch.cuda.synchronize()
    ms = {n: sum(evs[st][i].elapsed_time(evs[st][i + 1]) for st in range(steps)) / steps
          for i, (n, _) in enumerate(calls)}
    nf = len(F.forward_calls())
    fwd = sum(v for i, v in enumerate(ms.values()) if i < nf)
    bwd = sum(v for i, v in enumerate(ms.values()) if i >= nf)
    N, b = wl.N, 2
    gemm_flops = {k: c * N * H * Hp for k, c in FFN_GEMM_FLOPS.items()}
    act_bytes = {k: c * N * Hp * b for k, c in FFN_ACT_BYTES.items()}
    traffic = load_ffn_traffic(wl)
    out = {"forward_ms": round(fwd, 4), "backward_ms": round(bwd, 4),
           "gemm_tflops": round(sum(gemm_flops.values()) / (sum(ms[k] for k in gemm_flops) * 1e-3) / 1e12, 2),
           "stages_ms": {k: round(v, 4) for k, v in ms.items()}}
    for k, fl in gemm_flops.items():
        a = fl / (ms[k] * 1e-3) / 1e12
        out[k] = {"bound": "mfma", "achieved": round(a, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic.get(k),
                  "avg_launch_ms": round(ms[k], 4)}
    for k, by in act_bytes.items():
        a = by / (ms[k] * 1e-3) / 1e9
        out[k] = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic.get(k), "avg_launch_ms": round(ms[k], 4)}
    del F
    torch.cuda.empty_cache()
    return out


def algorithmic(wl, stats, slot_expert_np, L, cu=None):
    """Algorithmic work per launch of each stage: bytes for the bandwidth-bound stages (every input byte
    read once, every output byte written once), flops for the two GEMMs plus the least HBM bytes they can
    move (each operand read once, each output written once; wgrad's float32 gradient read and written)."""
    import numpy as np
    b = 4 if wl.dtype == "f32" else 2
    N, T, H = wl.N, wl.R * wl.S, wl.H
    out = {"plan": 8 * N, "dispatch": T * H * b + N * H * b + 4 * N}
    if wl.Hp is not None:
        Hp = wl.Hp
        G = wl.E + wl.B
        cu = (L.cu_seqlens.cpu().numpy() if cu is None else np.asarray(cu)).reshape(wl.R, G + 1)
        rows = np.diff(cu, axis=1)  # [R, E+B] rows per (rank, group)
        home_used = int((rows[:, :wl.E].sum(axis=0) > 0).sum())
        slots_used = int((rows[:, wl.E:] > 0).sum())
        out["prefetch"] = 2 * H * Hp * b * int(stats[1])
        out["group_gemm"] = 2 * N * H * Hp
        out["group_gemm_min_bytes"] = N * H * b + (home_used + slots_used) * H * Hp * b + N * Hp * b
        out["combine"] = N * Hp * b + T * Hp * 4 + 8 * N
        used = slot_expert_np[slot_expert_np >= 0]
        out["reduce_grad"] = 4 * H * Hp * (2 * len(np.unique(used)) + 2 * len(used))
        out["wgrad"] = 2 * N * H * Hp
        out["wgrad_min_bytes"] = N * (H + Hp) * b + 8 * H * Hp * (home_used + slots_used)
        # backward of the data path
        out["combine_backward"] = T * Hp * 4 + 2 * N * Hp * b + 12 * N
        out["dgrad"] = 2 * N * H * Hp
        out["dgrad_min_bytes"] = N * Hp * b + (home_used + slots_used) * H * Hp * b + N * H * b
        out["dispatch_backward"] = N * H * b + T * H * 4 + 4 * N
    return out


# library kernels of each stage, matched on "base<template args>" names, and the source file that holds them
STAGE_KERNELS = {
    "plan": r"^plan_(count|scan|solve|emit)$",
    "dispatch": r"^dispatch_rows<",
    "prefetch": r"^prefetch_slots<",
    "group_gemm": r"^(ggemm_tiles$|ggemm_bf16<false\b|ggemm_generic<.*false>)",
    "combine": r"^combine_(vec|scalar)<[^>]*\btrue\b",
    "wgrad": r"^wgrad_(schedule|bf16|generic)",
    "reduce_grad": r"^reduce_grad_(kernel|scalar)",
    "combine_backward": r"^combine_bwd_",
    "dgrad": r"^(ggemm_bf16<true\b|ggemm_generic<.*true>)",
    "dispatch_backward": r"^combine_(vec|scalar)<[^>]*\bfalse\b",
    "swiglu": r"^swiglu_(vec|scalar)<",
    "swiglu_backward": r"^swiglu_bwd_",
}
STAGE_SOURCE = {"plan": "plan.hip", "dispatch": "move.hip", "prefetch": "move.hip", "group_gemm": "ggemm.hip",
                "combine": "move.hip", "wgrad": "wgrad.hip", "reduce_grad": "move.hip",
                "combine_backward": "move.hip", "dgrad": "ggemm.hip", "dispatch_backward": "move.hip",
                "swiglu": "act.hip", "swiglu_backward": "act.hip"}
GEMM_STAGES = ("group_gemm", "wgrad", "dgrad")
CSRC = os.path.join(ROOT, "load_balanced_dispatch_amd", "csrc")


def kernel_base(name):
    """'base<template args>' of a demangled kernel name as rocprofv3 prints it (args kept: they tell
    instantiations such as the forward and dgrad GEMMs apart)."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    cut = len(n)
    for i, ch in enumerate(n):
        if ch in "<(":
            cut = i
            break
    base = n[:cut].rsplit("::", 1)[-1]
    if cut < len(n) and n[cut] == "<":
        depth, j = 0, cut
        while j < len(n):
            depth += (n[j] == "<") - (n[j] == ">")
            j += 1
            if depth == 0:
                break
        base += n[cut:j]
    return base


def stage_of(base):
    for st, pat in STAGE_KERNELS.items():
        if re.search(pat, base):
            return st
    return None


def sources_digest(stage):
    """Hash of the source a stage's kernels are compiled from (its .hip file and every csrc header)."""
    return sources_digest_files([STAGE_SOURCE[stage]])


def sources_digest_files(srcs):
    """Hash of the given csrc .hip files and every csrc header."""
    files = [os.path.join(CSRC, f) for f in srcs] + sorted(glob.glob(os.path.join(CSRC, "*.h")))
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(wl):
    return os.path.join(ROOT, "profiles", f"traffic_{wl.name}.md")


def load_traffic(wl, target):
    """HBM bytes per launch of each stage from the committed counter summary for this workload, or None for
    a stage whose kernel source has changed since the counters were taken."""
    path = traffic_path(wl)
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return {}
    rec = json.loads(m.group(1))
    if rec.get("workload") != wl.name or rec.get("maxvio_target") != target:
        return {}
    return {st: (v["bytes_per_launch"] if v.get("sources") == sources_digest(st) else None)
            for st, v in rec["stages"].items()}


def stage_roofline(name, alg, ms, traffic, f32, mfma=None):
    """Roofline entry of one stage.  A bandwidth stage is bound by HBM: achieved = its algorithmic bytes per
    launch over the launch's duration.  A GEMM stage is bound by the larger of its two floors: its flops at
    the MFMA peak (fp32 vector peak for float32), or its least bytes (each operand read once, each output
    written once; wgrad's float32 gradient read and written) at the HBM peak; `achieved` is then the flop
    rate or the least-bytes rate accordingly, and both floors are given."""
    gemm = name in GEMM_STAGES
    t = traffic.get(name)
    secs = ms * 1e-3
    if gemm:
        cpeak = MFMA_F32_VECTOR_TFLOPS if f32 else MFMA_BF16_PEAK_TFLOPS
        least = alg.get(name + "_min_bytes")
        floor_c = alg[name] / (cpeak * 1e12)
        floor_m = (least or 0) / (HBM_PEAK_GBS * 1e9)
        tflops = alg[name] / secs / 1e12
        if floor_m > floor_c:
            bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
            achieved = least / secs / 1e9
            per = f"{least:.4g} B (least bytes; {alg[name]:.4g} FLOP = 2*N*H*H')"
        else:
            bound, unit, peak = ("alu" if f32 else "mfma"), "TFLOP/s", cpeak
            achieved = tflops
            per = f"{alg[name]:.4g} FLOP (2*N*H*H')"
    else:
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
        achieved = alg[name] / secs / 1e9
        per = f"{alg[name]:.4g} B"
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": t, "avg_launch_ms": round(ms, 4),
         "algorithmic_per_launch": per}
    if gemm:
        r["tflops"] = round(tflops, 2)
        r["frac_of_mfma_peak"] = round(tflops / cpeak, 4)
        r["floors_ms"] = {"compute": round(floor_c * 1e3, 4), "hbm": round(floor_m * 1e3, 4)}
        r["least_bytes_per_launch"] = least
    least_b = least if gemm else alg[name]
    if t and least_b:
        r["traffic_over_least_bytes"] = round(t / least_b, 3)
    if gemm and not f32:
        r["mfma_util"] = (mfma or {}).get(name)  # from the committed counter summary, None once stale
    return r


def stats_markdown(csv_path):
    """Markdown table of the library kernels in a rocprofv3 --stats kernel summary (csv)."""
    rows = list(csv.DictReader(open(csv_path)))
    out = ["| kernel | stage | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        base = kernel_base(r["Name"])
        st = stage_of(base)
        if st is None:
            continue
        out.append(f"| `{base}` | {st} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    return "\n".join(out)


def traffic_markdown(fetch_csv, write_csv, wl, target):
    """Per-stage HBM bytes per launch from a FETCH_SIZE and a WRITE_SIZE counter run of --profile-pass,
    each scaled by what the same counter reads for the closing 1 GiB device copy."""
    def read(path, counter):
        per, calib = {}, None
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v, disp = float(r["Counter_Value"]), int(r["Dispatch_Id"])
            base = kernel_base(r["Kernel_Name"])
            if stage_of(base):
                per.setdefault(base, []).append(v)
            elif "copyBuffer" in r["Kernel_Name"] and (calib is None or disp > calib[0]):
                calib = (disp, v)  # the last device copy is the 1 GiB calibration copy
        return {k: sum(v) / len(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()}, calib[1]
    fetch, nf, cf = read(fetch_csv, "FETCH_SIZE")
    write, nw, cw = read(write_csv, "WRITE_SIZE")
    fs, ws = 1024 * 1024 / cf, 1024 * 1024 / cw  # KiB the 1 GiB copy should read / write, over the reading
    stages = {}
    lines = ["| stage | kernels | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |",
             "|---|---|---|---|---|---|"]
    for st in STAGE_KERNELS:
        ks = sorted(k for k in fetch if stage_of(k) == st and k in write)
        if not ks:
            continue
        f = sum(fetch[k] for k in ks)
        w = sum(write[k] for k in ks)
        b = f * 1024 * fs + w * 1024 * ws
        stages[st] = {"kernels": ks, "fetch_kib": round(f, 1), "write_kib": round(w, 1),
                      "bytes_per_launch": round(b), "dispatches": min(nf[k] for k in ks),
                      "sources": sources_digest(st)}
        lines.append(f"| {st} | {', '.join('`' + k + '`' for k in ks)} | {stages[st]['dispatches']} | "
                     f"{f:.1f} | {w:.1f} | {b:.4g} |")
    rec = {"workload": wl.name, "maxvio_target": target,
           "calibration": {"copy_bytes": 1 << 30, "fetch_kib": cf, "write_kib": cw, "fetch_scale": round(fs, 4),
                           "write_scale": round(ws, 4)},
           "stages": stages}
    return "\n".join(lines), rec


def mfma_markdown(counter_csv, wl, target):
    """MFMA utilisation of each GEMM kernel from a --profile-pass counter run, averaged over its dispatches.

    SQ_VALU_MFMA_BUSY_CYCLES sums the cycles each SIMD's matrix pipe is busy (32 per 32x32x16 bf16
    instruction) and SQ_BUSY_CU_CYCLES the cycles each CU has work, so their ratio over 4 SIMDs is the
    fraction of the kernel's own cycles the matrix pipes compute, and CU-busy cycles per CU over the
    dispatch's duration give the engine clock it ran at.  The busy cycles over 1024 SIMDs at the 2.4 GHz
    peak clock for that duration give its fraction of the nominal peak."""
    per = {}
    for r in csv.DictReader(open(counter_csv)):
        base = kernel_base(r["Kernel_Name"])
        if stage_of(base) not in GEMM_STAGES:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {"base": base})
        d["dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    kernels = {}
    for d in per.values():
        if any(c not in d for c in MFMA_COUNTERS) or d["SQ_INSTS_MFMA"] <= 0:
            continue  # the tile and schedule kernels beside the GEMMs issue no MFMA
        kernels.setdefault(d["base"], []).append(d)
    lines = ["| kernel | stage | dispatches | avg us (counted run) | MFMA instructions | engine clock GHz | "
             "MFMA busy / CU busy | issued TFLOP/s | of 2.5 PF nominal |",
             "|---|---|---|---|---|---|---|---|---|"]
    rec = {"workload": wl.name, "maxvio_target": target, "counters": list(MFMA_COUNTERS), "kernels": {}}
    for base in sorted(kernels):
        ds = kernels[base]
        avg = {k: sum(d[k] for d in ds) / len(ds) for k in MFMA_COUNTERS + ("dur_s",)}
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS_PER_CU * avg["SQ_BUSY_CU_CYCLES"])
        clock = avg["SQ_BUSY_CU_CYCLES"] / N_CU / avg["dur_s"] / 1e9
        issued = avg["SQ_INSTS_MFMA"] * MFMA_FLOP_PER_INST / avg["dur_s"] / 1e12
        nominal = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_CU * SIMDS_PER_CU * TOP_CLOCK_GHZ * 1e9 * avg["dur_s"])
        st = stage_of(base)
        rec["kernels"][base] = {"stage": st, "dispatches": len(ds), "avg_us": round(avg["dur_s"] * 1e6, 2),
                                "mfma_insts": round(avg["SQ_INSTS_MFMA"]),
                                "engine_clock_ghz": round(clock, 3), "mfma_busy_of_cu_busy": round(busy, 4),
                                "issued_tflops": round(issued, 1), "of_nominal_peak": round(nominal, 4),
                                "sources": sources_digest(st)}
        lines.append(f"| `{base}` | {st} | {len(ds)} | {avg['dur_s'] * 1e6:.1f} | {avg['SQ_INSTS_MFMA']:.4g} | "
                     f"{clock:.2f} | {busy:.3f} | {issued:.0f} | {nominal:.3f} |")
    return "\n".join(lines), rec


def load_mfma(wl, target):
    """Per GEMM stage, the MFMA utilisation of profiles/mfma_util_<workload>.md, or None for a stage whose
    kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"mfma_util_{wl.name}.md")
    if not os.path.exists(path):
        return {}
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return {}
    rec = json.loads(m.group(1))
    if rec.get("workload") != wl.name or rec.get("maxvio_target") != target:
        return {}
    out = {}
    for k in rec["kernels"].values():
        ok = k["sources"] == sources_digest(k["stage"])
        out[k["stage"]] = ({"mfma_busy_of_cu_busy": k["mfma_busy_of_cu_busy"],
                            "engine_clock_ghz": k["engine_clock_ghz"]} if ok else None)
    return out


def label_ffn_dispatches(names):
    """Call of FFN_CALLS that launched each library dispatch of an FFN-only run, given the dispatches'
    demangled names in launch order; every pass must launch the same kernel sequence."""
    bases = [kernel_base(n) for n in names]
    lib = [i for i, b in enumerate(bases) if stage_of(b)]
    labels = [c for c, n, _ in FFN_CALLS for _ in range(n)]
    allowed = [a for _, n, a in FFN_CALLS for _ in range(n)]
    per = len(labels)
    if not lib or len(lib) % per:
        raise SystemExit(f"{len(lib)} library dispatches: not a whole number of {per}-dispatch FFN passes")
    out = {}
    for j, i in enumerate(lib):
        p = j % per
        if stage_of(bases[i]) not in allowed[p] or bases[i] != bases[lib[p]]:
            raise SystemExit(f"dispatch {j} ({bases[i]}) does not fit call {labels[p]} of an FFN pass")
        out[i] = (labels[p], bases[i], p)
    return out


def ffn_stats_markdown(trace_csv):
    """Markdown table of an FFN-only rocprofv3 --kernel-trace: per (call, kernel), calls and durations."""
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    lab = label_ffn_dispatches([r["Kernel_Name"] for r in rows])
    per = {}
    for i, (c, b, _) in lab.items():
        per.setdefault((c, b), []).append((int(rows[i]["End_Timestamp"]) - int(rows[i]["Start_Timestamp"])) / 1e3)
    order = {c: k for k, (c, _, _) in enumerate(FFN_CALLS)}
    out = ["| call | kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for (c, b), v in sorted(per.items(), key=lambda kv: (order[kv[0][0]], kv[0][1])):
        out.append(f"| {c} | `{b}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(out)


def ffn_traffic_markdown(fetch_csv, write_csv, wl):
    """Per-call HBM bytes per launch of an FFN-only --profile-pass, scaled like traffic_markdown."""
    def read(path, counter):
        rows = sorted((r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter),
                      key=lambda r: int(r["Dispatch_Id"]))
        lab = label_ffn_dispatches([r["Kernel_Name"] for r in rows])
        per, kern, calib = {}, {}, None
        for i, r in enumerate(rows):
            if i in lab:  # average each position of the pass over passes, then sum a call's positions
                c, b, p = lab[i]
                per.setdefault(c, {}).setdefault(p, []).append(float(r["Counter_Value"]))
                kern.setdefault(c, set()).add(b)
            elif "copyBuffer" in r["Kernel_Name"]:
                calib = float(r["Counter_Value"])  # the last device copy is the 1 GiB calibration copy
        return {c: sum(sum(v) / len(v) for v in d.values()) for c, d in per.items()}, kern, calib
    fetch, kern, cf = read(fetch_csv, "FETCH_SIZE")
    write, _, cw = read(write_csv, "WRITE_SIZE")
    fs, ws = 1024 * 1024 / cf, 1024 * 1024 / cw
    calls = {}
    lines = ["| call | kernels | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |",
             "|---|---|---|---|---|"]
    for c, _, stages in FFN_CALLS:
        f, w, ks = fetch[c], write[c], sorted(kern[c])
        b = f * 1024 * fs + w * 1024 * ws
        srcs = sorted({STAGE_SOURCE[st] for st in stages})
        calls[c] = {"kernels": ks, "fetch_kib": round(f, 1), "write_kib": round(w, 1),
                    "bytes_per_launch": round(b), "sources": sources_digest_files(srcs)}
        lines.append(f"| {c} | {', '.join('`' + k + '`' for k in ks)} | {f:.1f} | {w:.1f} | {b:.4g} |")
    rec = {"workload": wl.name, "calibration": {"copy_bytes": 1 << 30, "fetch_kib": cf, "write_kib": cw,
                                                "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
           "calls": calls}
    return "\n".join(lines), rec


def load_ffn_traffic(wl):
    """HBM bytes per launch of each FFN call from profiles/traffic_<workload>_ffn.md, for the calls whose
    kernels' sources still hash as they did when the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}_ffn.md")
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    rec = json.loads(text[text.index("```json") + 7:text.rindex("```")])
    out = {}
    for c, _, stages in FFN_CALLS:
        r = rec["calls"].get(c)
        if r and r["sources"] == sources_digest_files(sorted({STAGE_SOURCE[st] for st in stages})):
            out[c] = r["bytes_per_launch"]
    return out


def cpu_baseline(wl, seed, alpha, tokens_per_rank=512, min_seconds=10.0, max_reps=60):
    """The oracle as it stands, on the metric's first term: plan + dispatch of a bounded sample of the
    workload (the same routing recipe and skew with S' tokens per rank, the full E, B and H), repeated
    until about `min_seconds` of oracle work; pairs/s = pairs planned and dispatched / oracle time.  The
    oracle's planner and permute are plain single-threaded numpy."""
    import numpy as np

    from oracle import layer as olayer
    from oracle import planner as oplanner
    from synthetic.router import router_output
    sw = wl.with_dims(S=min(wl.S, tokens_per_rank))
    idx, _ = router_output(sw.R, sw.S, sw.E, sw.K, seed, alpha=alpha, zipf_s=sw.zipf_s)
    X = np.random.default_rng(seed).standard_normal((sw.R, sw.S, sw.H))  # drawn before the clock starts
    spent, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or spent < min_seconds):
        t0 = time.perf_counter()
        p = oplanner.plan(idx, sw.E, sw.B)
        Xp = olayer.dispatch(X, p.dest_idx)
        spent += time.perf_counter() - t0
        reps += 1
        del Xp
    return {"value": sw.N * reps / spent, "unit": "pairs/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle plan + dispatch of the {wl.name} recipe with S={sw.S} tokens per rank ({sw.N} "
                      f"pairs, full E={sw.E}, B={sw.B}, H={sw.H}, float64 rows), {reps} passes, {spent:.1f} s; "
                      f"single-threaded numpy"}


def hot_rank_factor(idx, wl):
    """What an unbalanced EP would wait for: the most loaded rank's pairs (the pairs routed to its
    E/R home experts) over the P = S*K pairs every rank holds after balancing."""
    import numpy as np
    counts = np.bincount(np.asarray(idx).reshape(-1), minlength=wl.E)
    per_rank = counts.reshape(wl.R, wl.E // wl.R).sum(axis=1)
    return float(per_rank.max()) / float(wl.S * wl.K)


def runtime_copy_gbs(reps=5):
    """HBM rate of the HIP runtime's own device-to-device copy (torch's copy_ of 1 GiB: 1 GiB read,
    1 GiB written), timed with events on the current stream.  A reference point, not a ceiling: a
    one-shot copy kernel with one 16-byte vector per thread measured about 6.5 TB/s on this GPU."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


def library_copy_gbs(reps=5):
    """HBM rate of this library's own copy kernel, the prefetch, used as a plain copy: eight [8192, 8192]
    bf16 experts (1 GiB) into the eight slots of one rank, timed with events after one untimed pass; the
    2 GiB moved per pass is far larger than the last-level cache.  The ceiling the prefetch stage could
    reach in isolation, beside its rate inside the step."""
    import torch

    import load_balanced_dispatch_amd as m
    E, H = 8, 8192
    d = m.make_dims(1, E, E, 1, 1)
    W = torch.ones((E, H, H), dtype=torch.bfloat16, device="cuda")
    Ws = torch.empty((1, E, H, H), dtype=torch.bfloat16, device="cuda")
    slots = torch.arange(E, dtype=torch.int32, device="cuda").reshape(1, E)
    m.moonep_prefetch(d, H, H, W, slots, Ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        m.moonep_prefetch(d, H, H, W, slots, Ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del W, Ws
    torch.cuda.empty_cache()
    return 2 * E * H * H * 2 / (ms * 1e-3) / 1e9


def _evict(buf):
    """Writes a 1 GiB buffer, twice the size of the last-level cache, so that what follows starts cold."""
    buf.fill_(7)


def cold_copy_gbs(total_bytes, reps=5):
    """The HIP runtime's device copy moving `total_bytes` (half read, half written), each pass timed alone
    with events after the caches are evicted: the same-size cold reference of a bandwidth stage."""
    import torch
    half = max(256, (int(total_bytes) // 2 + 255) // 256 * 256)
    src = torch.ones(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ev = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst.copy_(src)
    ms = 0.0
    for _ in range(reps):
        _evict(ev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms += a.elapsed_time(b) / reps
    del src, dst, ev
    torch.cuda.empty_cache()
    return 2 * half / (ms * 1e-3) / 1e9


def cold_prefetch_gbs(L, nbytes, reps=5):
    """The prefetch stage on the current plan with cold weights: each call timed alone with events after
    the caches are evicted (inside the step the weights it reads may still sit in the last-level cache)."""
    import torch
    ev = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    L.plan()
    L.prefetch()
    ms = 0.0
    for _ in range(reps):
        _evict(ev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        L.prefetch()
        b.record()
        torch.cuda.synchronize()
        ms += a.elapsed_time(b) / reps
    del ev
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def vendor_gemm_tflops(wl, reps=5):
    """The vendor BLAS (hipBLASLt via torch.matmul, bf16) on the group GEMM's FLOPs: R dense GEMMs of
    [P, H] x [H, H'] (forward shape) and of [H, P] x [P, H'] (the weight-gradient shape), all
    operands contiguous 2-D tensors, timed with events.  Context for the MFMA fraction: the same work
    with one weight per P = S*K rows, an easier reuse pattern than the ragged groups."""
    import torch
    R = wl.R
    g = torch.Generator(device="cuda").manual_seed(1)
    out = {}
    for name, m, k, n in vendor_shapes(wl):
        a = torch.randn((m, k), device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn((k, n), device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(2):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps * R):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = 2.0 * R * m * k * n / (ms * 1e-3) / 1e12
        del a, b
    torch.cuda.empty_cache()
    return out


def vendor_shapes(wl):
    """(name, m, k, n) of the dense GEMMs vendor_gemm_tflops times, in the order it runs them."""
    P, H, Hp = wl.S * wl.K, wl.H, wl.Hp
    return (("fwd", P, H, Hp), ("wgrad", H, P, Hp))


def vendor_pass(wl):
    """The vendor GEMMs of vendor_gemm_tflops, 2 + R calls of each shape in turn, for a counter run."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(1)
    for _, m, k, n in vendor_shapes(wl):
        a = torch.randn((m, k), device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn((k, n), device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(2 + wl.R):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        del a, b
    torch.cuda.empty_cache()


def vendor_mfma_markdown(counter_csv, wl):
    """MFMA utilisation of the vendor GEMM kernels of a --vendor-pass counter run, per call.

    Every dispatch that issues MFMAs is a vendor GEMM call; the first 2 + R belong to the forward shape and
    the next 2 + R to the weight-gradient shape (vendor_pass runs them in that order).  The instruction the
    library picks need not be this path's 32x32x16, so the rate is taken from the busy cycles (1024 flop per
    SIMD and busy cycle at the dense bf16 rate) and checked against 2*m*k*n per call."""
    per = {}
    for r in csv.DictReader(open(counter_csv)):
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d["dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    calls = [per[i] for i in sorted(per) if per[i].get("SQ_VALU_MFMA_BUSY_CYCLES", 0) > 0
             and all(c in per[i] for c in MFMA_COUNTERS)]
    n_each = 2 + wl.R
    lines = ["| shape (m x k x n) | call | kernel | us | engine clock GHz | MFMA busy / CU busy | TFLOP/s (busy cycles) "
             "| TFLOP/s (2mkn) |", "|---|---|---|---|---|---|---|---|"]
    rec = {"workload": wl.name, "counters": list(MFMA_COUNTERS), "shapes": {}}
    for si, (name, m, k, n) in enumerate(vendor_shapes(wl)):
        rows = calls[si * n_each:(si + 1) * n_each]
        out = []
        for ci, d in enumerate(rows):
            busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS_PER_CU * d["SQ_BUSY_CU_CYCLES"])
            clock = d["SQ_BUSY_CU_CYCLES"] / N_CU / d["dur_s"] / 1e9
            tf_busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] * 1024 / d["dur_s"] / 1e12
            tf = 2.0 * m * k * n / d["dur_s"] / 1e12
            kname = d["name"].split("(")[0][:48]
            lines.append(f"| {name} {m}x{k}x{n} | {ci} | `{kname}` | {d['dur_s'] * 1e6:.1f} | {clock:.2f} | "
                         f"{busy:.3f} | {tf_busy:.0f} | {tf:.0f} |")
            out.append({"us": round(d["dur_s"] * 1e6, 1), "engine_clock_ghz": round(clock, 3),
                        "mfma_busy_of_cu_busy": round(busy, 4), "tflops": round(tf, 1)})
        rec["shapes"][name] = {"m": m, "k": k, "n": n, "calls": out}
    return "\n".join(lines), rec


def calibration_copy():
    """A plain copy kernel moving 1 GiB in and 1 GiB out, whose counters scale the traffic readings."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


SWEEPS = {"mid": (1.0, [0.0, 1.0, 2.0, 3.0]), "large": (1.0, [0.5, 1.0, 2.0, 4.0])}
FORWARD_STAGES = ("plan", "dispatch", "prefetch", "group_gemm", "combine")


def run_points(wl, L, backward, points, head_target, steps, warmup, seed, alpha_of):
    """Times the step at each maxvio target (the headline point with `steps` steps, the others with half)."""
    import torch

    from synthetic.router import measured_maxvio
    results = {}
    for tgt in points:
        alpha = alpha_of(wl, tgt)
        idx, _ = load_inputs(L, wl, seed, alpha)
        ms, stages = time_steps(L, backward, steps if tgt == head_target else max(5, steps // 2), warmup)
        torch.cuda.synchronize()
        stats = L.stats.cpu().numpy()
        slots = L.slot_expert.cpu().numpy()
        results[tgt] = dict(alpha=alpha, maxvio=float(L.maxvio.item()), ms=ms, stages=stages,
                            stats=stats.tolist(), slots=slots, maxvio_host=measured_maxvio(idx, wl.E),
                            hot_rank=hot_rank_factor(idx, wl), cu=L.cu_seqlens.cpu().numpy())
        log(f"{wl.name} maxvio target {tgt}: measured {results[tgt]['maxvio']:.3f}, {ms:.3f} ms/step, "
            f"stages {stages}")
    return results


def sweep_summary(wl, L, results, points):
    """Per sweep point: stage times, forward time, copies, each stage's roofline fraction at that point
    (prefetch and reduce_grad bytes follow its copies); flatness of every point against the lowest-maxvio one."""
    sweep = []
    for tgt in points:
        r = results[tgt]
        fwd = sum(r["stages"].get(n, 0.0) for n in FORWARD_STAGES)
        alg_p = algorithmic(wl, r["stats"], r["slots"], L, cu=r["cu"])
        frac_p = {n: stage_roofline(n, alg_p, ms_n, {}, wl.dtype == "f32")["frac"]
                  for n, ms_n in r["stages"].items() if alg_p.get(n)}
        sweep.append({"maxvio_target": tgt, "maxvio": round(r["maxvio"], 4), "ms_per_step": round(r["ms"], 4),
                      "forward_ms": round(fwd, 4), "copies_slotted_direct": r["stats"][:3],
                      "hot_rank_factor": round(r["hot_rank"], 4),
                      "plan_dispatch_pairs_per_s": round(wl.N / ((r["stages"]["plan"] + r["stages"]["dispatch"]) * 1e-3)),
                      "stages_ms": {k: round(v, 4) for k, v in r["stages"].items()},
                      "roofline_frac": frac_p})
    sweep.sort(key=lambda x: (x["maxvio_target"] is None, x["maxvio_target"]))
    flat = None
    if len(sweep) > 1:  # every point against the lowest-maxvio point: within +-10% is flat
        f0, s0 = sweep[0]["forward_ms"], sweep[0]["ms_per_step"]
        fr = [round(x["forward_ms"] / f0 - 1, 4) for x in sweep]
        sr = [round(x["ms_per_step"] / s0 - 1, 4) for x in sweep]
        flat = {"reference_maxvio": sweep[0]["maxvio"], "forward_rel": fr, "step_rel": sr,
                "forward_within_10pct": all(abs(v) <= 0.10 for v in fr),
                "step_within_10pct": all(abs(v) <= 0.10 for v in sr)}
    return sweep, flat


def point_rooflines(wl, L, r, traffic=None, mfma=None):
    alg = algorithmic(wl, r["stats"], r["slots"], L, cu=r["cu"])
    return alg, {n: stage_roofline(n, alg, r["stages"][n], traffic or {}, wl.dtype == "f32", mfma)
                 for n in r["stages"]}


def extra_workloads(args, alpha_of, no_ffn):
    """The other workloads of the benchmark, each timed the same way after the headline one (its buffers
    freed first): the mid sweep (maxvio ~ 0, 1, 3) together with the backward workload's point (mid dims,
    maxvio ~ 2: wgrad and reduce_grad), the full gated FFN on the mid dims, and the routing-stress workload
    (plan + dispatch)."""
    import torch

    from synthetic import WORKLOADS
    out = {}
    wl = WORKLOADS["mid_fwd"]
    head, pts = SWEEPS["mid"]
    log(f"extra workload: {wl.description}")
    L = make_layer(wl, True)
    res = run_points(wl, L, True, [head] + [t for t in pts if t != head], head, args.steps, args.warmup, args.seed,
                     alpha_of)
    sweep, flat = sweep_summary(wl, L, res, [head] + [t for t in pts if t != head])
    _, rl1 = point_rooflines(wl, L, res[head], load_traffic(wl, head), load_mfma(wl, head))
    h = res[head]["stages"]
    out["mid_fwd"] = {
        "workload": wl.description, "maxvio_target": head, "maxvio": round(res[head]["maxvio"], 4),
        "plan_dispatch_pairs_per_s": round(wl.N / ((h["plan"] + h["dispatch"]) * 1e-3)),
        "group_gemm_tflops": rl1["group_gemm"]["tflops"], "rooflines": rl1, "sweep": [x for x in sweep
                                                                                    if x["maxvio_target"] != 2.0],
        "sweep_flatness": sweep_summary(wl, L, res, [t for t in pts if t != 2.0])[1]}
    if not args.no_extras:
        # the mid prefetch moves few, small copies whose home weights may still be in the last-level cache
        # in the step: each sweep point's prefetch alone with cold caches, beside its in-step rate
        cold = {}
        for tgt in [head] + [t for t in pts if t != head]:
            nbytes = 2 * wl.H * wl.Hp * 2 * int(res[tgt]["stats"][1])
            if nbytes:
                load_inputs(L, wl, args.seed, res[tgt]["alpha"])
                cold[str(tgt)] = round(cold_prefetch_gbs(L, nbytes), 1)
        out["mid_fwd"]["prefetch_cold_GBs"] = cold
    wb = WORKLOADS["mid_bwd"]
    _, rl2 = point_rooflines(wb, L, res[2.0])
    out["mid_bwd"] = {"workload": wb.description, "maxvio_target": 2.0, "maxvio": round(res[2.0]["maxvio"], 4),
                      "copies_slotted_direct": res[2.0]["stats"][:3],
                      "wgrad": rl2["wgrad"], "reduce_grad": rl2["reduce_grad"]}
    out["mid_sweep_with_backward_point"] = {"sweep": sweep, "sweep_flatness": flat}
    del L
    torch.cuda.empty_cache()
    if not no_ffn:
        log("full gated expert FFN (forward + backward) on the mid dims")
        out["ffn_mid"] = time_ffn(wl, args.seed, alpha_of(wl, head), max(3, args.steps // 4), 2)
        out["ffn_mid"]["workload"] = (f"gate|up [E+B, {wl.H}, {2 * wl.Hp}], swiglu, down [E+B, {wl.Hp}, "
                                      f"{wl.H}] on the mid routing at maxvio ~ {head}")
    ws = WORKLOADS["plan_stress"]
    log(f"extra workload: {ws.description}")
    L = make_layer(ws, False)
    res = run_points(ws, L, False, [None], None, args.steps, args.warmup, args.seed, alpha_of)
    r = res[None]
    _, rls = point_rooflines(ws, L, r)
    out["plan_stress"] = {"workload": ws.description, "maxvio": round(r["maxvio"], 4),
                          "copies_slotted_direct": r["stats"][:3], "hot_rank_factor": round(r["hot_rank"], 4),
                          "plan_dispatch_pairs_per_s": round(ws.N / ((r["stages"]["plan"] + r["stages"]["dispatch"])
                                                                     * 1e-3)),
                          "plan_ms": round(r["stages"]["plan"], 4), "dispatch": rls["dispatch"]}
    del L
    torch.cuda.empty_cache()
    return out


PLANNER_POINTS = (("tiny_f32", (None,)), ("mid_fwd", (0.0, 1.0, 3.0)), ("large_fwd", (0.5, 1.0, 2.0, 4.0)),
                  ("mid_bwd", (2.0,)), ("plan_stress", (None,)))


def planner_table(args, alpha_of, reps=10):
    """Both planners on every workload's routing: copies (slotted, direct reads), the prefetch and reduce_grad
    bytes those copies cost (2*H*H'*b per slotted copy; 4*H*H'*(2 per expert with copies + 2 per copy)), and
    the plan's own time (HIP events around `reps` back-to-back plans, after 2 untimed)."""
    import numpy as np
    import torch

    import load_balanced_dispatch_amd as m
    from synthetic import WORKLOADS
    from synthetic.router import router_output
    out = {}
    for name, points in PLANNER_POINTS:
        wl = WORKLOADS[name]
        d = m.make_dims(wl.R, wl.E, wl.B, wl.S, wl.K)
        dev = dict(device="cuda")
        bufs = dict(counts=torch.empty(wl.E, dtype=torch.int32, **dev), mv=torch.empty(1, dtype=torch.float64, **dev),
                    cu=torch.empty((wl.R, wl.E + wl.B + 1), dtype=torch.int32, **dev),
                    slots=torch.empty((wl.R, wl.B), dtype=torch.int32, **dev) if wl.B else None,
                    dest=torch.empty((wl.R, wl.S, wl.K), dtype=torch.int32, **dev),
                    stats=torch.empty(4, dtype=torch.int32, **dev))
        ws = torch.empty(m.moonep_plan_workspace_bytes(d), dtype=torch.uint8, **dev)
        b = 4 if wl.dtype == "f32" else 2
        rows = []
        for tgt in points:
            idx, _ = router_output(wl.R, wl.S, wl.E, wl.K, args.seed, alpha=alpha_of(wl, tgt), zipf_s=wl.zipf_s)
            topk = torch.as_tensor(idx).cuda()
            row = {"maxvio_target": tgt}
            for planner in ("prefix", "mincopy"):
                def run():
                    m.moonep_plan_ex(d, planner, topk, bufs["counts"], bufs["mv"], bufs["cu"], bufs["slots"],
                                     bufs["dest"], None, bufs["stats"], ws)
                for _ in range(2):
                    run()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    run()
                e1.record()
                torch.cuda.synchronize()
                stats = bufs["stats"].cpu().numpy()
                slots = bufs["slots"].cpu().numpy() if wl.B else np.zeros((wl.R, 0), dtype=np.int32)
                used = slots[slots >= 0]
                r = {"copies_slotted_direct": stats[:3].tolist(), "plan_ms": round(e0.elapsed_time(e1) / reps, 4)}
                if wl.Hp is not None:
                    hh = wl.H * wl.Hp
                    r["prefetch_bytes"] = 2 * hh * b * int(stats[1])
                    r["reduce_grad_bytes"] = 4 * hh * (2 * len(np.unique(used)) + 2 * len(used))
                row[planner] = r
                row["maxvio"] = round(float(bufs["mv"].item()), 4)
            rows.append(row)
        out[name] = rows
        del bufs, ws
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; more than one GPU is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    from synthetic import WORKLOADS

    wl = WORKLOADS[WORKLOAD_KEYS[args.workload]]
    backward = wl.Hp is not None and not args.forward_only
    if args.workload in SWEEPS:
        head_target, sweep_targets = SWEEPS[args.workload]
        if args.maxvio is not None:
            head_target = args.maxvio
    else:
        head_target, sweep_targets = None, []
    if args.stats_md:
        print(stats_markdown(args.stats_md))
        return
    if args.ffn_stats_md:
        print(ffn_stats_markdown(args.ffn_stats_md))
        return
    if args.mfma_md:
        table, rec = mfma_markdown(args.mfma_md, wl, head_target)
        print(table)
        print()
        print("```json")
        print(json.dumps(rec, indent=1))
        print("```")
        return
    if args.vendor_mfma_md:
        table, rec = vendor_mfma_markdown(args.vendor_mfma_md, wl)
        print(table)
        print()
        print("```json")
        print(json.dumps(rec, indent=1))
        print("```")
        return
    if args.ffn_traffic_md or args.traffic_md:
        if args.ffn_traffic_md:
            table, rec = ffn_traffic_markdown(args.ffn_traffic_md[0], args.ffn_traffic_md[1], wl)
        else:
            table, rec = traffic_markdown(args.traffic_md[0], args.traffic_md[1], wl, head_target)
        print(table)
        print()
        print("```json")
        print(json.dumps(rec, indent=1))
        print("```")
        return

    import torch

    from synthetic.calibrate import alpha_for

    def alpha_of(w, target):
        if w.zipf_s is not None:
            return 0.0
        if target is None:
            return w.alpha or 0.0
        key_wl = WORKLOADS["mid_bwd"] if (w.name == "mid_fwd" and target == 2.0) else w
        return alpha_for(key_wl, args.seed, target)

    if args.ffn_only:
        if wl.Hp is None:
            raise SystemExit("--ffn-only needs a workload with H'")
        if args.profile_pass:
            F, calls = make_ffn(wl, args.seed, alpha_of(wl, head_target))
            for _ in range(1 + args.steps):
                for _, f in calls:
                    f()
            torch.cuda.synchronize()
            calibration_copy()
            log("profile pass done: FFN passes, then a 1 GiB copy")
        else:
            print(json.dumps({"ffn": time_ffn(wl, args.seed, alpha_of(wl, head_target), args.steps, args.warmup)}))
        return
    if args.vendor_pass:
        if wl.Hp is None:
            raise SystemExit("--vendor-pass needs a workload with H'")
        vendor_pass(wl)
        log("vendor pass done:", [s[0] for s in vendor_shapes(wl)])
        return
    log(f"workload {wl.description}; building buffers")
    L = make_layer(wl, backward)
    if args.profile_pass:
        load_inputs(L, wl, args.seed, alpha_of(wl, head_target))
        if backward:
            L.dout.normal_()
        for _ in range(1 + args.steps):
            for _, f in stage_calls(L, backward) + (next_calls(L) if backward else []):
                f()
        torch.cuda.synchronize()
        calibration_copy()
        log("profile pass done: stages", [n for n, _ in stage_calls(L, backward)], "then a 1 GiB copy")
        return
    points = [head_target] + ([t for t in sweep_targets if t != head_target] if not args.no_sweep else [])
    results = run_points(wl, L, backward, points, head_target, args.steps, args.warmup, args.seed, alpha_of)

    h = results[head_target]
    traffic = load_traffic(wl, head_target)
    mfma = load_mfma(wl, head_target)
    alg, rooflines = point_rooflines(wl, L, h, traffic, mfma)
    st = h["stages"]
    value = wl.N / ((st["plan"] + st["dispatch"]) * 1e-3)
    comp = {"plan_dispatch_pairs_per_s": value, "plan_ms": st["plan"],
            "dispatch_GBs": alg["dispatch"] / (st["dispatch"] * 1e-3) / 1e9}
    if wl.Hp is not None:
        comp["group_gemm_tflops"] = alg["group_gemm"] / (st["group_gemm"] * 1e-3) / 1e12
        comp["combine_GBs"] = alg["combine"] / (st["combine"] * 1e-3) / 1e9
        comp["prefetch_GBs"] = alg["prefetch"] / (st["prefetch"] * 1e-3) / 1e9 if alg["prefetch"] else None
        comp["forward_ms"] = sum(st[n] for n in FORWARD_STAGES)
        if backward:
            comp["wgrad_tflops"] = alg["wgrad"] / (st["wgrad"] * 1e-3) / 1e12
            comp["reduce_grad_GBs"] = (alg["reduce_grad"] / (st["reduce_grad"] * 1e-3) / 1e9
                                       if alg["reduce_grad"] else None)
    next_rows = None
    if backward:
        load_inputs(L, wl, args.seed, h["alpha"])  # the headline routing again (the sweep moved it)
        nx = time_next_rows(L, args.steps, args.warmup)
        log(f"backward of the data path: {nx}")
        next_rows = {n: stage_roofline(n, alg, nx[n], traffic, wl.dtype == "f32", mfma) for n in nx}
    dominant = max(st, key=lambda n: st[n])
    roofline = dict(rooflines[dominant], stage=dominant)
    sweep, flat = sweep_summary(wl, L, results, points)
    sweep_mincopy = None
    if args.workload in SWEEPS and not args.no_sweep and not args.no_extras:
        log("the same sweep with the fewest-copies planner")
        L.planner = "mincopy"
        res_mc = run_points(wl, L, backward, points, None, max(5, args.steps // 2), args.warmup, args.seed, alpha_of)
        sw_mc, flat_mc = sweep_summary(wl, L, res_mc, points)
        sweep_mincopy = {"sweep": sw_mc, "sweep_flatness": flat_mc}
        L.planner = "prefix"
    vendor = vendor_gemm_tflops(wl) if (wl.Hp is not None and wl.dtype == "bf16") else None
    cold = None
    if not args.no_extras:
        log("cold-cache references: the prefetch with evicted caches, and same-size cold copies")
        load_inputs(L, wl, args.seed, h["alpha"])
        cold = {"prefetch_cold_GBs": (round(cold_prefetch_gbs(L, alg["prefetch"]), 1) if alg.get("prefetch")
                                      else None)}
        for n, entry in rooflines.items():
            if n in ("prefetch", "dispatch", "combine", "reduce_grad") and "tflops" not in entry and alg.get(n):
                ref = cold_copy_gbs(alg[n])
                cold[f"{n}_same_bytes_cold_copy_GBs"] = round(ref, 1)
                entry["frac_of_cold_copy_same_bytes"] = round(entry["achieved"] / ref, 4)
                if roofline.get("stage") == n:
                    roofline["frac_of_cold_copy_same_bytes"] = entry["frac_of_cold_copy_same_bytes"]
    del L
    torch.cuda.empty_cache()

    extras = None
    planners = None
    if args.workload == "large" and not args.no_extras:
        extras = extra_workloads(args, alpha_of, args.no_ffn)
        log("both planners on every workload's routing")
        planners = planner_table(args, alpha_of)
        comp["stress_plan_dispatch_pairs_per_s"] = extras["plan_stress"]["plan_dispatch_pairs_per_s"]
        comp["stress_dispatch_GBs"] = extras["plan_stress"]["dispatch"]["achieved"]
        comp["mid_plan_dispatch_pairs_per_s"] = extras["mid_fwd"]["plan_dispatch_pairs_per_s"]
        comp["mid_group_gemm_tflops"] = extras["mid_fwd"]["group_gemm_tflops"]
        comp["backward_cfg_wgrad_tflops"] = extras["mid_bwd"]["wgrad"]["tflops"]
        comp["backward_cfg_reduce_grad_GBs"] = extras["mid_bwd"]["reduce_grad"]["achieved"]

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle's plan + dispatch on a bounded sample")
        cpu = cpu_baseline(wl, args.seed, h["alpha"])

    log("timing the runtime's 1 GiB device copy and the library's copy kernel (reference rates)")
    copy_gbs = runtime_copy_gbs()
    lib_copy_gbs = library_copy_gbs()
    if vendor:
        for n, key in (("group_gemm", "fwd"), ("dgrad", "fwd"), ("wgrad", "wgrad")):
            for entry in [rooflines.get(n), (next_rows or {}).get(n)] + ([roofline] if roofline.get("stage") == n else []):
                if entry:
                    entry["frac_of_vendor_gemm"] = round(entry["tflops"] / vendor[key], 4)
    for entry in list(rooflines.values()) + [roofline] + list((next_rows or {}).values()):
        if entry.get("unit") == "GB/s" and entry.get("bound") == "hbm" and "tflops" not in entry:
            entry["frac_of_runtime_copy"] = round(entry["achieved"] / copy_gbs, 4)
    line = {
        "metric": "token-expert pairs/s planned+dispatched; group-GEMM TFLOP/s; reduce_grad GB/s",
        "value": value,
        "unit": "pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(h["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded router skew, N(0,1) activations, N(0,1/H) weights)",
        "config": {"workload": f"{wl.name}: {wl.description}; step = "
                               + ("forward + backward" if backward else "forward")
                               + "; value = pairs / (plan + dispatch time)",
                   "R": wl.R, "E": wl.E, "B": wl.B, "S": wl.S, "K": wl.K, "H": wl.H, "Hp": wl.Hp,
                   "pairs_per_step": wl.N, "maxvio_target": head_target, "maxvio": round(h["maxvio"], 4),
                   "copies_slotted_direct": h["stats"][:3]},
        "components": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in comp.items()},
        "roofline": roofline,
        "rooflines": rooflines,
        "next_rows": next_rows,
        "cpu_baseline": cpu,
        "reference_rates": {"runtime_copy_GBs": round(copy_gbs, 1), "library_copy_GBs": round(lib_copy_gbs, 1),
                            "vendor_gemm_fwd_TFLOPs": round(vendor["fwd"], 1) if vendor else None,
                            "vendor_gemm_wgrad_TFLOPs": round(vendor["wgrad"], 1) if vendor else None,
                            "cold": cold,
                            "note": "the HIP runtime's device copy of 1 GiB (read + write), HIP events; a GB/s "
                                    "stage's frac_of_runtime_copy is its rate over this. library_copy: this "
                                    "library's prefetch kernel copying 1 GiB (eight [8192, 8192] bf16 experts) "
                                    "outside the step. cold: the headline prefetch timed alone after a 1 GiB "
                                    "write evicts the caches, and for each GB/s stage the runtime's copy of "
                                    "the stage's algorithmic bytes (half read, half written) timed the same "
                                    "way; a stage's frac_of_cold_copy_same_bytes is its in-step rate over "
                                    "that. vendor_gemm_*: "
                                    "hipBLASLt (torch.matmul, bf16) on the same FLOPs as R dense GEMMs, "
                                    "[P,H]x[H,H'] and [H,P]x[P,H']; a GEMM stage's frac_of_vendor_gemm is its "
                                    "flop rate over that."},
        "sweep": sweep,
        "sweep_flatness": flat,
        "sweep_mincopy_planner": sweep_mincopy,
        "planners": planners,
        "other_workloads": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
