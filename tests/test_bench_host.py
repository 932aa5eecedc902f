"""Host logic of bench.py, CPU only: the one-GPU refusal, kernel-name parsing and stage mapping, the
per-call labelling of full-FFN profiles, and the counter scaling of the traffic summaries, on small
synthetic rocprofv3 CSVs."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# demangled names as rocprofv3 prints them, one per library kernel an FFN pass launches
NAMES = {
    "plan_count": "void moonep::(anonymous namespace)::plan_count(moonep_dims, int const*, int*)",
    "plan_scan": "void moonep::(anonymous namespace)::plan_scan(int*)",
    "plan_solve": "void moonep::(anonymous namespace)::plan_solve(moonep_dims, int*)",
    "plan_emit": "void moonep::(anonymous namespace)::plan_emit(moonep_dims, int const*, int*)",
    "dispatch": "void moonep::(anonymous namespace)::dispatch_rows<unsigned int __vector(4), false>(long, int, void const*)",
    "prefetch": "void moonep::(anonymous namespace)::prefetch_slots<unsigned int __vector(4)>(long)",
    "tiles": "moonep::(anonymous namespace)::ggemm_tiles(moonep_dims, int const*, int*)",
    "fwd": "void moonep::fwd::(anonymous namespace)::ggemm_bf16<false>(moonep::fwd::GemmArgs)",
    "dgrad": "void moonep::fwd::(anonymous namespace)::ggemm_bf16<true>(moonep::fwd::GemmArgs)",
    "fwd_tails": "void moonep::(anonymous namespace)::fwd::ggemm_bf16<false, true>(unsigned short const*, int, int)",
    "dgrad_full": "void moonep::(anonymous namespace)::fwd::ggemm_bf16<true, false>(unsigned short const*, int, int)",
    "swiglu": "void moonep::(anonymous namespace)::swiglu_vec<unsigned short>(unsigned short const*, long, int)",
    "swiglu_bwd": "void moonep::(anonymous namespace)::swiglu_bwd_vec<unsigned short>(unsigned short const*)",
    "combine": "void moonep::(anonymous namespace)::combine_vec<8, 2, true, unsigned int, 6>(long)",
    "combine_bwd": "void moonep::(anonymous namespace)::combine_bwd_vec<8, 2, 4>(long)",
    "dispatch_bwd": "void moonep::(anonymous namespace)::combine_vec<8, 2, false, unsigned int, 6>(long)",
    "wsched": "void moonep::wg::(anonymous namespace)::wgrad_schedule(moonep_dims, int*)",
    "wgrad": "void moonep::wg::(anonymous namespace)::wgrad_bf16(moonep::wg::WArgs)",
    "reduce": "void moonep::(anonymous namespace)::reduce_grad_kernel(long, float*)",
}
PASS = ["plan_count", "plan_scan", "plan_solve", "plan_emit", "prefetch", "prefetch", "dispatch",
        "tiles", "fwd", "swiglu", "tiles", "fwd", "combine", "combine_bwd", "tiles", "dgrad", "wsched", "wgrad",
        "swiglu_bwd", "tiles", "dgrad", "wsched", "wgrad", "dispatch_bwd", "reduce", "reduce"]
TORCH = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>(int, float)"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


@pytest.mark.parametrize("key,base,stage", [
    ("fwd", "ggemm_bf16<false>", "group_gemm"), ("dgrad", "ggemm_bf16<true>", "dgrad"),
    ("fwd_tails", "ggemm_bf16<false, true>", "group_gemm"), ("dgrad_full", "ggemm_bf16<true, false>", "dgrad"),
    ("tiles", "ggemm_tiles", "group_gemm"), ("combine", "combine_vec<8, 2, true, unsigned int, 6>", "combine"),
    ("dispatch_bwd", "combine_vec<8, 2, false, unsigned int, 6>", "dispatch_backward"), ("wgrad", "wgrad_bf16", "wgrad"),
    ("dispatch", "dispatch_rows<unsigned int __vector(4), false>", "dispatch"), ("swiglu_bwd",
     "swiglu_bwd_vec<unsigned short>", "swiglu_backward"), ("plan_emit", "plan_emit", "plan"),
])
def test_kernel_base_and_stage(key, base, stage):
    assert bench.kernel_base(NAMES[key]) == base
    assert bench.stage_of(base) == stage


def test_torch_kernels_have_no_stage():
    assert bench.stage_of(bench.kernel_base(TORCH)) is None


@pytest.mark.parametrize("base,stage", [
    ("combine_vec<4, 4, true, long, 0>", "combine"), ("combine_scalar<unsigned short, true>", "combine"),
    ("combine_vec<8, 2, false, long, 0>", "dispatch_backward"), ("combine_scalar<float, false>", "dispatch_backward"),
    ("combine_bwd_vec<8, 2, 4>", "combine_backward"), ("combine_bwd_scalar<float>", "combine_backward"),
])
def test_combine_instances_map_to_their_stage(base, stage):
    assert bench.stage_of(base) == stage


def test_ffn_call_table_matches_the_pass():
    assert sum(n for _, n, _ in bench.FFN_CALLS) == len(PASS)


def test_ffn_labels_follow_the_pass_and_skip_foreign_kernels():
    names = [TORCH] + [NAMES[k] for k in PASS] + [TORCH, TORCH] + [NAMES[k] for k in PASS]
    lab = bench.label_ffn_dispatches(names)
    assert len(lab) == 2 * len(PASS) and 0 not in lab
    calls = [lab[i][0] for i in sorted(lab)]
    # the two forward GEMMs and the two dgrads are told apart by their place in the pass
    fwd = [c for i, c in zip(sorted(lab), calls) if lab[i][1] == "ggemm_bf16<false>"]
    assert fwd == ["gemm_gate_up", "gemm_down"] * 2
    dg = [c for i, c in zip(sorted(lab), calls) if lab[i][1] == "ggemm_bf16<true>"]
    assert dg == ["dgrad_down", "dgrad_gate_up"] * 2
    assert calls[:4] == ["plan"] * 4 and calls[-2:] == ["reduce_grad"] * 2


def test_ffn_labels_reject_a_broken_pass():
    bad = [NAMES[k] for k in PASS]
    bad[9], bad[13] = bad[13], bad[9]  # swiglu where combine backward should be
    with pytest.raises(SystemExit):
        bench.label_ffn_dispatches([NAMES[k] for k in PASS] + bad)
    with pytest.raises(SystemExit):
        bench.label_ffn_dispatches([NAMES[k] for k in PASS[:-1]])


def _trace(path, names, dur):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for n, d in zip(names, dur):
            w.writerow({"Kernel_Name": n, "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d + 10


def test_ffn_stats_table_averages_per_call(tmp_path):
    names = [NAMES[k] for k in PASS] * 3
    dur = []
    for p in range(3):
        for i, k in enumerate(PASS):
            gemm = k == "fwd"
            first = PASS.index("fwd") == i
            dur.append((2000 if first else 1000) * (p + 1) if gemm else 100)
    path = str(tmp_path / "trace.csv")
    _trace(path, names, dur)
    md = bench.ffn_stats_markdown(path)
    rows = {tuple(c.strip(" `") for c in line.split("|")[1:3]): line for line in md.splitlines()[2:]}
    assert "| 3 | 4.00 | 2.00 | 6.00 |" in rows[("gemm_gate_up", "ggemm_bf16<false>")]
    assert "| 3 | 2.00 | 1.00 | 3.00 |" in rows[("gemm_down", "ggemm_bf16<false>")]
    assert "| 6 | 0.10 |" in rows[("prefetch", "prefetch_slots<unsigned int __vector(4)>")]


def _counters(path, counter, names, values):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (n, v) in enumerate(zip(names, values)):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": n, "Counter_Name": counter, "Counter_Value": v})


def test_ffn_traffic_sums_a_calls_dispatches_and_scales_by_the_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    names = [NAMES[k] for k in PASS] * 2 + [copy]
    # fetch counter reads half of the copy's 1 GiB, write counter all of it
    fv = [10.0] * (2 * len(PASS)) + [524288.0]
    wv = [3.0] * (2 * len(PASS)) + [1048576.0]
    f, w = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    _counters(f, "FETCH_SIZE", names, fv)
    _counters(w, "WRITE_SIZE", names, wv)
    from synthetic import WORKLOADS
    _, rec = bench.ffn_traffic_markdown(f, w, WORKLOADS["mid_fwd"])
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    # reduce_grad launches two kernels per pass: 2 x (10 KiB x 2 + 3 KiB) per call
    assert rec["calls"]["reduce_grad"]["bytes_per_launch"] == 2 * (10 * 1024 * 2 + 3 * 1024)
    assert rec["calls"]["swiglu"]["bytes_per_launch"] == 10 * 1024 * 2 + 3 * 1024
    assert rec["calls"]["plan"]["bytes_per_launch"] == 4 * (10 * 1024 * 2 + 3 * 1024)


def test_hot_rank_factor_extremes():
    import numpy as np
    from synthetic import WORKLOADS
    wl = WORKLOADS["mid_fwd"].with_dims(S=16)
    per = wl.E // wl.R
    # every token of every rank routed to rank 0's home experts: that rank would hold R times P
    idx = np.tile(np.arange(wl.K) % per, (wl.R, wl.S, 1))
    assert bench.hot_rank_factor(idx, wl) == wl.R
    # each rank's pairs spread evenly over all ranks' experts: every rank holds exactly P
    flat = (np.arange(wl.R * wl.S * wl.K) % wl.E).reshape(wl.R, wl.S, wl.K)
    assert bench.hot_rank_factor(flat, wl) == 1.0


def test_mfma_table_from_counters(tmp_path):
    # two forward GEMM dispatches of 1 ms whose CUs are busy 1.9e6 cycles each at half the matrix pipes'
    # cycles, one wgrad dispatch, and the tile kernel beside them, which issues no MFMA
    path = str(tmp_path / "sq.csv")
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for disp, key, dur_ns, insts in ((1, "fwd", 1_000_000, 1e7), (2, "tiles", 4_000, 0.0), (3, "fwd", 1_000_000, 1e7),
                                     (4, "wgrad", 2_000_000, 2e7)):
        cu = 256 * 1.9e9 * dur_ns * 1e-9
        vals = {"SQ_INSTS_MFMA": insts, "SQ_BUSY_CU_CYCLES": cu, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 4 * cu if insts else 0}
        for c, v in vals.items():
            rows.append({"Dispatch_Id": disp, "Kernel_Name": NAMES[key], "Counter_Name": c, "Counter_Value": v,
                         "Start_Timestamp": 10_000 * disp, "End_Timestamp": 10_000 * disp + dur_ns})
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)
    from synthetic import WORKLOADS
    table, rec = bench.mfma_markdown(path, WORKLOADS["mid_fwd"], 1.0)
    k = rec["kernels"]
    assert set(k) == {"ggemm_bf16<false>", "wgrad_bf16"}
    f = k["ggemm_bf16<false>"]
    assert f["stage"] == "group_gemm" and f["dispatches"] == 2
    assert f["engine_clock_ghz"] == 1.9 and f["mfma_busy_of_cu_busy"] == 0.5
    assert f["issued_tflops"] == round(1e7 * 32768 / 1e-3 / 1e12, 1)
    # half the pipes' cycles at 1.9 GHz of a 2.4 GHz peak
    assert f["of_nominal_peak"] == round(0.5 * 1.9 / 2.4, 4)
    assert k["wgrad_bf16"]["stage"] == "wgrad" and k["wgrad_bf16"]["avg_us"] == 2000.0
    assert "`ggemm_bf16<false>` | group_gemm | 2 |" in table


def test_vendor_mfma_table_splits_the_calls_by_shape(tmp_path):
    # a vendor pass on the mid workload: 2 + R calls of the forward shape, then of the weight-gradient shape,
    # with a copy kernel between them that issues no MFMA; each call's matrix pipes are busy 60% of its CU
    # cycles at 1.5 GHz
    from synthetic import WORKLOADS
    wl = WORKLOADS["mid_fwd"]
    path = str(tmp_path / "vendor.csv")
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    shapes = bench.vendor_shapes(wl)
    calls = [(s, 1_000_000 + 1000 * i) for s in shapes for i in range(2 + wl.R)]
    calls.insert(2 + wl.R, (None, 5000))
    rows = []
    for disp, (shape, dur_ns) in enumerate(calls):
        cu = 256 * 1.5e9 * dur_ns * 1e-9
        vals = {"SQ_INSTS_MFMA": 1e6 if shape else 0, "SQ_BUSY_CU_CYCLES": cu,
                "SQ_VALU_MFMA_BUSY_CYCLES": 0.6 * 4 * cu if shape else 0}
        name = "Cijk_Ailk_Bljk_BBS_MT256x256x64(args)" if shape else "copy_kernel(args)"
        for c, v in vals.items():
            rows.append({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v,
                         "Start_Timestamp": 10_000_000 * disp, "End_Timestamp": 10_000_000 * disp + dur_ns})
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)
    table, rec = bench.vendor_mfma_markdown(path, wl)
    assert list(rec["shapes"]) == ["fwd", "wgrad"]
    fwd, wg = rec["shapes"]["fwd"], rec["shapes"]["wgrad"]
    assert (fwd["m"], fwd["k"], fwd["n"]) == (wl.S * wl.K, wl.H, wl.Hp)
    assert (wg["m"], wg["k"], wg["n"]) == (wl.H, wl.S * wl.K, wl.Hp)
    assert len(fwd["calls"]) == len(wg["calls"]) == 2 + wl.R
    c0 = fwd["calls"][0]
    assert c0["engine_clock_ghz"] == 1.5 and c0["mfma_busy_of_cu_busy"] == 0.6 and c0["us"] == 1000.0
    assert c0["tflops"] == round(2.0 * wl.S * wl.K * wl.H * wl.Hp / 1e-3 / 1e12, 1)
    assert wg["calls"][0]["us"] == 1000.0  # the copy kernel between the shapes was skipped
    assert "| fwd " in table and "`Cijk_Ailk_Bljk_BBS_MT256x256x64`" in table


def test_stage_roofline_fraction_and_algorithmic_bytes():
    # the per-point roofline fractions of the sweep: achieved = algorithmic work / time, frac = achieved / peak;
    # prefetch moves 2*H*H'*b per slotted copy, reduce_grad 4*H*H'*(2 per expert with copies + 2 per copy)
    import numpy as np
    from synthetic import WORKLOADS

    wl = WORKLOADS["mid_fwd"]

    class FakeLayer:  # algorithmic() reads only the plan's cu_seqlens from the layer
        def __init__(self):
            import torch
            G = wl.E + wl.B
            cu = np.zeros((wl.R, G + 1), dtype=np.int32)
            cu[:, 1:] = np.linspace(0, wl.P, G + 1, dtype=np.int64)[1:].astype(np.int32)
            self.cu_seqlens = torch.as_tensor(cu)

    slots = -np.ones((wl.R, wl.B), dtype=np.int32)
    slots[1, 0] = slots[2, 0] = slots[3, 1] = 5  # three copies of expert 5
    slots[4, 0] = 9                              # one copy of expert 9
    stats = [4, 4, 0, 0]
    alg = bench.algorithmic(wl, stats, slots, FakeLayer())
    hh = wl.H * wl.Hp
    assert alg["prefetch"] == 2 * hh * 2 * 4
    assert alg["reduce_grad"] == 4 * hh * (2 * 2 + 2 * 4)
    assert alg["group_gemm"] == 2 * wl.N * hh
    r = bench.stage_roofline("reduce_grad", alg, 0.05, {}, False)
    assert r["unit"] == "GB/s" and r["bound"] == "hbm"
    assert abs(r["achieved"] - alg["reduce_grad"] / 0.05e-3 / 1e9) < 0.01
    assert abs(r["frac"] - r["achieved"] / bench.HBM_PEAK_GBS) < 1e-4
    g = bench.stage_roofline("group_gemm", alg, 1.0, {}, False)
    assert g["unit"] == "TFLOP/s" and abs(g["frac"] - (alg["group_gemm"] / 1e-3 / 1e12) / bench.MFMA_BF16_PEAK_TFLOPS) < 1e-4


def test_gemm_roofline_takes_the_higher_floor():
    # large wgrad: 7.7 TFLOP (3.08 ms at the MFMA peak) but 39.7 GB of least bytes (4.96 ms at 8 TB/s): HBM binds
    alg = {"wgrad": 2 * 262144 * 7168 * 2048, "wgrad_min_bytes": 39.7e9}
    r = bench.stage_roofline("wgrad", alg, 10.0, {}, False)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert abs(r["achieved"] - 39.7e9 / 10e-3 / 1e9) < 0.01
    assert r["floors_ms"]["hbm"] > r["floors_ms"]["compute"]
    assert abs(r["tflops"] - alg["wgrad"] / 10e-3 / 1e12) < 0.01
    # mid forward GEMM: 1.134 TFLOP (0.45 ms) against 1.77 GB (0.22 ms): MFMA binds
    alg = {"group_gemm": 1.134e12, "group_gemm_min_bytes": 1.77e9}
    g = bench.stage_roofline("group_gemm", alg, 1.0, {}, False)
    assert g["bound"] == "mfma" and g["unit"] == "TFLOP/s" and g["achieved"] == g["tflops"]
    # float32 GEMMs price against the fp32 vector peak
    f = bench.stage_roofline("group_gemm", alg, 1.0, {}, True)
    assert f["bound"] == "alu" and f["peak"] == bench.MFMA_F32_VECTOR_TFLOPS
