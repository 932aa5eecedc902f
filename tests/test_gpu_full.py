"""Parity at the workloads' full sizes, in the launch configuration the benchmark times (GPU).

The planner is compared bit for bit on every array, at every sweep point.  Every dispatched row and
every prefetched slot is compared bitwise.  Float results are compared element by element against the
oracle on whole units -- every GEMM row of two whole ranks (one holding the most slot groups, and the
last rank, whose tail holds the GEMM's last raster band), every combined token of one rank, the whole
gradient of four experts after wgrad + reduce_grad -- within 1e-2*(1+|ref|) for the bf16 GEMMs and
1e-2*(1+sum|g*y|) for tokens combined from bf16 rows; and every GEMM row, combined token and expert
gradient through row-sum properties that follow from that bound.  Also: guard regions around every
output buffer, bitwise run-to-run determinism, HIP-graph replay, and no allocation across a sweep.
"""
import numpy as np
import pytest
import torch

from oracle import layer as olayer
from oracle import planner as oplanner
from synthetic import WORKLOADS
from synthetic.calibrate import alpha_for
from synthetic.router import TAG_DY, TAG_W, TAG_X, normal_tensor, router_output
from tests.gpu_util import (DEV, DeviceExperts, DeviceRows, DispatchedRows, Guarded, OracleSlots,
                            assert_gemm_close, np64, npi, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import load_balanced_dispatch_amd as mod
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return mod


def routing(wl, target, seed=0):
    alpha = 0.0 if wl.zipf_s is not None else (wl.alpha if target is None else alpha_for(wl, seed, target))
    return router_output(wl.R, wl.S, wl.E, wl.K, seed, alpha=alpha, zipf_s=wl.zipf_s)


def build_layer(m, wl, target, backward=False, seed=0, data_grad=False):
    idx, gates = routing(wl, target, seed)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    L = m.MoeLayer(wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp, dtype=dt, backward=backward, data_grad=data_grad)
    L.topk_idx.copy_(torch.as_tensor(idx))
    L.gates.copy_(torch.as_tensor(gates))
    L.X.copy_(normal_tensor((wl.R, wl.S, wl.H), 1.0, wl.dtype, seed, TAG_X, "cuda", slices=wl.R))
    if wl.Hp is not None:
        L.W_home.copy_(normal_tensor((wl.E, wl.H, wl.Hp), wl.H ** -0.5, wl.dtype, seed, TAG_W, "cuda", slices=wl.E))
        if backward:
            L.dY.copy_(normal_tensor((wl.N, wl.Hp), 1.0, wl.dtype, seed, TAG_DY, "cuda", slices=wl.R))
    return L, idx, gates


PLAN_CASES = [("mid_fwd", 0.0), ("mid_fwd", 1.0), ("mid_fwd", 3.0), ("large_fwd", 0.5), ("large_fwd", 1.0),
              ("large_fwd", 2.0), ("large_fwd", 4.0), ("mid_bwd", 2.0), ("plan_stress", None), ("tiny_f32", None)]


@pytest.mark.parametrize("planner", ["prefix", "mincopy"])
@pytest.mark.parametrize("name,target", PLAN_CASES)
def test_full_plan_bit_exact(m, name, target, planner):
    wl = WORKLOADS[name]
    idx, _ = routing(wl, target)
    say("full plan", name, target, planner)
    d = m.make_dims(wl.R, wl.E, wl.B, wl.S, wl.K)
    dev = dict(device="cuda")
    counts = torch.empty(wl.E, dtype=torch.int32, **dev)
    mv = torch.empty(1, dtype=torch.float64, **dev)
    cu = torch.empty((wl.R, wl.E + wl.B + 1), dtype=torch.int32, **dev)
    slots = torch.empty((wl.R, wl.B), dtype=torch.int32, **dev)
    dest = torch.empty((wl.R, wl.S, wl.K), dtype=torch.int32, **dev)
    src = torch.empty(wl.N, dtype=torch.int32, **dev)
    stats = torch.empty(4, dtype=torch.int32, **dev)
    ws = torch.empty(m.moonep_plan_workspace_bytes(d), dtype=torch.uint8, **dev)
    m.moonep_plan_ex(d, planner, torch.as_tensor(idx).cuda(), counts, mv, cu, slots, dest, src, stats, ws)
    torch.cuda.synchronize()
    p = oplanner.plan(idx, wl.E, wl.B, planner=planner)
    assert npi(counts).tolist() == p.expert_counts.tolist()
    assert mv.item() == p.maxvio
    assert np.array_equal(npi(cu), p.cu_seqlens)
    assert np.array_equal(npi(slots), p.slot_expert)
    assert np.array_equal(npi(dest), p.dest_idx)
    assert np.array_equal(npi(src), p.src_of_row)
    assert npi(stats).tolist() == p.stats.tolist()
    if target is not None and target > 0:
        assert abs(p.maxvio - target) < 0.06


def check_ranks(p, wl):
    """Whole ranks the float checks cover: the rank holding the most slot groups (its buffer mixes home,
    slot and short groups) and the last rank, whose last groups hold the GEMM's last raster band."""
    r_slots = int(np.argmax((p.slot_expert >= 0).sum(axis=1))) if wl.B > 0 else 0
    return sorted({r_slots, wl.R - 1})


def expert_row_sums(W_home: torch.Tensor):
    """sum_n W[e, h, n] and sum_n |W[e, h, n]| in float64 for every expert (generated weights)."""
    ws = torch.empty(W_home.shape[:2], dtype=torch.float64, device=W_home.device)
    wa = torch.empty_like(ws)
    for e in range(W_home.shape[0]):
        w = W_home[e].double()
        ws[e] = w.sum(dim=1)
        wa[e] = w.abs().sum(dim=1)
    return ws, wa


def check_projected_rows(got_rows: torch.Tensor, xrows: torch.Tensor, experts: torch.Tensor, wsum, wabs, what):
    """Every output row at once, through the row-sum property: sum_n y[i, n] = x_i . wsum[e_i].  From the
    element bound |y - ref| <= 1e-2 (1 + |ref|) and |ref_n| <= sum_h |x_h w_hn|, the row sums may differ by
    at most 1e-2 (D + |x_i| . wabs[e_i])."""
    n = got_rows.shape[0]
    bad = 0
    for a in range(0, n, 16384):
        b = min(n, a + 16384)
        x = xrows[a:b].double()
        e = experts[a:b]
        ref = (x * wsum[e]).sum(dim=1)
        bound = 1e-2 * (got_rows.shape[1] + (x.abs() * wabs[e]).sum(dim=1))
        err = (got_rows[a:b].double().sum(dim=1) - ref).abs()
        bad += int((err > bound).sum().item())
    assert bad == 0, f"{what}: {bad} of {n} rows break the row-sum bound"


FWD_CASES = [("mid_fwd", 1.0, "prefix"), ("mid_fwd", 3.0, "prefix"), ("large_fwd", 0.5, "prefix"),
             ("large_fwd", 1.0, "prefix"), ("large_fwd", 2.0, "prefix"), ("large_fwd", 4.0, "prefix"),
             ("mid_fwd", 3.0, "mincopy"), ("large_fwd", 4.0, "mincopy")]


@pytest.mark.parametrize("name,target,planner", FWD_CASES)
def test_full_forward(m, name, target, planner):
    """Plan, every dispatched row (bitwise), every used slot (bitwise), every GEMM row of two whole ranks and
    every combined token of one rank (element by element against float64), and every GEMM row and combined
    token through the row-sum property."""
    wl = WORKLOADS[name]
    L, idx, gates = build_layer(m, wl, target)
    L.planner = planner
    say("full forward", name, target, planner)
    L.forward()
    torch.cuda.synchronize()
    p = oplanner.plan(idx, wl.E, wl.B, planner=planner)
    assert np.array_equal(npi(L.dest_idx), p.dest_idx)
    assert np.array_equal(npi(L.cu_seqlens), p.cu_seqlens)
    assert np.array_equal(npi(L.slot_expert), p.slot_expert)
    R, S, K, H, Hp, P = wl.R, wl.S, wl.K, wl.H, wl.Hp, wl.P
    Xf = L.X.reshape(-1, H)
    src_tok = torch.as_tensor(p.src_of_row // K, device=DEV)
    assert torch.equal(L.Xp, Xf[src_tok]), "dispatch: some row differs"
    for r in range(R):
        for j in range(wl.B):
            e = p.slot_expert[r, j]
            if e >= 0:
                assert torch.equal(L.W_slots[r, j], L.W_home[e])
    W = DeviceExperts(L.W_home)
    Ws = OracleSlots(W, p.slot_expert)
    Xp = DispatchedRows(Xf, p.src_of_row, K)
    ranks = check_ranks(p, wl)
    for r in ranks:
        say("  whole-rank GEMM rows", r)
        ref = olayer.group_gemm(Xp, W, Ws, p.cu_seqlens, P, ranks=[r])
        assert_gemm_close(np64(L.Yp[r * P:(r + 1) * P]), ref, 1e-2, f"group GEMM rows of rank {r}")
    rc = ranks[0]
    say("  combine of every token of rank", rc)
    ids = idx.reshape(-1, K)[rc * S:(rc + 1) * S]
    ref, scale = olayer.moe_forward_rows(np64(Xf[rc * S:(rc + 1) * S]), W, ids,
                                         gates.reshape(-1, K)[rc * S:(rc + 1) * S])
    got = np64(L.out.reshape(-1, Hp)[rc * S:(rc + 1) * S])
    bad = np.abs(got - ref) > 1e-2 * (1 + scale)
    assert not bad.any(), f"combined tokens of rank {rc}: {bad.sum()} elements outside the bound"
    say("  row-sum property of every GEMM row and combined token")
    wsum, wabs = expert_row_sums(L.W_home)
    expert_of_row = torch.as_tensor(idx.reshape(-1)[p.src_of_row], device=DEV)
    check_projected_rows(L.Yp, Xf[src_tok], expert_of_row, wsum, wabs, "group GEMM")
    del src_tok
    out_f = L.out.reshape(-1, Hp).double().sum(dim=1)
    ids_t = torch.as_tensor(idx.reshape(-1, K), device=DEV).long()
    g_t = torch.as_tensor(gates.reshape(-1, K), device=DEV).double()
    ref_t = torch.zeros(R * S, dtype=torch.float64, device=DEV)
    bound_t = torch.full((R * S,), 1e-2 * Hp, dtype=torch.float64, device=DEV)
    for a in range(0, R * S, 8192):
        b = min(R * S, a + 8192)
        x = Xf[a:b].double()
        for k in range(K):
            e = ids_t[a:b, k]
            ref_t[a:b] += g_t[a:b, k] * (x * wsum[e]).sum(dim=1)
            bound_t[a:b] += 1e-2 * g_t[a:b, k].abs() * (x.abs() * wabs[e]).sum(dim=1)
    nbad = int(((out_f - ref_t).abs() > bound_t).sum().item())
    assert nbad == 0, f"combine: {nbad} tokens break the row-sum bound"


BWD_CASES = [("mid_bwd", 2.0), ("large_fwd", 1.0)]


@pytest.mark.parametrize("name,target", BWD_CASES)
def test_full_weight_gradient(m, name, target):
    """wgrad + reduce_grad at full size: the whole [H, H'] gradient of four experts (the two with the most
    slot copies, the hottest, and one without copies) element by element against float64, every expert's
    row and column sums through the same property, and every slot cleared."""
    wl = WORKLOADS[name]
    L, idx, _ = build_layer(m, wl, target, backward=True)
    say("full weight gradient", name, target)
    L.plan()
    L.dispatch()
    L.wgrad()
    L.reduce_grad()
    torch.cuda.synchronize()
    p = oplanner.plan(idx, wl.E, wl.B)
    assert np.array_equal(npi(L.dest_idx), p.dest_idx)
    assert p.stats[1] > 0
    assert float(L.dW_slots.abs().max().item()) == 0.0  # every slot consumed and cleared
    R, S, K, H, Hp = wl.R, wl.S, wl.K, wl.H, wl.Hp
    copies = np.bincount(p.slot_expert[p.slot_expert >= 0], minlength=wl.E)
    by_copies = [int(e) for e in np.argsort(-copies, kind="stable") if copies[e] > 0]
    hottest = int(np.argmax(p.expert_counts))
    lone = int(np.nonzero(copies == 0)[0][0])
    experts = list(dict.fromkeys(by_copies[:2] + [hottest, lone]))
    X = L.X.float().cpu().numpy()  # bf16 values, exact in float32
    dY_of_pair = DeviceRows(L.dY, index=p.dest_idx.reshape(-1))  # the gradient row of each pair
    ref = olayer.expert_weight_grad(X, dY_of_pair, idx, wl.E, experts=experts)
    for i, e in enumerate(experts):
        say("  dW_home of expert", e, "copies", int(copies[e]))
        assert_gemm_close(np64(L.dW_home[e]), ref[i], 1e-2, f"dW_home[{e}]")
    say("  row and column sums of every expert's gradient")
    Xf = L.X.reshape(-1, H)
    dest = torch.as_tensor(p.dest_idx.reshape(-1), device=DEV).long()
    ids = torch.as_tensor(idx.reshape(-1), device=DEV).long()
    for e in range(wl.E):
        q = torch.nonzero(ids == e).flatten()
        if q.numel() == 0:
            assert float(L.dW_home[e].abs().max().item()) == 0.0
            continue
        x = Xf[q // K].double()
        dy = L.dY[dest[q]].double()
        dw = L.dW_home[e].double()
        col_ref = x.sum(dim=1) @ dy  # sum_h dW[h, n] = sum_i (sum_h x_ih) dy_in
        col_bound = 1e-2 * (H + x.abs().sum(dim=1) @ dy.abs())
        row_ref = x.T @ dy.sum(dim=1)  # sum_n dW[h, n]
        row_bound = 1e-2 * (Hp + x.abs().T @ dy.abs().sum(dim=1))
        assert bool(((dw.sum(dim=0) - col_ref).abs() <= col_bound).all()), f"column sums of dW_home[{e}]"
        assert bool(((dw.sum(dim=1) - row_ref).abs() <= row_bound).all()), f"row sums of dW_home[{e}]"


@pytest.mark.parametrize("name,target", [("mid_fwd", 1.0), ("large_fwd", 1.0)])
def test_full_dgrad_and_dispatch_backward(m, name, target):
    """dgrad on a generated dYp (the dY buffer, seeded N(0,1)): every dXp row of two whole ranks element by
    element against float64 and every row through the row-sum property; then dispatch backward: every
    token of one rank against the plain input gradient, its rows being sums of K bf16-rounded dXp rows."""
    wl = WORKLOADS[name]
    L, idx, _ = build_layer(m, wl, target, backward=True, data_grad=True)
    L.dY.copy_(normal_tensor((wl.N, wl.Hp), 1.0, wl.dtype, 0, TAG_DY, "cuda", slices=wl.R))
    say("full dgrad + dispatch backward", name, target)
    L.plan()
    L.prefetch()
    L.dgrad()
    L.dispatch_backward()
    torch.cuda.synchronize()
    p = oplanner.plan(idx, wl.E, wl.B)
    assert np.array_equal(npi(L.dest_idx), p.dest_idx)
    R, S, K, H, Hp, P = wl.R, wl.S, wl.K, wl.H, wl.Hp, wl.P
    W = DeviceExperts(L.W_home)
    Ws = OracleSlots(W, p.slot_expert)
    dY = DeviceRows(L.dY)
    ranks = check_ranks(p, wl)
    for r in ranks:
        say("  whole-rank dXp rows", r)
        ref = olayer.group_gemm_dgrad(dY, W, Ws, p.cu_seqlens, P, ranks=[r])
        assert_gemm_close(np64(L.dXp[r * P:(r + 1) * P]), ref, 1e-2, f"dXp rows of rank {r}")
    rc = ranks[0]
    say("  dX of every token of rank", rc)
    dest_rc = p.dest_idx[rc]  # [S, K]
    dY_rows = np64(L.dY[torch.as_tensor(dest_rc.reshape(-1), device=DEV)]).reshape(S, K, Hp)
    ref, scale = olayer.moe_input_grad_rows(dY_rows, W, idx[rc])
    got = np64(L.dX[rc])
    bad = np.abs(got - ref) > 1e-2 * (K + scale)
    assert not bad.any(), f"dX of rank {rc}: {bad.sum()} elements outside the bound"
    say("  row-sum property of every dXp row")
    csum = torch.empty((wl.E, Hp), dtype=torch.float64, device=DEV)
    cabs = torch.empty_like(csum)
    for e in range(wl.E):
        w = L.W_home[e].double()
        csum[e] = w.sum(dim=0)
        cabs[e] = w.abs().sum(dim=0)
    expert_of_row = torch.as_tensor(idx.reshape(-1)[p.src_of_row], device=DEV)
    check_projected_rows(L.dXp, L.dY, expert_of_row, csum, cabs, "dgrad")


def test_guard_regions_around_every_output(m):
    """Every stage of the forward, the weight backward and the data backward at the large workload's most
    skewed point, with each output inside a guarded allocation: after each stage, nothing has been written
    outside any output buffer."""
    wl = WORKLOADS["large_fwd"]
    L, _, _ = build_layer(m, wl, 4.0, backward=True, data_grad=True)
    L.dout.normal_(generator=torch.Generator(device="cuda").manual_seed(3))
    guards = {}
    for name in ("expert_counts", "cu_seqlens", "slot_expert", "dest_idx", "src_of_row", "stats", "Xp", "W_slots",
                 "Yp", "out", "dW_home", "dW_slots", "dY", "dgates", "dXp", "dX"):
        t = getattr(L, name)
        g = Guarded(t.shape, t.dtype)
        g.view.copy_(t)
        setattr(L, name, g.view)
        guards[name] = g
    torch.cuda.synchronize()
    stages = [("plan", L.plan), ("prefetch", L.prefetch), ("dispatch", L.dispatch), ("group_gemm", L.group_gemm),
              ("combine", L.combine), ("combine_backward", L.combine_backward), ("wgrad", L.wgrad),
              ("reduce_grad", L.reduce_grad), ("dgrad", L.dgrad), ("dispatch_backward", L.dispatch_backward)]
    for name, f in stages:
        say("  guarded stage", name)
        f()
        torch.cuda.synchronize()
        broken = [n for n, g in guards.items() if not g.intact()]
        assert not broken, f"{name} wrote outside {broken}"
    assert int(L.stats[1].item()) > 0


def test_full_stress_dispatch(m):
    """The routing-stress workload (1 048 576 pairs, maxvio ~ 46, direct reads): every dispatched row
    bitwise, with the dispatched buffer inside a guarded allocation."""
    wl = WORKLOADS["plan_stress"]
    L, idx, _ = build_layer(m, wl, None)
    g = Guarded(L.Xp.shape, L.Xp.dtype)
    L.Xp = g.view
    say("full stress plan+dispatch")
    L.forward()
    torch.cuda.synchronize()
    assert g.intact()
    p = oplanner.plan(idx, wl.E, wl.B)
    assert np.array_equal(npi(L.dest_idx), p.dest_idx)
    assert p.stats[2] > 0  # inference budget B=4: direct reads happen
    Xf = L.X.reshape(-1, wl.H)
    for a in range(0, wl.N, 1 << 18):  # every row, a quarter million at a time
        b = min(wl.N, a + (1 << 18))
        src_tok = torch.as_tensor(p.src_of_row[a:b] // wl.K, device=DEV)
        assert torch.equal(L.Xp[a:b], Xf[src_tok]), f"dispatched rows [{a}, {b})"


def test_run_to_run_bitwise(m):
    wl = WORKLOADS["mid_bwd"]
    L, _, _ = build_layer(m, wl, 2.0, backward=True)
    say("determinism")
    outs = []
    for _ in range(2):
        L.dW_home.zero_()
        L.dW_slots.zero_()
        L.Yp.fill_(float("nan"))
        L.out.fill_(float("nan"))
        L.forward()
        L.backward()
        torch.cuda.synchronize()
        outs.append((L.Yp.clone(), L.out.clone(), L.dW_home.clone(), L.dest_idx.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_graph_replay_matches_eager(m):
    wl = WORKLOADS["mid_bwd"].with_dims(S=512)
    L, _, _ = build_layer(m, wl, 2.0, backward=True)
    say("graph replay")
    L.forward()
    L.backward()  # warm up (device attributes, caches) before capture
    torch.cuda.synchronize()

    def reset():
        L.dW_home.zero_()
        L.dW_slots.zero_()

    reset()
    L.forward()
    L.backward()
    torch.cuda.synchronize()
    eager = (L.Yp.clone(), L.out.clone(), L.dW_home.clone(), L.cu_seqlens.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            L.forward()
            L.backward()
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        reset()
        L.Yp.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, (L.Yp, L.out, L.dW_home, L.cu_seqlens)):
            assert torch.equal(a, b)


def test_static_memory_across_sweep(m):
    wl = WORKLOADS["mid_fwd"]
    L, _, _ = build_layer(m, wl, 0.0)
    say("static memory sweep")
    L.forward()
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for tgt in (1.0, 3.0):
        idx, gates = routing(wl, tgt)
        L.topk_idx.copy_(torch.as_tensor(idx))
        L.gates.copy_(torch.as_tensor(gates))
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        L.forward()
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
