"""Pins the layer-stage oracle (dispatch, prefetch, group GEMM, combine, wgrad, reduce_grad), CPU only.

Pins: the combine/dispatch round trip (gates sum to one), the planned chain
against the plain MoE definition for many random plans (slots and direct reads
included), identity weights, the all-ones weight-gradient closed form, the
plan-independent weight gradient, accumulate-then-zero semantics, the fixed
rank order of reduce_grad in float32, and planted mistakes.
"""
import numpy as np
import pytest

from oracle import layer, planner
from tests.plan_checks import random_routing


def _case(seed, H=8, Hp=6, B=None):
    rng = np.random.default_rng(3000 + seed)
    R = int(rng.integers(1, 5))
    per = int(rng.integers(1, 4))
    E = R * per
    K = int(rng.integers(1, min(E, 3) + 1))
    S = int(rng.integers(1, 7))
    if B is None:
        B = int(rng.integers(0, per + 2))
    idx = random_routing(rng, R, S, K, E, float(rng.uniform(0, 3)))
    logits = rng.standard_normal((R, S, K))
    gates = np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)
    X = rng.standard_normal((R, S, H))
    W = rng.standard_normal((E, H, Hp)) / np.sqrt(H)
    return dict(R=R, E=E, K=K, S=S, B=B, H=H, Hp=Hp, idx=idx, gates=gates, X=X, W=W, rng=rng)


def _chain(c):
    p = planner.plan(c["idx"], c["E"], c["B"])
    Xp = layer.dispatch(c["X"], p.dest_idx)
    Ws = layer.prefetch(c["W"], p.slot_expert)
    Yp = layer.group_gemm(Xp, c["W"], Ws, p.cu_seqlens, c["S"] * c["K"])
    return p, Xp, Ws, Yp, layer.combine(Yp, p.dest_idx, c["gates"])


def test_round_trip_is_gate_sum_times_x():
    for seed in range(20):
        c = _case(seed)
        p = planner.plan(c["idx"], c["E"], c["B"])
        out = layer.combine(layer.dispatch(c["X"], p.dest_idx), p.dest_idx, c["gates"])
        assert np.allclose(out, c["X"] * c["gates"].sum(-1, keepdims=True), rtol=1e-13, atol=1e-13)


def test_dispatch_rows_are_source_tokens():
    c = _case(1)
    p = planner.plan(c["idx"], c["E"], c["B"])
    Xp = layer.dispatch(c["X"], p.dest_idx)
    K = c["K"]
    Xf = c["X"].reshape(-1, c["H"])
    for row in range(Xp.shape[0]):
        assert np.array_equal(Xp[row], Xf[p.src_of_row[row] // K])


@pytest.mark.parametrize("seed", range(40))
def test_planned_chain_equals_plain_moe(seed):
    c = _case(seed)
    _, _, _, _, out = _chain(c)
    ref = layer.moe_forward(c["X"], c["W"], c["idx"], c["gates"])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_direct_reads_and_slots_both_exercised():
    seen_direct = seen_slot = False
    for seed in range(40):
        c = _case(seed)
        p = planner.plan(c["idx"], c["E"], c["B"])
        seen_slot |= p.stats[1] > 0
        seen_direct |= p.stats[2] > 0
    assert seen_direct and seen_slot


def test_identity_weights_return_dispatched_rows():
    c = _case(4, H=6, Hp=6)
    scale = np.arange(1, c["E"] + 1, dtype=np.float64)
    W = np.stack([s * np.eye(6) for s in scale])
    p = planner.plan(c["idx"], c["E"], c["B"])
    Xp = layer.dispatch(c["X"], p.dest_idx)
    Yp = layer.group_gemm(Xp, W, layer.prefetch(W, p.slot_expert), p.cu_seqlens, c["S"] * c["K"])
    expert_of_row = c["idx"].reshape(-1)[p.src_of_row]
    assert np.allclose(Yp, Xp * scale[expert_of_row][:, None], rtol=0, atol=1e-14)


def test_sampled_rows_match_full_gemm():
    c = _case(9)
    p, Xp, Ws, Yp, _ = _chain(c)
    rows = np.arange(0, Xp.shape[0], 3)
    got = layer.group_gemm(Xp, c["W"], Ws, p.cu_seqlens, c["S"] * c["K"], rows=rows)
    assert np.allclose(got, Yp[rows], rtol=1e-13, atol=1e-13)


def test_prefetch_copies_and_leaves_unused_slots():
    c = _case(12)
    p = planner.plan(c["idx"], c["E"], c["B"])
    init = np.full((c["R"], c["B"], c["H"], c["Hp"]), 7.0)
    Ws = layer.prefetch(c["W"], p.slot_expert, init)
    for r in range(c["R"]):
        for j in range(c["B"]):
            e = p.slot_expert[r, j]
            assert np.array_equal(Ws[r, j], c["W"][e] if e >= 0 else init[r, j])


@pytest.mark.parametrize("seed", range(30))
def test_wgrad_then_reduce_equals_plain_gradient(seed):
    c = _case(seed)
    p = planner.plan(c["idx"], c["E"], c["B"])
    P, N = c["S"] * c["K"], c["R"] * c["S"] * c["K"]
    Xp = layer.dispatch(c["X"], p.dest_idx)
    dY = c["rng"].standard_normal((N, c["Hp"]))
    init = c["rng"].standard_normal((c["E"], c["H"], c["Hp"]))
    dWh = init.copy()
    dWs = np.zeros((c["R"], c["B"], c["H"], c["Hp"]))
    layer.wgrad(Xp, dY, p.cu_seqlens, P, dWh, dWs)
    layer.reduce_grad(p.slot_expert, dWh, dWs)
    dY_of_pair = dY[p.dest_idx.reshape(-1)]
    ref = layer.expert_weight_grad(c["X"], dY_of_pair, c["idx"], c["E"])
    assert np.allclose(dWh, init + ref, rtol=1e-12, atol=1e-12)  # accumulate, not overwrite
    assert np.all(dWs == 0)


def test_all_ones_gradient_is_expert_count():
    c = _case(21)
    p = planner.plan(c["idx"], c["E"], c["B"])
    P, N = c["S"] * c["K"], c["R"] * c["S"] * c["K"]
    Xp = np.ones((N, c["H"]))
    dY = np.ones((N, c["Hp"]))
    dWh = np.zeros((c["E"], c["H"], c["Hp"]))
    dWs = np.zeros((c["R"], c["B"], c["H"], c["Hp"]))
    layer.wgrad(Xp, dY, p.cu_seqlens, P, dWh, dWs)
    layer.reduce_grad(p.slot_expert, dWh, dWs)
    assert np.array_equal(dWh, np.broadcast_to(p.expert_counts[:, None, None].astype(float), dWh.shape))


def test_reduce_grad_rank_order_in_float32():
    # home + rank0 + rank1 in that order: (1e8 + 1) rounds back to 1e8 in float32, then -1e8 -> 0.
    # Any other order of the same three terms gives 1.
    slot_expert = np.array([[3, -1], [3, -1]])
    dWh = np.zeros((4, 1, 1), dtype=np.float32)
    dWh[3] = 1e8
    dWs = np.zeros((2, 2, 1, 1), dtype=np.float32)
    dWs[0, 0] = 1.0
    dWs[1, 0] = -1e8
    dWs[1, 1] = 5.0  # unused slot: never read, never cleared
    layer.reduce_grad(slot_expert, dWh, dWs, dtype=np.float32)
    assert dWh[3, 0, 0] == np.float32(0.0)
    assert dWs[0, 0, 0, 0] == 0 and dWs[1, 0, 0, 0] == 0 and dWs[1, 1, 0, 0] == 5.0


def test_combine_abs_bounds_combine():
    c = _case(5)
    p, _, _, Yp, out = _chain(c)
    assert np.all(np.abs(out) <= layer.combine_abs(Yp, p.dest_idx, c["gates"]) + 1e-15)


# ------------------------------------------------------------ planted mistakes


def test_pins_catch_transposed_weight(monkeypatch):
    real = layer.rank_weight
    monkeypatch.setattr(layer, "rank_weight", lambda Wh, Ws, r, g: real(Wh, Ws, r, g).T)
    c = _case(2, H=5, Hp=5)
    _, _, _, _, out = _chain(c)
    assert not np.allclose(out, layer.moe_forward(c["X"], c["W"], c["idx"], c["gates"]))


def test_pins_catch_dropped_slot_gradient(monkeypatch):
    def no_fold(slot_expert, dWh, dWs, dtype=np.float64):
        dWs[...] = 0
        return dWh, dWs

    monkeypatch.setattr(layer, "reduce_grad", no_fold)
    for seed in range(30):
        c = _case(seed)
        p = planner.plan(c["idx"], c["E"], c["B"])
        if p.stats[1] == 0:
            continue
        P, N = c["S"] * c["K"], c["R"] * c["S"] * c["K"]
        Xp = layer.dispatch(c["X"], p.dest_idx)
        dY = c["rng"].standard_normal((N, c["Hp"]))
        dWh = np.zeros((c["E"], c["H"], c["Hp"]))
        dWs = np.zeros((c["R"], c["B"], c["H"], c["Hp"]))
        layer.wgrad(Xp, dY, p.cu_seqlens, P, dWh, dWs)
        layer.reduce_grad(p.slot_expert, dWh, dWs)
        ref = layer.expert_weight_grad(c["X"], dY[p.dest_idx.reshape(-1)], c["idx"], c["E"])
        assert not np.allclose(dWh, ref)
        return
    pytest.fail("no case with a slot")


@pytest.mark.parametrize("seed", range(20))
def test_block_forms_equal_the_plain_definitions(seed):
    # the whole-rank, token-block and expert-subset forms that the full-size GPU checks use give the same
    # numbers as the pinned plain forms (H = 8 != H' = 6, so a missing transpose cannot even run)
    c = _case(seed)
    R, S, K, H, Hp, E = c["R"], c["S"], c["K"], c["H"], c["Hp"], c["E"]
    P = S * K
    rng = c["rng"]
    p, Xp, Ws, Yp, _ = _chain(c)
    ranks = sorted({R - 1, 0}, reverse=True)
    got = layer.group_gemm(Xp, c["W"], Ws, p.cu_seqlens, P, ranks=ranks)
    assert np.array_equal(got, np.concatenate([Yp[r * P:(r + 1) * P] for r in ranks]))
    dYp = rng.standard_normal((R * P, Hp))
    full = layer.group_gemm_dgrad(dYp, c["W"], Ws, p.cu_seqlens, P)
    got = layer.group_gemm_dgrad(dYp, c["W"], Ws, p.cu_seqlens, P, ranks=ranks)
    assert np.array_equal(got, np.concatenate([full[r * P:(r + 1) * P] for r in ranks]))

    toks = np.arange(R * S)[::2]
    ids = c["idx"].reshape(-1, K)[toks]
    g = c["gates"].reshape(-1, K)[toks]
    out, scale = layer.moe_forward_rows(c["X"].reshape(-1, H)[toks], c["W"], ids, g)
    ref = layer.moe_forward(c["X"], c["W"], c["idx"], c["gates"], tokens=toks)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)
    assert np.all(scale + 1e-12 >= np.abs(out))

    dout = rng.standard_normal((R, S, Hp))
    dX_ref, _ = layer.moe_backward(c["X"], c["W"], c["idx"], c["gates"], dout)
    dY_rows = g[:, :, None] * dout.reshape(-1, Hp)[toks][:, None, :]  # gate * dout: combine's backward
    dx, dscale = layer.moe_input_grad_rows(dY_rows, c["W"], ids)
    assert np.allclose(dx, dX_ref.reshape(-1, H)[toks], rtol=1e-12, atol=1e-12)
    assert np.all(dscale + 1e-12 >= np.abs(dx))

    dY_of_pair = rng.standard_normal((R * S * K, Hp))
    full = layer.expert_weight_grad(c["X"], dY_of_pair, c["idx"], E)
    ex = sorted({E - 1, 0}, reverse=True)
    got = layer.expert_weight_grad(c["X"], dY_of_pair, c["idx"], E, experts=ex)
    assert np.array_equal(got, full[ex])
