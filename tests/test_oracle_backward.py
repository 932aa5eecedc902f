"""Pins the backward data-path oracle (combine backward, group-GEMM dgrad, dispatch backward), CPU only.

Pins: each stage is the adjoint (transpose) of its forward stage, which is itself pinned
(<C^T u, v> = <u, C v> on random vectors, with H != H' so a missing transpose cannot even run);
the gate gradient equals the exact finite difference of the forward output (the output is linear
in each gate); the planned backward chain equals the plain per-token gradient for many random
plans (slots and direct reads included); the plain gradient and the weight gradient after wgrad +
reduce_grad equal float64 torch autograd of the plain forward; planted mistakes fail the pins.
"""
import numpy as np
import pytest
import torch

from oracle import layer, planner
from tests.test_oracle_layer import _case


def _plan(c):
    return planner.plan(c["idx"], c["E"], c["B"])


def _dot(a, b):
    return float(np.sum(np.asarray(a, dtype=np.float64) * np.asarray(b, dtype=np.float64)))


def _close(a, b, scale):
    return abs(a - b) <= 1e-11 * (1.0 + scale)


def _combine_adjoint_holds(c, combine_backward):
    p = _plan(c)
    rng = c["rng"]
    N = c["R"] * c["S"] * c["K"]
    Yp = rng.standard_normal((N, c["Hp"]))
    dout = rng.standard_normal((c["R"], c["S"], c["Hp"]))
    dYp, _ = combine_backward(dout, Yp, p.dest_idx, c["gates"])
    lhs = _dot(dYp, Yp)
    rhs = _dot(dout, layer.combine(Yp, p.dest_idx, c["gates"]))
    return _close(lhs, rhs, float(np.abs(dYp).sum() * np.abs(Yp).max()))


def _dispatch_adjoint_holds(c, dispatch_backward):
    p = _plan(c)
    rng = c["rng"]
    N = c["R"] * c["S"] * c["K"]
    dXp = rng.standard_normal((N, c["H"]))
    dX = dispatch_backward(dXp, p.dest_idx)
    lhs = _dot(dX, c["X"])
    rhs = _dot(dXp, layer.dispatch(c["X"], p.dest_idx))
    return _close(lhs, rhs, float(np.abs(dXp).sum() * np.abs(c["X"]).max()))


def _gemm_adjoint_holds(c, dgrad):
    p = _plan(c)
    rng = c["rng"]
    N = c["R"] * c["S"] * c["K"]
    P = c["S"] * c["K"]
    Ws = layer.prefetch(c["W"], p.slot_expert)
    Xp = rng.standard_normal((N, c["H"]))
    dYp = rng.standard_normal((N, c["Hp"]))
    lhs = _dot(dgrad(dYp, c["W"], Ws, p.cu_seqlens, P), Xp)
    rhs = _dot(dYp, layer.group_gemm(Xp, c["W"], Ws, p.cu_seqlens, P))
    return _close(lhs, rhs, float(np.abs(dYp).sum() * np.abs(Xp).max() * np.abs(c["W"]).max() * c["H"]))


@pytest.mark.parametrize("seed", range(30))
def test_combine_backward_is_adjoint_of_combine(seed):
    assert _combine_adjoint_holds(_case(seed), layer.combine_backward)


@pytest.mark.parametrize("seed", range(30))
def test_dispatch_backward_is_adjoint_of_dispatch(seed):
    assert _dispatch_adjoint_holds(_case(seed), layer.dispatch_backward)


@pytest.mark.parametrize("seed", range(30))
def test_dgrad_is_adjoint_of_group_gemm(seed):
    assert _gemm_adjoint_holds(_case(seed), layer.group_gemm_dgrad)


def test_gate_gradient_is_exact_finite_difference():
    for seed in range(10):
        c = _case(seed)
        p = _plan(c)
        rng = c["rng"]
        N = c["R"] * c["S"] * c["K"]
        Yp = rng.standard_normal((N, c["Hp"]))
        dout = rng.standard_normal((c["R"], c["S"], c["Hp"]))
        _, dgate = layer.combine_backward(dout, Yp, p.dest_idx, c["gates"])
        base = _dot(dout, layer.combine(Yp, p.dest_idx, c["gates"]))
        for (r, s, k) in [(0, 0, 0), (c["R"] - 1, c["S"] - 1, c["K"] - 1)]:
            g = c["gates"].copy()
            g[r, s, k] += 1.0  # the output is linear in each gate, so a unit step is exact
            diff = _dot(dout, layer.combine(Yp, p.dest_idx, g)) - base
            assert abs(diff - dgate[r, s, k]) <= 1e-11 * (1 + np.abs(dout[r, s]).sum() * np.abs(Yp).max())


@pytest.mark.parametrize("seed", range(40))
def test_planned_backward_equals_plain_gradient(seed):
    c = _case(seed)
    p = _plan(c)
    P = c["S"] * c["K"]
    Ws = layer.prefetch(c["W"], p.slot_expert)
    Xp = layer.dispatch(c["X"], p.dest_idx)
    Yp = layer.group_gemm(Xp, c["W"], Ws, p.cu_seqlens, P)
    dout = c["rng"].standard_normal((c["R"], c["S"], c["Hp"]))
    dYp, dgate = layer.combine_backward(dout, Yp, p.dest_idx, c["gates"])
    dX = layer.dispatch_backward(layer.group_gemm_dgrad(dYp, c["W"], Ws, p.cu_seqlens, P), p.dest_idx)
    ref_dX, ref_dgate = layer.moe_backward(c["X"], c["W"], c["idx"], c["gates"], dout)
    assert np.allclose(dX, ref_dX, rtol=1e-12, atol=1e-12)
    assert np.allclose(dgate, ref_dgate, rtol=1e-12, atol=1e-12)


def test_sampled_rows_match_full_dgrad():
    c = _case(5)
    p = _plan(c)
    P = c["S"] * c["K"]
    Ws = layer.prefetch(c["W"], p.slot_expert)
    N = c["R"] * P
    dYp = c["rng"].standard_normal((N, c["Hp"]))
    full = layer.group_gemm_dgrad(dYp, c["W"], Ws, p.cu_seqlens, P)
    rows = np.arange(N)[::2]
    assert np.allclose(layer.group_gemm_dgrad(dYp, c["W"], Ws, p.cu_seqlens, P, rows=rows), full[rows],
                       rtol=1e-13, atol=1e-13)
    tok = np.arange(c["R"] * c["S"])[::3]
    dXp = c["rng"].standard_normal((N, c["H"]))
    assert np.allclose(layer.dispatch_backward(dXp, p.dest_idx, tokens=tok),
                       layer.dispatch_backward(dXp, p.dest_idx).reshape(-1, c["H"])[tok], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(8))
def test_plain_and_planned_gradients_match_torch_autograd(seed):
    c = _case(seed)
    R, S, K, E, H, Hp = c["R"], c["S"], c["K"], c["E"], c["H"], c["Hp"]
    dout = c["rng"].standard_normal((R, S, Hp))
    X = torch.tensor(c["X"], dtype=torch.float64, requires_grad=True)
    W = torch.tensor(c["W"], dtype=torch.float64, requires_grad=True)
    G = torch.tensor(c["gates"], dtype=torch.float64, requires_grad=True)
    ids = torch.tensor(np.asarray(c["idx"]), dtype=torch.int64)
    y = torch.einsum("rsh,rskhn->rskn", X, W[ids])  # float64 on the CPU
    out = (G.unsqueeze(-1) * y).sum(dim=2)
    (out * torch.tensor(dout)).sum().backward()
    ref_dX, ref_dgate = layer.moe_backward(c["X"], c["W"], c["idx"], c["gates"], dout)
    assert np.allclose(X.grad.numpy(), ref_dX, rtol=1e-12, atol=1e-12)
    assert np.allclose(G.grad.numpy(), ref_dgate, rtol=1e-12, atol=1e-12)
    # weight gradient through the planned chain: wgrad on dYp, then reduce_grad
    p = _plan(c)
    P = S * K
    Ws = layer.prefetch(c["W"], p.slot_expert)
    Xp = layer.dispatch(c["X"], p.dest_idx)
    Yp = layer.group_gemm(Xp, c["W"], Ws, p.cu_seqlens, P)
    dYp, _ = layer.combine_backward(dout, Yp, p.dest_idx, c["gates"])
    dWh = np.zeros((E, H, Hp))
    dWs = np.zeros((R, max(c["B"], 0), H, Hp))
    layer.wgrad(Xp, dYp, p.cu_seqlens, P, dWh, dWs)
    layer.reduce_grad(p.slot_expert, dWh, dWs)
    assert np.allclose(dWh, W.grad.numpy(), rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------------ planted mistakes

def test_pins_catch_untransposed_dgrad_weight():
    def wrong(dYp, W_home, W_slots, cu, P):  # forgets the transpose (square weights so it runs)
        return layer.group_gemm(dYp, W_home, W_slots, cu, P)
    caught = 0
    for seed in range(10):
        c = _case(seed, H=6, Hp=6)
        c["W"] = c["rng"].standard_normal((c["E"], 6, 6))
        caught += not _gemm_adjoint_holds(c, wrong)
    assert caught >= 8


def test_pins_catch_dropped_last_k():
    def wrong(dXp, dest_idx):
        return layer.dispatch_backward(dXp, dest_idx[:, :, :-1])
    caught = sum(not _dispatch_adjoint_holds(_case(seed), wrong) for seed in range(20) if _case(seed)["K"] > 1)
    assert caught >= 1 and caught == sum(1 for seed in range(20) if _case(seed)["K"] > 1)


def test_pins_catch_gate_of_wrong_k():
    def wrong(dout, Yp, dest_idx, gates):
        return layer.combine_backward(dout, Yp, dest_idx, np.roll(gates, 1, axis=2))
    ks = [seed for seed in range(20) if _case(seed)["K"] > 1]
    caught = sum(not _combine_adjoint_holds(_case(seed), wrong) for seed in ks)
    assert caught == len(ks) and caught >= 1
