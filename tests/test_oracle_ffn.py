"""Pins the full gated expert FFN in the oracle (silu, swiglu and its gradient, the planned chain), CPU only.

Pins: silu equals torch's library silu in float64 (extreme arguments included) and satisfies the
odd-part identity silu(g) - silu(-g) = g; the swiglu gradient equals central finite differences
and float64 torch autograd; the planned FFN (dispatch -> gate|up GEMM -> swiglu -> down GEMM ->
combine) equals the plain gated-expert MoE on random plans with slots and direct reads; its
backward (combine backward, dgrad and wgrad of both projections, swiglu backward, dispatch
backward, reduce_grad) equals float64 torch autograd of the plain forward; swapped gate/up halves
fail the pins.
"""
import numpy as np
import pytest
import torch

from oracle import layer, planner
from tests.plan_checks import random_routing


def _ffn_case(seed, H=8, Hp=5):
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.integers(1, 4))
    per = int(rng.integers(1, 4))
    E = R * per
    K = int(rng.integers(1, min(E, 3) + 1))
    S = int(rng.integers(1, 6))
    B = int(rng.integers(0, per + 2))
    idx = random_routing(rng, R, S, K, E, float(rng.uniform(0, 3)))
    logits = rng.standard_normal((R, S, K))
    gates = np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)
    X = rng.standard_normal((R, S, H))
    Wgu = rng.standard_normal((E, H, 2 * Hp)) / np.sqrt(H)
    Wd = rng.standard_normal((E, Hp, H)) / np.sqrt(Hp)
    return dict(R=R, E=E, K=K, S=S, B=B, H=H, Hp=Hp, idx=idx, gates=gates, X=X, Wgu=Wgu, Wd=Wd, rng=rng)


def test_silu_matches_library_and_odd_part_identity():
    g = np.concatenate([np.linspace(-30, 30, 601), [-800.0, -50.0, 0.0, 50.0, 800.0]])
    ref = torch.nn.functional.silu(torch.tensor(g, dtype=torch.float64)).numpy()
    assert np.allclose(layer.silu(g), ref, rtol=1e-15, atol=1e-300)
    assert np.allclose(layer.silu(g) - layer.silu(-g), g, rtol=1e-13, atol=1e-13)
    assert layer.silu(np.array([0.0]))[0] == 0.0


def test_swiglu_gradient_is_finite_difference_and_autograd():
    rng = np.random.default_rng(1)
    Y = rng.standard_normal((7, 10)) * 3
    dA = rng.standard_normal((7, 5))
    got = layer.swiglu_backward(Y, dA)
    h = 1e-6
    fd = np.zeros_like(Y)
    for i in range(Y.shape[0]):
        for j in range(Y.shape[1]):
            Yp, Ym = Y.copy(), Y.copy()
            Yp[i, j] += h
            Ym[i, j] -= h
            fd[i, j] = np.sum(dA * (layer.swiglu(Yp) - layer.swiglu(Ym))) / (2 * h)
    assert np.allclose(got, fd, rtol=1e-7, atol=1e-8)
    Yt = torch.tensor(Y, requires_grad=True)
    a = torch.nn.functional.silu(Yt[:, :5]) * Yt[:, 5:]
    (a * torch.tensor(dA)).sum().backward()
    assert np.allclose(got, Yt.grad.numpy(), rtol=1e-13, atol=1e-13)


def _planned_ffn(c, swiglu=layer.swiglu):
    p = planner.plan(c["idx"], c["E"], c["B"])
    P = c["S"] * c["K"]
    Xp = layer.dispatch(c["X"], p.dest_idx)
    Wgus = layer.prefetch(c["Wgu"], p.slot_expert)
    Wds = layer.prefetch(c["Wd"], p.slot_expert)
    Ygu = layer.group_gemm(Xp, c["Wgu"], Wgus, p.cu_seqlens, P)
    A = swiglu(Ygu)
    Zp = layer.group_gemm(A, c["Wd"], Wds, p.cu_seqlens, P)
    out = layer.combine(Zp, p.dest_idx, c["gates"])
    return p, P, Xp, Wgus, Wds, Ygu, A, Zp, out


@pytest.mark.parametrize("seed", range(30))
def test_planned_ffn_equals_plain_gated_moe(seed):
    c = _ffn_case(seed)
    out = _planned_ffn(c)[-1]
    ref = layer.moe_ffn_forward(c["X"], c["Wgu"], c["Wd"], c["idx"], c["gates"])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_planned_ffn_backward_equals_autograd(seed):
    c = _ffn_case(seed)
    R, S, K, E, H, Hp = c["R"], c["S"], c["K"], c["E"], c["H"], c["Hp"]
    p, P, Xp, Wgus, Wds, Ygu, A, Zp, out = _planned_ffn(c)
    dout = c["rng"].standard_normal((R, S, H))
    dZp, dgate = layer.combine_backward(dout, Zp, p.dest_idx, c["gates"])
    dA = layer.group_gemm_dgrad(dZp, c["Wd"], Wds, p.cu_seqlens, P)
    dYgu = layer.swiglu_backward(Ygu, dA)
    dX = layer.dispatch_backward(layer.group_gemm_dgrad(dYgu, c["Wgu"], Wgus, p.cu_seqlens, P), p.dest_idx)
    B = max(c["B"], 0)
    dWd, dWds = np.zeros((E, Hp, H)), np.zeros((R, B, Hp, H))
    layer.wgrad(A, dZp, p.cu_seqlens, P, dWd, dWds)
    layer.reduce_grad(p.slot_expert, dWd, dWds)
    dWgu, dWgus = np.zeros((E, H, 2 * Hp)), np.zeros((R, B, H, 2 * Hp))
    layer.wgrad(Xp, dYgu, p.cu_seqlens, P, dWgu, dWgus)
    layer.reduce_grad(p.slot_expert, dWgu, dWgus)
    # float64 autograd of the plain forward (CPU)
    X = torch.tensor(c["X"], requires_grad=True)
    Wgu = torch.tensor(c["Wgu"], requires_grad=True)
    Wd = torch.tensor(c["Wd"], requires_grad=True)
    G = torch.tensor(c["gates"], requires_grad=True)
    ids = torch.tensor(np.asarray(c["idx"]), dtype=torch.int64)
    y = torch.einsum("rsh,rskhn->rskn", X, Wgu[ids])
    a = torch.nn.functional.silu(y[..., :Hp]) * y[..., Hp:]
    z = torch.einsum("rskn,rsknh->rskh", a, Wd[ids])
    o = (G.unsqueeze(-1) * z).sum(dim=2)
    assert np.allclose(o.detach().numpy(), out, rtol=1e-12, atol=1e-12)
    (o * torch.tensor(dout)).sum().backward()
    assert np.allclose(dX, X.grad.numpy(), rtol=1e-11, atol=1e-11)
    assert np.allclose(dgate, G.grad.numpy(), rtol=1e-11, atol=1e-11)
    assert np.allclose(dWd, Wd.grad.numpy(), rtol=1e-11, atol=1e-11)
    assert np.allclose(dWgu, Wgu.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_pins_catch_swapped_gate_and_up():
    def swapped(Ygu):
        Hp = Ygu.shape[1] // 2
        return layer.swiglu(np.concatenate([Ygu[:, Hp:], Ygu[:, :Hp]], axis=1))
    caught = 0
    for seed in range(10):
        c = _ffn_case(seed)
        out = _planned_ffn(c, swapped)[-1]
        ref = layer.moe_ffn_forward(c["X"], c["Wgu"], c["Wd"], c["idx"], c["gates"])
        caught += not np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert caught == 10
