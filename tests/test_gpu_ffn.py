"""Parity of the gated expert FFN (swiglu, its gradient, wgrad with partial tiles, the whole FFN layer)
against the CPU oracle (GPU).

swiglu and its gradient are float32 arithmetic rounded once to the row dtype: |gpu - ref| <=
2^-8 |ref| for bf16 (one rounding plus a few float32 ulps), 1e-6 |ref| for float32, plus 1e-6 times
the size of the gradient's terms where its factor (1 + g(1 - s)) crosses zero.  The tiny float32
FFN layer (forward and backward) is held to 1e-4 (1 + |ref|) against the oracle's planned chain; the
mid bf16 FFN at full size to the bf16-GEMM bound on sampled tokens and on the whole weight gradients
of three experts (two with slot copies), with the oracle rounding the intermediates to bf16 at the same
points (Ygu, A, dYp, dA, dYgu).
"""
import numpy as np
import pytest
import torch

from oracle import layer as olayer
from oracle import planner as oplanner
from synthetic import WORKLOADS
from synthetic.calibrate import alpha_for
from synthetic.router import TAG_W, TAG_WD, TAG_X, normal_tensor, router_output
from tests.gpu_util import DEV, assert_gemm_close, bf16_round_np, f32, i32, np64, rand_tensor, say
from tests.plan_checks import random_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import load_balanced_dispatch_amd as mod
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return mod


def _rel_bound(dtype):
    return 2.0 ** -8 if dtype == torch.bfloat16 else 1e-6


@pytest.mark.parametrize("dtype,Hp", [(torch.bfloat16, 1408), (torch.bfloat16, 2048), (torch.float32, 256),
                                      (torch.bfloat16, 13), (torch.float32, 6)])
def test_swiglu(m, dtype, Hp):
    R, E, B, S, K = 2, 4, 1, 60, 3
    d = m.make_dims(R, E, B, S, K)
    N = R * S * K
    Ygu = rand_tensor((N, 2 * Hp), dtype, seed=Hp, std=3.0)
    A = torch.full((N, Hp), float("nan"), dtype=dtype, device=DEV)
    say("swiglu", dtype, Hp)
    m.moonep_swiglu(d, Hp, Ygu, A)
    torch.cuda.synchronize()
    ref = olayer.swiglu(np64(Ygu))
    err = np.abs(np64(A) - ref)
    assert np.all(err <= _rel_bound(dtype) * np.abs(ref) + 1e-30), float((err / (np.abs(ref) + 1e-30)).max())


@pytest.mark.parametrize("dtype,Hp", [(torch.bfloat16, 1408), (torch.float32, 256), (torch.bfloat16, 13),
                                      (torch.float32, 6)])
def test_swiglu_backward(m, dtype, Hp):
    R, E, B, S, K = 2, 4, 1, 60, 3
    d = m.make_dims(R, E, B, S, K)
    N = R * S * K
    Ygu = rand_tensor((N, 2 * Hp), dtype, seed=Hp + 1, std=3.0)
    dA = rand_tensor((N, Hp), dtype, seed=Hp + 2)
    dYgu = torch.full((N, 2 * Hp), float("nan"), dtype=dtype, device=DEV)
    say("swiglu_backward", dtype, Hp)
    m.moonep_swiglu_backward(d, Hp, Ygu, dA, dYgu)
    torch.cuda.synchronize()
    y, da = np64(Ygu), np64(dA)
    ref = olayer.swiglu_backward(y, da)
    # size of the gradient's terms (for the absolute part of the bound)
    g, u = y[:, :Hp], y[:, Hp:]
    s = np.abs(olayer.silu(g)) / np.maximum(np.abs(g), 1e-300)
    scale = np.concatenate([np.abs(da * u) * s * (1 + np.abs(g)), np.abs(da * g) * s], axis=1)
    err = np.abs(np64(dYgu) - ref)
    bound = _rel_bound(dtype) * np.abs(ref) + 1e-6 * scale + 1e-30
    assert np.all(err <= bound), float((err - bound).max())


@pytest.mark.parametrize("H,Hp", [(384, 256), (1408, 128)])
def test_wgrad_partial_h_tile(m, H, Hp):
    # H % 256 != 0: the last 256-row output tile is half empty (MFMA path, H % 128 == 0)
    rng = np.random.default_rng(H)
    R, E, B, S, K = 2, 4, 2, 150, 2
    topk = random_routing(rng, R, S, K, E, 2.0)
    p = oplanner.plan(topk, E, B)
    d = m.make_dims(R, E, B, S, K)
    N = R * S * K
    Xp = rand_tensor((N, H), torch.bfloat16, seed=1)
    dY = rand_tensor((N, Hp), torch.bfloat16, seed=2)
    dWh = rand_tensor((E, H, Hp), torch.float32, seed=3)
    dWs = torch.zeros((R, B, H, Hp), dtype=torch.float32, device=DEV)
    init_h = np64(dWh)
    ws = torch.empty(m.moonep_wgrad_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    say("wgrad partial h tile", H, Hp)
    m.moonep_wgrad(d, H, Hp, Xp, dY, i32(p.cu_seqlens), dWh, dWs, ws)
    torch.cuda.synchronize()
    ref_h, ref_s = olayer.wgrad(np64(Xp), np64(dY), p.cu_seqlens, S * K, init_h.copy(), np.zeros((R, B, H, Hp)))
    assert_gemm_close(np64(dWh), ref_h, 1e-2, "dW_home")
    assert_gemm_close(np64(dWs), ref_s, 1e-2, "dW_slots")


def _oracle_ffn(c_idx, gates, X, Wgu, Wd, E, B, dout, dtype_round=None):
    """The oracle's planned FFN chain (forward and backward) on the given inputs."""
    p = oplanner.plan(c_idx, E, B)
    R, S, K = c_idx.shape
    P = S * K
    Hp = Wd.shape[1]
    rnd = (lambda a: a) if dtype_round is None else dtype_round
    Xp = olayer.dispatch(X, p.dest_idx)
    Wgus, Wds = olayer.prefetch(Wgu, p.slot_expert), olayer.prefetch(Wd, p.slot_expert)
    Ygu = rnd(olayer.group_gemm(Xp, Wgu, Wgus, p.cu_seqlens, P))
    A = rnd(olayer.swiglu(Ygu))
    Zp = rnd(olayer.group_gemm(A, Wd, Wds, p.cu_seqlens, P))
    out = olayer.combine(Zp, p.dest_idx, gates)
    dZp, dgate = olayer.combine_backward(dout, Zp, p.dest_idx, gates)
    dZp = rnd(dZp)
    dA = rnd(olayer.group_gemm_dgrad(dZp, Wd, Wds, p.cu_seqlens, P))
    dYgu = rnd(olayer.swiglu_backward(Ygu, dA))
    dX = olayer.dispatch_backward(rnd(olayer.group_gemm_dgrad(dYgu, Wgu, Wgus, p.cu_seqlens, P)), p.dest_idx)
    Bm = max(B, 0)
    dWd, dWds = np.zeros((E, Hp, Wd.shape[2])), np.zeros((R, Bm, Hp, Wd.shape[2]))
    olayer.wgrad(A, dZp, p.cu_seqlens, P, dWd, dWds)
    olayer.reduce_grad(p.slot_expert, dWd, dWds)
    dWgu, dWgus = np.zeros(Wgu.shape), np.zeros((R, Bm) + Wgu.shape[1:])
    olayer.wgrad(Xp, dYgu, p.cu_seqlens, P, dWgu, dWgus)
    olayer.reduce_grad(p.slot_expert, dWgu, dWgus)
    return dict(out=out, dgate=dgate, dX=dX, dWd=dWd, dWgu=dWgu)


def test_tiny_ffn_layer_forward_backward(m):
    R, E, B, S, K, H, Hp = 4, 16, 4, 64, 2, 128, 256
    rng = np.random.default_rng(11)
    idx = random_routing(rng, R, S, K, E, 1.5)
    gates = rng.dirichlet(np.ones(K), size=(R, S)).astype(np.float32)
    L = m.MoeFFN(R, E, B, S, K, H, Hp, dtype=torch.float32, backward=True)
    L.topk_idx.copy_(torch.as_tensor(np.asarray(idx, dtype=np.int32)))
    L.gates.copy_(torch.as_tensor(gates))
    L.X.copy_(rand_tensor((R, S, H), torch.float32, seed=1))
    L.W_gu_home.copy_(rand_tensor((E, H, 2 * Hp), torch.float32, seed=2, std=H ** -0.5))
    L.W_down_home.copy_(rand_tensor((E, Hp, H), torch.float32, seed=3, std=Hp ** -0.5))
    L.dout.copy_(rand_tensor((R, S, H), torch.float32, seed=4))
    say("tiny FFN layer")
    L.forward()
    L.backward()
    torch.cuda.synchronize()
    ref = _oracle_ffn(np.asarray(idx), gates, np64(L.X), np64(L.W_gu_home), np64(L.W_down_home), E, B, np64(L.dout))
    assert_gemm_close(np64(L.out), ref["out"], 1e-4, "out")
    assert_gemm_close(np64(L.dgates), ref["dgate"], 1e-4, "dgates")
    assert_gemm_close(np64(L.dX), ref["dX"], 1e-4, "dX")
    assert_gemm_close(np64(L.dW_down_home), ref["dWd"], 1e-4, "dW_down")
    assert_gemm_close(np64(L.dW_gu_home), ref["dWgu"], 1e-4, "dW_gate_up")
    assert float(L.dW_gu_slots.abs().max()) == 0.0 and float(L.dW_down_slots.abs().max()) == 0.0


def test_mid_ffn_full_size(m):
    wl = WORKLOADS["mid_fwd"]
    R, E, B, S, K, H, Hp = wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp
    idx, gates = router_output(R, S, E, K, 0, alpha=alpha_for(wl, 0, 1.0))
    L = m.MoeFFN(R, E, B, S, K, H, Hp, backward=True)
    L.topk_idx.copy_(torch.as_tensor(idx))
    L.gates.copy_(torch.as_tensor(gates))
    L.X.copy_(normal_tensor((R, S, H), 1.0, "bf16", 0, TAG_X, "cuda", slices=R))
    L.W_gu_home.copy_(normal_tensor((E, H, 2 * Hp), H ** -0.5, "bf16", 0, TAG_W, "cuda", slices=E))
    L.W_down_home.copy_(normal_tensor((E, Hp, H), Hp ** -0.5, "bf16", 0, TAG_WD, "cuda", slices=E))
    g = torch.Generator().manual_seed(17)
    dout = torch.randn((R, S, H), generator=g, dtype=torch.float32)
    L.dout.copy_(dout)
    say("mid FFN full size")
    L.forward()
    L.backward()
    torch.cuda.synchronize()
    X = np64(L.X).reshape(-1, H)
    Wgu = L.W_gu_home.cpu().float().numpy()
    Wd = L.W_down_home.cpu().float().numpy()
    ids = np.asarray(idx).reshape(-1, K)
    gf = np.asarray(gates, dtype=np.float64).reshape(-1, K)
    do = dout.numpy().astype(np.float64).reshape(-1, H)
    out = np64(L.out).reshape(-1, H)
    dX = np64(L.dX).reshape(-1, H)
    rng = np.random.default_rng(3)
    for t in rng.choice(R * S, 12, replace=False):
        ref_out = np.zeros(H)
        scale_out = np.zeros(H)
        ref_dx = np.zeros(H)
        scale_dx = np.zeros(H)
        for k in range(K):
            e = ids[t, k]
            wgu, wd = Wgu[e].astype(np.float64), Wd[e].astype(np.float64)
            ygu = bf16_round_np((X[t] @ wgu)[None, :])
            a = bf16_round_np(olayer.swiglu(ygu))
            z = bf16_round_np(a @ wd)[0]
            ref_out += gf[t, k] * z
            scale_out += np.abs(gf[t, k] * z)
            dz = bf16_round_np((np.float32(gates.reshape(-1, K)[t, k]) * do[t].astype(np.float32))[None, :]
                               .astype(np.float64))
            da = bf16_round_np(dz @ wd.T)
            dygu = bf16_round_np(olayer.swiglu_backward(ygu, da))
            term = (dygu @ wgu.T)[0]
            ref_dx += term
            scale_dx += np.abs(term)
        assert np.all(np.abs(out[t] - ref_out) <= 1e-2 * (1 + scale_out)), t
        assert np.all(np.abs(dX[t] - ref_dx) <= 2e-2 * (1 + scale_dx)), t
    # both projections' weight gradients after wgrad + reduce_grad: the whole gradient of three experts
    # (the two with the most slot copies and one without), from the same bf16 intermediates
    p = oplanner.plan(idx, E, B)
    copies = np.bincount(p.slot_expert[p.slot_expert >= 0], minlength=E)
    by_copies = [int(e) for e in np.argsort(-copies, kind="stable") if copies[e] > 0]
    experts = list(dict.fromkeys(by_copies[:2] + [int(np.nonzero(copies == 0)[0][0])]))
    assert copies[experts[0]] > 0
    flat_ids = np.asarray(idx).reshape(-1)
    g32 = np.asarray(gates, dtype=np.float32).reshape(-1)
    do32 = dout.numpy().reshape(-1, H)
    for e in experts:
        say("  FFN weight gradients of expert", e, "copies", int(copies[e]))
        q = np.nonzero(flat_ids == e)[0]
        x = X[q // K]
        wgu, wd = Wgu[e].astype(np.float64), Wd[e].astype(np.float64)
        ygu = bf16_round_np(x @ wgu)
        a = bf16_round_np(olayer.swiglu(ygu))
        dz = bf16_round_np((g32[q][:, None] * do32[q // K]).astype(np.float64))  # float32 product, rounded once
        da = bf16_round_np(dz @ wd.T)
        dygu = bf16_round_np(olayer.swiglu_backward(ygu, da))
        ref_d, ref_gu = a.T @ dz, x.T @ dygu
        got_d, got_gu = np64(L.dW_down_home[e]), np64(L.dW_gu_home[e])
        assert np.all(np.abs(got_d - ref_d) <= 2e-2 * (1 + np.abs(a).T @ np.abs(dz))), f"dW_down[{e}]"
        assert np.all(np.abs(got_gu - ref_gu) <= 2e-2 * (1 + np.abs(x).T @ np.abs(dygu))), f"dW_gate_up[{e}]"
    assert float(L.dW_gu_slots.abs().max()) == 0.0 and float(L.dW_down_slots.abs().max()) == 0.0
