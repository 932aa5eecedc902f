"""Parity of the backward of the data path (combine backward, group-GEMM dgrad, dispatch backward)
against the CPU oracle (GPU).

dYp is the float32 product gate * dout rounded once to the row dtype: the test takes that same
rounding decision in the same precision (float32 multiply, round-to-nearest-even) on the seeded
inputs and requires bit equality.  dgate and dX are float32 sums: |gpu - ref| <= 1e-5 * sum|terms|.
dgrad: bf16 |gpu - ref| <= 1e-2 * (1 + |ref|) against float64 on bf16-rounded inputs, float32 1e-4.
At the mid workload's full size, sampled outputs are checked against the oracle computed one by
one from the generated inputs.
"""
import numpy as np
import pytest
import torch

from oracle import layer as olayer
from oracle import planner as oplanner
from synthetic import WORKLOADS
from synthetic.calibrate import alpha_for
from synthetic.router import TAG_W, TAG_X, normal_tensor, router_output
from tests.gpu_util import (DEV, assert_gemm_close, assert_sum_close, f32, i32, np64, npi, rand_tensor, say)
from tests.plan_checks import random_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import load_balanced_dispatch_amd as mod
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return mod


def scaled_rounded(g: np.ndarray, dout: np.ndarray, dtype) -> torch.Tensor:
    """float32 product g * dout, rounded once to dtype (round to nearest even), on the CPU."""
    prod = torch.as_tensor(np.asarray(g, dtype=np.float32)) * torch.as_tensor(np.asarray(dout, dtype=np.float32))
    return prod.to(dtype)


# ------------------------------------------------------------------ combine backward


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 1408), (torch.bfloat16, 2048), (torch.float32, 256),
                                     (torch.bfloat16, 1024), (torch.bfloat16, 4096), (torch.float32, 1000),
                                     (torch.bfloat16, 13), (torch.float32, 6)])
def test_combine_backward(m, dtype, D):
    rng = np.random.default_rng(100 + D)
    R, E, B, S, K = 4, 16, 4, 150, 4
    topk = random_routing(rng, R, S, K, E, 2.0)
    p = oplanner.plan(topk, E, B)
    d = m.make_dims(R, E, B, S, K)
    Yp = rand_tensor((R * S * K, D), dtype, seed=D + 1)
    dout = rand_tensor((R, S, D), torch.float32, seed=D + 2)
    gates = rng.dirichlet(np.ones(K), size=(R, S)).astype(np.float32)
    dYp = torch.full((R * S * K, D), float("nan"), dtype=dtype, device=DEV)
    dgates = torch.full((R, S, K), float("nan"), dtype=torch.float32, device=DEV)
    say("combine_backward", dtype, D)
    m.moonep_combine_backward(d, D, dout, Yp, i32(p.dest_idx), f32(gates), dYp, dgates)
    torch.cuda.synchronize()
    # dYp: every row written, each equal to the once-rounded float32 product
    do = dout.cpu().numpy()
    want = torch.empty((R * S * K, D), dtype=dtype)
    dflat = p.dest_idx.reshape(R * S, K)
    for k in range(K):
        want[torch.as_tensor(dflat[:, k])] = scaled_rounded(gates.reshape(R * S, K)[:, k:k + 1],
                                                            do.reshape(R * S, D), dtype)
    assert torch.equal(dYp.cpu(), want), "dYp differs from the rounded products"
    # dgates: float32 sums against float64
    y = np64(Yp)
    _, ref = olayer.combine_backward(do.astype(np.float64), y, p.dest_idx, gates)
    _, scale = olayer.combine_backward(np.abs(do.astype(np.float64)), np.abs(y), p.dest_idx, gates)
    assert_sum_close(np64(dgates), ref, scale, 1e-5, "dgates")


# ------------------------------------------------------------------ dgrad


@pytest.mark.parametrize("dtype,R,E,B,S,K,H,Hp", [
    (torch.bfloat16, 2, 4, 2, 300, 2, 256, 192),    # MFMA path: 2+ M tiles per group, partial tiles, 6 k-stages
    (torch.bfloat16, 4, 16, 4, 160, 3, 128, 128),   # MFMA path, many small groups and slots, 128-wide n tile
    (torch.bfloat16, 3, 6, 0, 200, 2, 384, 64),     # MFMA path, no slots, direct reads, 2 n tiles
    (torch.bfloat16, 2, 4, 2, 200, 2, 64, 128),     # MFMA path, one 64-wide n tile (narrow wave layout)
    (torch.bfloat16, 2, 4, 2, 300, 2, 512, 160),    # MFMA path with 128 x 512 tail tiles (N = H a multiple of 512)
    (torch.bfloat16, 3, 6, 1, 170, 3, 1024, 96),    # tail tiles, two 512-wide tail n tiles, direct reads
    (torch.bfloat16, 2, 4, 1, 50, 2, 72, 40),       # generic bf16 path (H % 64 != 0)
    (torch.float32, 4, 16, 4, 64, 2, 128, 256),     # tiny workload shape, float32
    (torch.float32, 2, 6, 1, 37, 3, 33, 65),        # float32, ragged everything
])
def test_group_gemm_dgrad(m, dtype, R, E, B, S, K, H, Hp):
    rng = np.random.default_rng(S * 5 + H)
    topk = random_routing(rng, R, S, K, E, 2.5)
    p = oplanner.plan(topk, E, B)
    W = rand_tensor((E, H, Hp), dtype, seed=22, std=H ** -0.5)
    dYp = rand_tensor((R * S * K, Hp), dtype, seed=21)
    Ws_ref = olayer.prefetch(np64(W), p.slot_expert)
    d = m.make_dims(R, E, B, S, K)
    Ws = torch.as_tensor(Ws_ref, dtype=torch.float32).to(dtype).to(DEV) if B > 0 else None
    dXp = torch.full((R * S * K, H), float("nan"), dtype=dtype, device=DEV)
    ws = torch.empty(m.moonep_group_gemm_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    say("group_gemm_dgrad", dtype, R, E, B, S, K, H, Hp)
    m.moonep_group_gemm_dgrad(d, H, Hp, dYp, W, Ws, i32(p.cu_seqlens), dXp, ws)
    torch.cuda.synchronize()
    ref = olayer.group_gemm_dgrad(np64(dYp), np64(W), Ws_ref, p.cu_seqlens, S * K)
    rel = 1e-2 if dtype == torch.bfloat16 else 1e-4
    assert_gemm_close(np64(dXp), ref, rel, "group_gemm_dgrad")


# ------------------------------------------------------------------ dispatch backward


@pytest.mark.parametrize("dtype,H", [(torch.bfloat16, 2048), (torch.bfloat16, 7168), (torch.float32, 128),
                                     (torch.bfloat16, 13), (torch.float32, 6)])
def test_dispatch_backward(m, dtype, H):
    rng = np.random.default_rng(200 + H)
    R, E, B, S, K = 4, 16, 4, 100, 3
    topk = random_routing(rng, R, S, K, E, 2.0)
    p = oplanner.plan(topk, E, B)
    dXp = rand_tensor((R * S * K, H), dtype, seed=H + 3)
    dX = torch.full((R, S, H), float("nan"), dtype=torch.float32, device=DEV)
    say("dispatch_backward", dtype, H)
    m.moonep_dispatch_backward(m.make_dims(R, E, B, S, K), H, dXp, i32(p.dest_idx), dX)
    torch.cuda.synchronize()
    x = np64(dXp)
    assert_sum_close(np64(dX), olayer.dispatch_backward(x, p.dest_idx), olayer.dispatch_backward(np.abs(x), p.dest_idx),
                     1e-5, "dispatch_backward")


def test_dispatch_backward_of_dispatch_is_k_times_x(m):
    # dispatch_backward(dispatch(X)) = K * X: a sum of K copies of each row
    rng = np.random.default_rng(3)
    R, E, B, S, K, H = 4, 16, 4, 128, 3, 2048
    topk = random_routing(rng, R, S, K, E, 2.0)
    p = oplanner.plan(topk, E, B)
    d = m.make_dims(R, E, B, S, K)
    X = rand_tensor((R, S, H), torch.bfloat16, seed=4)
    Xp = torch.empty((R * S * K, H), dtype=torch.bfloat16, device=DEV)
    dX = torch.empty((R, S, H), dtype=torch.float32, device=DEV)
    say("dispatch round trip")
    m.moonep_dispatch(d, H, X, i32(p.dest_idx), Xp)
    m.moonep_dispatch_backward(d, H, Xp, i32(p.dest_idx), dX)
    torch.cuda.synchronize()
    assert np.array_equal(np64(dX), K * np64(X))  # K small: the float32 sums are exact


# ------------------------------------------------------------------ whole chain


def test_tiny_backward_chain_matches_plain_gradient(m):
    wl = WORKLOADS["tiny_f32"]
    idx, gates = router_output(wl.R, wl.S, wl.E, wl.K, 0, alpha=wl.alpha)
    L = m.MoeLayer(wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp, dtype=torch.float32, backward=True, data_grad=True)
    L.topk_idx.copy_(torch.as_tensor(idx))
    L.gates.copy_(torch.as_tensor(gates))
    L.X.copy_(normal_tensor((wl.R, wl.S, wl.H), 1.0, "f32", 0, TAG_X, "cuda", slices=wl.R))
    L.W_home.copy_(normal_tensor((wl.E, wl.H, wl.Hp), wl.H ** -0.5, "f32", 0, TAG_W, "cuda", slices=wl.E))
    dout = rand_tensor((wl.R, wl.S, wl.Hp), torch.float32, seed=9)
    L.dout.copy_(dout)
    say("tiny backward chain")
    L.forward()
    L.backward_data()
    torch.cuda.synchronize()
    ref_dX, ref_dg = olayer.moe_backward(np64(L.X), np64(L.W_home), idx, gates, np64(dout))
    assert_gemm_close(np64(L.dX), ref_dX, 1e-4, "dX")
    assert_gemm_close(np64(L.dgates), ref_dg, 1e-4, "dgates")


# ------------------------------------------------------------------ full size (mid workload), sampled


class _XpRows:
    """Dispatched rows of X the oracle side reads on demand (row -> its pair's token)."""

    def __init__(self, X, src_of_row, K):
        self.X, self.src, self.K = X, src_of_row, K

    def __getitem__(self, row):
        return self.X[int(self.src[row]) // self.K]


class _RowsOf:
    """dYp rows the oracle side computes on demand: the once-rounded product gate * dout of the row's pair."""

    def __init__(self, src_of_row, gates, dout, K, dtype):
        self.src, self.g, self.do, self.K, self.dtype = src_of_row, gates.reshape(-1), dout, K, dtype

    def __getitem__(self, row):
        q = int(self.src[row])
        return scaled_rounded(self.g[q:q + 1], self.do[q // self.K], self.dtype).float().numpy().astype(np.float64)


def test_full_mid_backward_data_sampled(m):
    wl = WORKLOADS["mid_fwd"]
    idx, gates = router_output(wl.R, wl.S, wl.E, wl.K, 0, alpha=alpha_for(wl, 0, 1.0))
    L = m.MoeLayer(wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp, backward=True, data_grad=True)
    L.topk_idx.copy_(torch.as_tensor(idx))
    L.gates.copy_(torch.as_tensor(gates))
    L.X.copy_(normal_tensor((wl.R, wl.S, wl.H), 1.0, "bf16", 0, TAG_X, "cuda", slices=wl.R))
    L.W_home.copy_(normal_tensor((wl.E, wl.H, wl.Hp), wl.H ** -0.5, "bf16", 0, TAG_W, "cuda", slices=wl.E))
    g = torch.Generator().manual_seed(31)
    dout = torch.randn((wl.R, wl.S, wl.Hp), generator=g, dtype=torch.float32)
    L.dout.copy_(dout)
    say("full mid backward data")
    L.forward()
    L.backward_data()
    torch.cuda.synchronize()
    p = oplanner.plan(idx, wl.E, wl.B)
    assert np.array_equal(npi(L.dest_idx), p.dest_idx)
    X = L.X.cpu().float().numpy().astype(np.float64).reshape(-1, wl.H)
    W = L.W_home.cpu().float().numpy().astype(np.float64)
    Ws = olayer.prefetch(W, p.slot_expert)
    do = dout.numpy().reshape(-1, wl.Hp)
    K, P = wl.K, wl.P
    rng = np.random.default_rng(5)
    # dY rows of sampled pairs: bit equal to the rounded products
    pairs = rng.choice(wl.N, 256, replace=False)
    rows = p.dest_idx.reshape(-1)[pairs]
    want = scaled_rounded(gates.reshape(-1)[pairs][:, None], do[pairs // K], torch.bfloat16)
    assert torch.equal(L.dY[torch.as_tensor(rows, device=DEV)].cpu(), want)
    # dgates of sampled tokens: <dout, Yp row> with Yp from the oracle (GPU Yp is bf16-rounded: GEMM bound)
    toks = rng.choice(wl.R * wl.S, 64, replace=False)
    got_dg = np64(L.dgates).reshape(-1, K)[toks]
    for i, t in enumerate(toks):
        r_ids = p.dest_idx.reshape(-1, K)[t]
        y = olayer.group_gemm(_XpRows(X, p.src_of_row, K), W, Ws, p.cu_seqlens, P, rows=r_ids)
        ref = y @ do[t]
        scale = np.abs(y) @ np.abs(do[t])
        assert np.all(np.abs(got_dg[i] - ref) <= 1e-2 * (1 + scale)), (t, got_dg[i], ref)
    # dXp rows of sampled pairs and dX of sampled tokens, from the oracle's dgrad of the rounded dYp
    dyp = _RowsOf(p.src_of_row, gates, do, K, torch.bfloat16)
    ref_rows = olayer.group_gemm_dgrad(dyp, W, Ws, p.cu_seqlens, P, rows=rows)
    assert_gemm_close(np64(L.dXp[torch.as_tensor(rows, device=DEV)]), ref_rows, 1e-2, "dXp (full mid)")
    got_dX = np64(L.dX).reshape(-1, wl.H)
    for t in toks[:16]:
        r_ids = p.dest_idx.reshape(-1, K)[t]
        terms = olayer.group_gemm_dgrad(dyp, W, Ws, p.cu_seqlens, P, rows=r_ids)
        ref = terms.sum(axis=0)
        bound = 1e-2 * (K + np.abs(terms).sum(axis=0))
        assert np.all(np.abs(got_dX[t] - ref) <= bound), t
