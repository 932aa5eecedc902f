"""The whole step through the C ABI on seeded random shapes: plan -> prefetch -> dispatch -> group GEMM
-> combine -> wgrad -> reduce_grad (MoeLayer), every intermediate checked against the oracle chain.

The shapes mix the GEMMs' MFMA and generic paths (H % 32 / 128, H' % 64), narrow last tiles, no slots
(B = 0, every copy a direct read), one expert per rank, K = 1, float32, and a routing where the same K
experts are every token's top-K.  The oracle runs the whole chain in float64 from the same seeded
inputs (generated on the host; nothing the GPU computed is fed to it), and every stage's output is
compared: plan, indices and moved rows bit for bit; the group GEMM and wgrad + reduce_grad within
rel (1 + |ref|) with rel = 1e-2 for bf16 and 1e-4 for float32; combine within rel (1 + sum_k g |y|),
which also covers its input's rounding in the GEMM stage; consumed slots zeroed.
"""
import numpy as np
import pytest
import torch

from oracle import layer as olayer
from oracle import planner as oplanner
from tests.gpu_util import DEV, assert_gemm_close, np64, npi, say
from tests.plan_checks import random_routing

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def m():
    import load_balanced_dispatch_amd as mod
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return mod

# seed, dtype, R, E, B, S, K, H, Hp, routing ("skew:<s>", or "hot": every token picks experts 0..K-1)
CASES = [
    (1, BF, 2, 4, 2, 300, 2, 128, 192, "skew:2.0"),   # MFMA forward and wgrad; one 192-wide n tile
    (2, BF, 4, 8, 0, 200, 3, 256, 320, "skew:3.0"),   # no slots: overflow read directly; 256 + 64 n tiles
    (3, BF, 3, 3, 1, 150, 1, 64, 128, "skew:1.5"),    # one expert per rank, K = 1; wgrad generic (H % 128)
    (4, BF, 4, 16, 4, 128, 4, 384, 64, "skew:4.0"),   # strong skew, 64-wide n tile, 3 h tiles
    (5, BF, 2, 6, 3, 100, 2, 96, 72, "skew:1.0"),     # generic GEMMs (H' % 64 != 0)
    (6, F32, 2, 4, 2, 64, 2, 64, 64, "skew:2.0"),     # float32 throughout
    (7, BF, 8, 16, 1, 64, 3, 128, 128, "hot"),        # three experts take every pair: direct reads
]


def host_rand(shape, dtype, seed, std=1.0):
    """Seeded host tensor rounded to dtype: the oracle takes it, the GPU a copy."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(dtype)


def routing(rng, R, S, K, E, spec):
    if spec == "hot":
        return np.broadcast_to(np.arange(K, dtype=np.int64), (R, S, K)).copy()
    return random_routing(rng, R, S, K, E, float(spec.split(":")[1]))


@pytest.mark.parametrize("seed,dtype,R,E,B,S,K,H,Hp,spec", CASES)
def test_step_chain_matches_oracle(m, seed, dtype, R, E, B, S, K, H, Hp, spec):
    rng = np.random.default_rng(900 + seed)
    topk = routing(rng, R, S, K, E, spec)
    logits = rng.standard_normal((R, S, K))
    gates = (np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)).astype(np.float32)
    N, P = R * S * K, S * K
    Xh = host_rand((R, S, H), dtype, 40 + seed)
    Wh = host_rand((E, H, Hp), dtype, 50 + seed, std=H ** -0.5)
    dYh = host_rand((N, Hp), dtype, 60 + seed)
    L = m.MoeLayer(R, E, B, S, K, H, Hp, dtype=dtype, backward=True)
    L.topk_idx.copy_(torch.as_tensor(topk, dtype=torch.int32))
    L.gates.copy_(torch.as_tensor(gates))
    L.X.copy_(Xh)
    L.W_home.copy_(Wh)
    L.dY.copy_(dYh)
    say("step chain", seed, dtype, R, E, B, S, K, H, Hp, spec)
    L.forward()
    L.backward()
    torch.cuda.synchronize()

    # plan: bit for bit
    p = oplanner.plan(topk, E, B)
    assert np.array_equal(npi(L.expert_counts), p.expert_counts)
    assert np.array_equal(npi(L.cu_seqlens), p.cu_seqlens)
    assert np.array_equal(npi(L.dest_idx), p.dest_idx)
    assert np.array_equal(npi(L.stats), p.stats)
    if B > 0:
        assert np.array_equal(npi(L.slot_expert), p.slot_expert)
    if spec == "hot" or B == 0:
        assert p.stats[2] > 0  # the case exercises direct reads

    # moved rows: bit for bit
    X = Xh.float().numpy().astype(np.float64)
    W = Wh.float().numpy().astype(np.float64)
    dY = dYh.float().numpy().astype(np.float64)
    Xp = olayer.dispatch(X, p.dest_idx)
    assert np.array_equal(np64(L.Xp), Xp)
    Ws = olayer.prefetch(W, p.slot_expert) if B > 0 else None
    if B > 0:
        for r in range(R):
            for j in range(B):
                if p.slot_expert[r, j] >= 0:
                    assert np.array_equal(np64(L.W_slots[r, j]), Ws[r, j])

    # group GEMM
    rel = 1e-2 if dtype == BF else 1e-4
    Yp = olayer.group_gemm(Xp, W, Ws, p.cu_seqlens, P)
    assert_gemm_close(np64(L.Yp), Yp, rel, "group GEMM")

    # combine: the GEMM stage's error on each gathered row, weighted by the gates, plus float32 sums
    g64 = gates.astype(np.float64)
    ref = olayer.combine(Yp, p.dest_idx, g64)
    bound = rel * (1.0 + olayer.combine_abs(Yp, p.dest_idx, g64))
    err = np.abs(np64(L.out) - ref)
    assert (err <= bound).all(), f"combine: worst excess {np.max(err - bound)!r}"

    # wgrad + reduce_grad from zero gradients: slots consumed and zeroed, home holds the expert sum
    dWh = np.zeros((E, H, Hp))
    dWs = np.zeros((R, B, H, Hp))
    olayer.wgrad(Xp, dY, p.cu_seqlens, P, dWh, dWs)
    olayer.reduce_grad(p.slot_expert, dWh, dWs)
    assert_gemm_close(np64(L.dW_home), dWh, rel, "wgrad + reduce_grad (home)")
    if B > 0:
        assert not np.any(np64(L.dW_slots)), "reduce_grad leaves every slot zero"
