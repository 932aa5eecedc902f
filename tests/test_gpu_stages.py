"""Per-call parity of the HIP library against the CPU oracle on small inputs that still span
several tiles and ragged tails (GPU).

Integers and copies must match bit for bit; bf16 GEMMs |gpu-ref| <= 1e-2*(1+|ref|)
against float64 on the bf16-rounded inputs; float32 GEMMs 1e-4*(1+|ref|); combine
1e-5 * sum|g*y|; reduce_grad bitwise equal to float32 additions in rank order.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import layer as olayer
from oracle import planner as oplanner
from tests.gpu_util import (DEV, assert_gemm_close, assert_sum_close, f32, i32, np64, npi, rand_tensor, say)
from tests.plan_checks import check_plan_invariants, random_routing

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def m():
    import load_balanced_dispatch_amd as mod
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return mod


def gpu_plan(m, topk, E, B, src=True, planner="prefix"):
    topk = np.asarray(topk)
    R, S, K = topk.shape
    d = m.make_dims(R, E, B, S, K)
    out = dict(
        counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
        maxvio=torch.full((1,), -7.0, dtype=torch.float64, device=DEV),
        cu=torch.full((R, E + B + 1), -7, dtype=torch.int32, device=DEV),
        slots=torch.full((R, B), -7, dtype=torch.int32, device=DEV) if B > 0 else None,
        dest=torch.full((R, S, K), -7, dtype=torch.int32, device=DEV),
        src=torch.full((R * S * K,), -7, dtype=torch.int32, device=DEV) if src else None,
        stats=torch.full((4,), -7, dtype=torch.int32, device=DEV),
    )
    ws = torch.full((max(1, m.moonep_plan_workspace_bytes(d)),), 0xAB, dtype=torch.uint8, device=DEV)
    m.moonep_plan_ex(d, planner, i32(topk), out["counts"], out["maxvio"], out["cu"], out["slots"], out["dest"],
                     out["src"], out["stats"], ws)
    torch.cuda.synchronize()
    return d, out


def assert_plan_equal(out, p, B):
    assert npi(out["counts"]).tolist() == p.expert_counts.tolist()
    assert float(out["maxvio"].item()) == p.maxvio  # same float64 expression on both sides
    assert np.array_equal(npi(out["cu"]), p.cu_seqlens)
    if B > 0:
        assert np.array_equal(npi(out["slots"]), p.slot_expert)
    assert np.array_equal(npi(out["dest"]), p.dest_idx)
    if out["src"] is not None:
        assert np.array_equal(npi(out["src"]), p.src_of_row)
    assert npi(out["stats"]).tolist() == p.stats.tolist()


# ------------------------------------------------------------------ planner


@pytest.mark.parametrize("name", ["plan_example1.json", "plan_example2.json"])
def test_plan_hand_worked_examples(m, name):
    g = json.load(open(os.path.join(GOLD, name)))
    say("plan golden", name)
    _, out = gpu_plan(m, g["topk_idx"], g["E"], g["B"])
    assert npi(out["cu"]).tolist() == g["cu_seqlens"]
    assert npi(out["dest"]).tolist() == g["dest_idx"]
    assert npi(out["stats"]).tolist() == g["stats"]
    assert npi(out["slots"]).tolist() == g["slot_expert"]
    assert abs(out["maxvio"].item() - g["maxvio_num"] / g["maxvio_den"]) < 1e-15


def small_plan_case(seed):
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.integers(1, 9))
    per = int(rng.integers(1, 9))
    E = R * per
    K = int(rng.integers(1, min(E, 8) + 1))
    S = int(rng.integers(1, 400))
    B = int(rng.integers(0, per + 3))
    return random_routing(rng, R, S, K, E, float(rng.uniform(0, 3))), E, B


@pytest.mark.parametrize("seed", range(30))
def test_plan_random_bit_exact(m, seed):
    topk, E, B = small_plan_case(seed)
    say("plan random", seed, topk.shape, E, B)
    _, out = gpu_plan(m, topk, E, B)
    p = oplanner.plan(topk, E, B)
    assert_plan_equal(out, p, B)
    if topk.size <= 4000:
        check_plan_invariants(topk, E, B, npi(out["cu"]), npi(out["slots"]) if B else np.zeros((topk.shape[0], 0)),
                              npi(out["dest"]), npi(out["src"]), npi(out["stats"]))


@pytest.mark.parametrize("R,E,B,S,K", [
    (4, 16, 4, 64, 2),       # tiny workload shape
    (3, 12, 0, 777, 3),      # no slots: every copy is a direct read
    (1, 5, 2, 1000, 5),      # one rank: nothing can move, K = E
    (8, 64, 8, 2731, 6),     # several count/emit blocks with a ragged last block
    (16, 64, 1, 300, 4),     # many ranks, one slot
    # largest tables the planner's blocks hold in LDS: emit 8E + 3R ints = 152 KiB
    (2048, 4096, 2, 2, 2),
    (512, 4096, 8, 8, 4),    # E at its limit with many blocks of the count/emit grids
    (2048, 2048, 3, 3, 5),   # 2048 ranks of one expert each
    (2, 4096, 4, 3, 1500),   # K above the 1024 pairs of a block: one token per block
])
def test_plan_shapes_bit_exact(m, R, E, B, S, K):
    rng = np.random.default_rng(R * 1000 + S)
    topk = random_routing(rng, R, S, K, E, 2.0)
    say("plan shape", R, E, B, S, K)
    _, out = gpu_plan(m, topk, E, B)
    assert_plan_equal(out, oplanner.plan(topk, E, B), B)


@pytest.mark.parametrize("name", ["plan_example1_mincopy.json", "plan_example2_mincopy.json",
                                  "plan_example4_tie.json"])
def test_plan_mincopy_hand_worked_examples(m, name):
    g = json.load(open(os.path.join(GOLD, name)))
    say("plan mincopy golden", name)
    _, out = gpu_plan(m, g["topk_idx"], g["E"], g["B"], planner="mincopy")
    assert npi(out["cu"]).tolist() == g["cu_seqlens"]
    assert npi(out["dest"]).tolist() == g["dest_idx"]
    assert npi(out["stats"]).tolist() == g["stats"]
    assert npi(out["slots"]).tolist() == g["slot_expert"]


def test_plan_mincopy_example3_counts(m):
    g = json.load(open(os.path.join(GOLD, "plan_example3_counts.json")))
    lst = np.repeat(np.arange(g["E"]), g["expert_counts"])  # token t takes the ids at t and t + R*S
    T = g["R"] * g["S"]
    topk = np.stack([lst[k * T:(k + 1) * T] for k in range(g["K"])], axis=1).reshape(g["R"], g["S"], g["K"])
    say("plan mincopy example 3")
    _, out = gpu_plan(m, topk, g["E"], g["B"], planner="mincopy")
    assert npi(out["stats"]).tolist() == g["mincopy"]["stats"]
    assert npi(out["slots"])[3].tolist() == g["mincopy"]["slot_expert_rank3"]
    assert_plan_equal(out, oplanner.plan(topk, g["E"], g["B"], planner="mincopy"), g["B"])


@pytest.mark.parametrize("seed", range(30))
def test_plan_mincopy_random_bit_exact(m, seed):
    topk, E, B = small_plan_case(seed)
    say("plan mincopy random", seed, topk.shape, E, B)
    _, out = gpu_plan(m, topk, E, B, planner="mincopy")
    p = oplanner.plan(topk, E, B, planner="mincopy")
    assert_plan_equal(out, p, B)
    if topk.size <= 4000:
        check_plan_invariants(topk, E, B, npi(out["cu"]), npi(out["slots"]) if B else np.zeros((topk.shape[0], 0)),
                              npi(out["dest"]), npi(out["src"]), npi(out["stats"]), planner="mincopy")


@pytest.mark.parametrize("R,E,B,S,K", [
    (4, 16, 4, 64, 2), (3, 12, 0, 777, 3), (1, 5, 2, 1000, 5), (8, 64, 8, 2731, 6), (16, 64, 1, 300, 4),
    (2048, 4096, 2, 2, 2), (512, 4096, 8, 8, 4), (2048, 2048, 3, 3, 5), (2, 4096, 4, 3, 1500),
    (2, 512, 8, 500, 16),    # 256 experts per rank: the keep count of each walks its rank's 256 counts
])
def test_plan_mincopy_shapes_bit_exact(m, R, E, B, S, K):
    rng = np.random.default_rng(R * 1000 + S + 1)
    topk = random_routing(rng, R, S, K, E, 2.5)
    say("plan mincopy shape", R, E, B, S, K)
    _, out = gpu_plan(m, topk, E, B, planner="mincopy")
    assert_plan_equal(out, oplanner.plan(topk, E, B, planner="mincopy"), B)


def test_plan_mincopy_counts_invalid_and_repeated_ids(m):
    rng = np.random.default_rng(4)
    topk = random_routing(rng, 2, 50, 3, 8, 1.5)
    topk[0, 3, 1] = 8       # out of range
    topk[1, 7, 0] = -2      # negative
    topk[1, 9, 2] = topk[1, 9, 0]  # repeated within a token
    say("plan mincopy invalid ids")
    _, out = gpu_plan(m, topk, 8, 2, planner="mincopy")
    assert npi(out["stats"])[3] == 3
    dest = npi(out["dest"])
    assert dest[0, 3, 1] == -1 and dest[1, 7, 0] == -1
    valid = dest[dest >= 0]
    assert len(np.unique(valid)) == len(valid) and valid.max() < topk.size


def test_plan_empty_routing(m):
    say("plan empty")
    topk = np.zeros((4, 0, 2), dtype=np.int64)
    d = m.make_dims(4, 8, 2, 0, 2)
    counts = torch.full((8,), -1, dtype=torch.int32, device=DEV)
    mv = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    cu = torch.full((4, 11), -1, dtype=torch.int32, device=DEV)
    slots = torch.full((4, 2), -5, dtype=torch.int32, device=DEV)
    stats = torch.full((4,), -1, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(1, m.moonep_plan_workspace_bytes(d)), dtype=torch.uint8, device=DEV)
    dummy = torch.zeros(1, dtype=torch.int32, device=DEV)
    from load_balanced_dispatch_amd import _lib
    rc = _lib.lib().moonep_plan(d, dummy.data_ptr(), counts.data_ptr(), mv.data_ptr(), cu.data_ptr(),
                                slots.data_ptr(), dummy.data_ptr(), None, stats.data_ptr(), ws.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert npi(counts).tolist() == [0] * 8
    assert mv.item() == 0.0
    assert np.all(npi(cu) == 0)
    assert np.all(npi(slots) == -1)
    assert npi(stats).tolist() == [0, 0, 0, 0]


def test_plan_counts_invalid_and_repeated_ids(m):
    rng = np.random.default_rng(3)
    topk = random_routing(rng, 2, 50, 3, 8, 1.0)
    topk[0, 3, 1] = 8       # out of range
    topk[1, 7, 0] = -2      # negative
    topk[1, 9, 2] = topk[1, 9, 0]  # repeated within a token
    say("plan invalid ids")
    _, out = gpu_plan(m, topk, 8, 2)
    assert npi(out["stats"])[3] == 3
    dest = npi(out["dest"])
    assert dest[0, 3, 1] == -1 and dest[1, 7, 0] == -1
    valid = dest[dest >= 0]
    assert len(np.unique(valid)) == len(valid) and valid.max() < topk.size


# ------------------------------------------------------------------ dispatch / prefetch


@pytest.mark.parametrize("dtype,H", [(torch.bfloat16, 2048), (torch.bfloat16, 7168), (torch.float32, 128),
                                     (torch.float32, 7), (torch.bfloat16, 5)])
def test_dispatch_bit_exact(m, dtype, H):
    rng = np.random.default_rng(H)
    R, E, B, S, K = 4, 16, 3, 97, 4
    topk = random_routing(rng, R, S, K, E, 2.0)
    p = oplanner.plan(topk, E, B)
    X = rand_tensor((R, S, H), dtype, seed=H)
    Xp = torch.full((R * S * K, H), float("nan"), dtype=dtype, device=DEV)
    say("dispatch", dtype, H)
    m.moonep_dispatch(m.make_dims(R, E, B, S, K), H, X, i32(p.dest_idx), Xp)
    torch.cuda.synchronize()
    ref = olayer.dispatch(X.cpu().float().numpy(), p.dest_idx)
    assert np.array_equal(Xp.cpu().float().numpy(), ref)  # also proves every row was written (no NaN)


@pytest.mark.parametrize("dtype,H,Hp", [(torch.bfloat16, 256, 384), (torch.float32, 24, 40), (torch.bfloat16, 3, 5)])
def test_prefetch_bit_exact_and_unused_slots_untouched(m, dtype, H, Hp):
    rng = np.random.default_rng(Hp)
    R, E, B, S, K = 4, 16, 3, 64, 3
    topk = random_routing(rng, R, S, K, E, 3.0)
    p = oplanner.plan(topk, E, B)
    assert p.stats[1] > 0
    W = rand_tensor((E, H, Hp), dtype, seed=5)
    Ws = torch.full((R, B, H, Hp), 7.0, dtype=dtype, device=DEV)
    say("prefetch", dtype, H, Hp)
    m.moonep_prefetch(m.make_dims(R, E, B, S, K), H, Hp, W, i32(p.slot_expert), Ws)
    torch.cuda.synchronize()
    ref = olayer.prefetch(W.cpu().float().numpy(), p.slot_expert, np.full((R, B, H, Hp), 7.0))
    assert np.array_equal(Ws.cpu().float().numpy(), ref)


def test_prefetch_several_items_per_block(m):
    # expert 0 is in every token's top-2, so all 7 other ranks take a copy of it: 7 slots of
    # 2047 x 4080 bf16 (1020 items of 1024 vectors each, the last one partial) are 3-4 items for each
    # of the persistent blocks, which load one item ahead of their stores
    R, E, B, S, K, H, Hp = 8, 8, 2, 32, 2, 2047, 4080
    rng = np.random.default_rng(11)
    topk = np.zeros((R, S, K), dtype=np.int32)
    topk[:, :, 1] = rng.integers(1, E, size=(R, S))
    p = oplanner.plan(topk, E, B)
    used = [(r, j, int(p.slot_expert[r, j])) for r in range(R) for j in range(B) if p.slot_expert[r, j] >= 0]
    assert sum(e == 0 for _, _, e in used) == R - 1
    W = rand_tensor((E, H, Hp), torch.bfloat16, seed=13)
    Ws = torch.full((R, B, H, Hp), 7.0, dtype=torch.bfloat16, device=DEV)
    say("prefetch several items per block", R, E, B, H, Hp)
    m.moonep_prefetch(m.make_dims(R, E, B, S, K), H, Hp, W, i32(p.slot_expert), Ws)
    torch.cuda.synchronize()
    for r in range(R):  # W_slots[r, j] == W_home[slot_expert[r, j]] bit for bit; unused slots untouched
        for j in range(B):
            e = int(p.slot_expert[r, j])
            want = W[e] if e >= 0 else torch.full((H, Hp), 7.0, dtype=torch.bfloat16, device=DEV)
            assert torch.equal(Ws[r, j].view(torch.int16), want.view(torch.int16)), (r, j, e)


# ------------------------------------------------------------------ group GEMM


@pytest.mark.parametrize("dtype,R,E,B,S,K,H,Hp", [
    (torch.bfloat16, 2, 4, 2, 300, 2, 192, 256),    # MFMA path: 2+ M tiles per group, partial tiles, 2 N tiles
    (torch.bfloat16, 4, 16, 4, 160, 3, 128, 128),   # MFMA path, many small groups and slots
    (torch.bfloat16, 3, 6, 0, 200, 2, 64, 384),     # MFMA path, no slots, direct reads
    (torch.bfloat16, 2, 4, 2, 200, 2, 128, 320),    # MFMA path, 64-wide last n tile (narrow wave layout)
    (torch.bfloat16, 2, 4, 2, 300, 2, 160, 512),    # MFMA path with 128 x 512 tail tiles (N a multiple of 512)
    (torch.bfloat16, 3, 6, 1, 170, 3, 96, 1024),    # tail tiles, two 512-wide tail n tiles, direct reads
    (torch.bfloat16, 2, 4, 1, 50, 2, 40, 72),       # generic bf16 path (H % 64 != 0)
    (torch.float32, 4, 16, 4, 64, 2, 128, 256),     # tiny workload shape, float32
    (torch.float32, 2, 6, 1, 37, 3, 33, 65),        # float32, ragged everything
])
def test_group_gemm(m, dtype, R, E, B, S, K, H, Hp):
    rng = np.random.default_rng(S * 7 + H)
    topk = random_routing(rng, R, S, K, E, 2.5)
    p = oplanner.plan(topk, E, B)
    X = rand_tensor((R, S, H), dtype, seed=11)
    W = rand_tensor((E, H, Hp), dtype, seed=12, std=H ** -0.5)
    Xp_ref = olayer.dispatch(X.cpu().float().numpy().astype(np.float64), p.dest_idx)
    Ws_ref = olayer.prefetch(W.cpu().float().numpy().astype(np.float64), p.slot_expert)
    d = m.make_dims(R, E, B, S, K)
    Xp = torch.as_tensor(Xp_ref, dtype=torch.float32).to(dtype).to(DEV)
    Ws = torch.as_tensor(Ws_ref, dtype=torch.float32).to(dtype).to(DEV) if B > 0 else None
    Yp = torch.full((R * S * K, Hp), float("nan"), dtype=dtype, device=DEV)
    ws = torch.empty(m.moonep_group_gemm_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    say("group_gemm", dtype, R, E, B, S, K, H, Hp)
    m.moonep_group_gemm(d, H, Hp, Xp, W, Ws, i32(p.cu_seqlens), Yp, ws)
    torch.cuda.synchronize()
    ref = olayer.group_gemm(Xp_ref, W.cpu().float().numpy().astype(np.float64), Ws_ref, p.cu_seqlens, S * K)
    rel = 1e-2 if dtype == torch.bfloat16 else 1e-4
    assert_gemm_close(np64(Yp), ref, rel, "group_gemm")


@pytest.mark.parametrize("dgrad", [False, True])
def test_group_gemm_tail_tile_boundaries(m, dgrad):
    """Groups whose last 256-row m-tile holds exactly 1, 127, 128 (a 128 x 512 tail tile) or 129 and 256
    (a full tile) rows, with and without full m-tiles before them, on an output width that is a multiple
    of 512 (tail tiles on) and on one that is not (off); cu_seqlens are set by hand, every row checked."""
    R, E, B, K = 2, 8, 2, 1
    sizes = [[128, 129, 1, 384, 385, 0, 256, 127, 0, 2],   # rank 0: home groups 0..7, then 2 slot groups
             [512 + 128, 0, 200, 1, 0, 257, 128, 0, 5, 130]]  # rank 1
    P = max(sum(r) for r in sizes)
    for r, pad in ((0, 5), (1, 1)):  # fill each rank to P rows in one of its empty groups
        sizes[r][pad] += P - sum(sizes[r])
    cu = np.zeros((R, E + B + 1), dtype=np.int64)
    for r in range(R):
        cu[r, 1:] = np.cumsum(sizes[r])
    assert (cu[:, -1] == P).all()
    S = P // K
    d = m.make_dims(R, E, B, S, K)
    for K_, N_ in ((96, 512), (64, 1024), (96, 768)):
        H, Hp = (N_, K_) if dgrad else (K_, N_)
        A = rand_tensor((R * P, K_), torch.bfloat16, seed=N_ + K_)
        W = rand_tensor((E, H, Hp), torch.bfloat16, seed=N_ + 1, std=H ** -0.5)
        Ws = rand_tensor((R, B, H, Hp), torch.bfloat16, seed=N_ + 2, std=H ** -0.5)
        C = torch.full((R * P, N_), float("nan"), dtype=torch.bfloat16, device=DEV)
        ws = torch.empty(m.moonep_group_gemm_workspace_bytes(d), dtype=torch.uint8, device=DEV)
        say("group_gemm tail boundaries", "dgrad" if dgrad else "fwd", H, Hp)
        f = m.moonep_group_gemm_dgrad if dgrad else m.moonep_group_gemm
        f(d, H, Hp, A, W, Ws, i32(cu), C, ws)
        torch.cuda.synchronize()
        A64, W64, Ws64 = (np.asarray(t.cpu().float().numpy(), dtype=np.float64) for t in (A, W, Ws))
        g = olayer.group_gemm_dgrad if dgrad else olayer.group_gemm
        ref = g(A64, W64, Ws64, cu, P)
        assert_gemm_close(np64(C), ref, 1e-2, f"tail boundaries {'dgrad' if dgrad else 'fwd'} N={N_}")


# ------------------------------------------------------------------ combine


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 1408), (torch.bfloat16, 2048), (torch.float32, 256),
                                     (torch.bfloat16, 13), (torch.float32, 6)])
def test_combine(m, dtype, D):
    rng = np.random.default_rng(D)
    R, E, B, S, K = 4, 16, 4, 150, 4
    topk = random_routing(rng, R, S, K, E, 2.0)
    p = oplanner.plan(topk, E, B)
    Yp = rand_tensor((R * S * K, D), dtype, seed=D)
    gates = rng.dirichlet(np.ones(K), size=(R, S)).astype(np.float32)
    out = torch.full((R, S, D), float("nan"), dtype=torch.float32, device=DEV)
    say("combine", dtype, D)
    m.moonep_combine(m.make_dims(R, E, B, S, K), D, Yp, i32(p.dest_idx), f32(gates), out)
    torch.cuda.synchronize()
    y = np64(Yp)
    ref = olayer.combine(y, p.dest_idx, gates)
    scale = olayer.combine_abs(y, p.dest_idx, gates)
    assert_sum_close(np64(out), ref, scale, 1e-5, "combine")


def test_combine_dispatch_round_trip(m):
    # combine(dispatch(X)) = X * sum_k gates at the [S, H] shape
    rng = np.random.default_rng(1)
    R, E, B, S, K, H = 4, 16, 4, 128, 2, 2048
    topk = random_routing(rng, R, S, K, E, 2.0)
    p = oplanner.plan(topk, E, B)
    d = m.make_dims(R, E, B, S, K)
    X = rand_tensor((R, S, H), torch.bfloat16, seed=2)
    gates = rng.dirichlet(np.ones(K), size=(R, S)).astype(np.float32)
    Xp = torch.empty((R * S * K, H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((R, S, H), dtype=torch.float32, device=DEV)
    say("round trip")
    m.moonep_dispatch(d, H, X, i32(p.dest_idx), Xp)
    m.moonep_combine(d, H, Xp, i32(p.dest_idx), f32(gates), out)
    torch.cuda.synchronize()
    x = np64(X)
    ref = x * gates.astype(np.float64).sum(-1, keepdims=True)
    assert_sum_close(np64(out), ref, np.abs(ref) + 1e-30, 1e-5, "round trip")


# ------------------------------------------------------------------ wgrad / reduce_grad


@pytest.mark.parametrize("dtype,R,E,B,S,K,H,Hp", [
    (torch.bfloat16, 2, 4, 2, 300, 2, 256, 256),    # MFMA path, several 64-row chunks, ragged segments
    (torch.bfloat16, 4, 8, 1, 100, 3, 512, 128),    # MFMA path with direct reads (B=1)
    (torch.bfloat16, 3, 6, 0, 90, 2, 256, 384),     # MFMA path, no slots
    (torch.bfloat16, 72, 72, 1, 24, 4, 128, 64),    # MFMA path, home jobs read on ranks of two 64-rank words
    (torch.bfloat16, 520, 520, 0, 8, 2, 128, 64),   # MFMA path, ranks past the 512 whose bounds sit in LDS
    (torch.bfloat16, 2, 4, 1, 40, 2, 40, 72),       # generic bf16
    (torch.float32, 4, 16, 4, 64, 2, 128, 256),     # float32
    (torch.float32, 2, 6, 1, 70, 3, 72, 100),       # float32, partial 64 x 64 tiles in both H and H'
])
def test_wgrad_accumulates(m, dtype, R, E, B, S, K, H, Hp):
    rng = np.random.default_rng(S + H)
    topk = random_routing(rng, R, S, K, E, 2.5)
    p = oplanner.plan(topk, E, B)
    N = R * S * K
    Xp = rand_tensor((N, H), dtype, seed=21)
    dY = rand_tensor((N, Hp), dtype, seed=22)
    init_h = np.asarray(rand_tensor((E, H, Hp), torch.float32, seed=23).cpu(), dtype=np.float64)
    init_s = np.asarray(rand_tensor((R, B, H, Hp), torch.float32, seed=24).cpu(), dtype=np.float64)
    dWh = f32(init_h)
    dWs = f32(init_s) if B > 0 else None
    say("wgrad", dtype, R, E, B, S, K, H, Hp)
    d = m.make_dims(R, E, B, S, K)
    ws = torch.full((m.moonep_wgrad_workspace_bytes(d),), 0xCD, dtype=torch.uint8, device=DEV)
    m.moonep_wgrad(d, H, Hp, Xp, dY, i32(p.cu_seqlens), dWh, dWs, ws)
    torch.cuda.synchronize()
    rh, rs = init_h.copy(), init_s.copy()
    olayer.wgrad(np64(Xp), np64(dY), p.cu_seqlens, S * K, rh, rs)
    rel = 1e-2 if dtype == torch.bfloat16 else 1e-4
    assert_gemm_close(np64(dWh), rh, rel, "wgrad home")
    if B > 0:
        assert_gemm_close(np64(dWs), rs, rel, "wgrad slots")
        # slots no group used keep their initial contents exactly
        for r in range(R):
            for j in range(B):
                if p.cu_seqlens[r, E + j + 1] == p.cu_seqlens[r, E + j]:
                    assert np.array_equal(np64(dWs[r, j]), init_s[r, j])


# the last three have R*B = 128 or 200 slots: the per-block slot lists are built 64 slots per round,
# with copies of one expert in several rounds
@pytest.mark.parametrize("R,E,B,H,Hp", [(8, 64, 8, 64, 44), (4, 16, 4, 3, 5), (8, 32, 4, 128, 256),
                                        (16, 64, 8, 16, 24), (20, 40, 10, 32, 20), (32, 64, 4, 16, 16)])
def test_reduce_grad_rank_order_bitwise(m, R, E, B, H, Hp):
    rng = np.random.default_rng(E)
    S, K = 80, 4
    topk = random_routing(rng, R, S, K, E, 3.0)
    p = oplanner.plan(topk, E, B)
    assert p.stats[1] > 0
    hs = rand_tensor((E, H, Hp), torch.float32, seed=31)
    ss = rand_tensor((R, B, H, Hp), torch.float32, seed=32) * 1e3
    ref_h32 = hs.cpu().numpy().copy()
    ref_s32 = ss.cpu().numpy().copy()
    olayer.reduce_grad(p.slot_expert, ref_h32, ref_s32, dtype=np.float32)
    ref_h64 = hs.cpu().numpy().astype(np.float64)
    ref_s64 = ss.cpu().numpy().astype(np.float64)
    scale_h = np.abs(ref_h64).copy()
    olayer.reduce_grad(p.slot_expert, ref_h64, ref_s64.copy())
    sabs = np.abs(ss.cpu().numpy().astype(np.float64))
    olayer.reduce_grad(p.slot_expert, scale_h, sabs)
    say("reduce_grad", R, E, B, H, Hp)
    m.moonep_reduce_grad(m.make_dims(R, E, B, S, K), H, Hp, i32(p.slot_expert), hs, ss)
    torch.cuda.synchronize()
    assert np.array_equal(hs.cpu().numpy(), ref_h32)  # float32, ranks ascending, bit for bit
    assert np.array_equal(ss.cpu().numpy(), ref_s32)  # consumed slots zero, unused slots untouched
    assert_sum_close(hs.cpu().numpy(), ref_h64, scale_h, 1e-5, "reduce_grad vs float64")


@pytest.mark.parametrize("H,Hp", [(24, 40), (64, 44)])
def test_reduce_grad_many_copies_of_one_expert(m, H, Hp):
    # expert 0 is in every token's top-2, so its home rank overflows into all 15 other ranks: 15 copies,
    # several batches of slot loads per item; H*Hp/4 = 240 or 704 vectors leaves a partial item
    R, E, B, S, K = 16, 16, 2, 40, 2
    rng = np.random.default_rng(7)
    topk = np.zeros((R, S, K), dtype=np.int32)
    topk[:, :, 1] = rng.integers(1, E, size=(R, S))
    p = oplanner.plan(topk, E, B)
    se = p.slot_expert.reshape(-1)
    assert int((se == 0).sum()) == R - 1
    hs = rand_tensor((E, H, Hp), torch.float32, seed=41)
    ss = rand_tensor((R, B, H, Hp), torch.float32, seed=42) * 1e3
    ref_h32 = hs.cpu().numpy().copy()
    ref_s32 = ss.cpu().numpy().copy()
    olayer.reduce_grad(p.slot_expert, ref_h32, ref_s32, dtype=np.float32)
    say("reduce_grad many copies", R, E, B, H, Hp)
    m.moonep_reduce_grad(m.make_dims(R, E, B, S, K), H, Hp, i32(p.slot_expert), hs, ss)
    torch.cuda.synchronize()
    assert np.array_equal(hs.cpu().numpy(), ref_h32)  # float32, ranks ascending, bit for bit
    assert np.array_equal(ss.cpu().numpy(), ref_s32)  # consumed slots zero, unused slots untouched


# ------------------------------------------------------------------ tiny workload end to end


def test_tiny_workload_forward_matches_plain_moe(m):
    from synthetic import WORKLOADS
    from synthetic.router import layer_inputs
    wl = WORKLOADS["tiny_f32"]
    inp = layer_inputs(wl, seed=0, device="cpu")
    L = m.MoeLayer(wl.R, wl.E, wl.B, wl.S, wl.K, wl.H, wl.Hp, dtype=torch.float32)
    L.topk_idx.copy_(torch.as_tensor(inp["topk_idx"]))
    L.gates.copy_(torch.as_tensor(inp["gates"]))
    L.X.copy_(inp["X"])
    L.W_home.copy_(inp["W_home"])
    say("tiny workload forward")
    L.forward()
    torch.cuda.synchronize()
    p = oplanner.plan(inp["topk_idx"], wl.E, wl.B)
    assert np.array_equal(npi(L.cu_seqlens), p.cu_seqlens)
    assert np.array_equal(npi(L.dest_idx), p.dest_idx)
    x = inp["X"].numpy().astype(np.float64)
    w = inp["W_home"].numpy().astype(np.float64)
    ref = olayer.moe_forward(x, w, inp["topk_idx"], inp["gates"])
    assert_gemm_close(np64(L.out), ref, 1e-4, "tiny forward")
