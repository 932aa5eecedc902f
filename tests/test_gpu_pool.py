"""One slot pool shared by several layers (GPU): the pages keep a single process-wide pool of B slot
rows (and their reduce buffers) for all layers.  Two layers share one pool through forward A, forward B,
backward B, then backward A (which re-prefetches its slots, since B's forward overwrote them); every
output, weight gradient and data gradient equals that of the same two layers with pools of their own,
bit for bit, and the shared slot gradients end at zero."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, rand_tensor, say
from tests.plan_checks import random_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import load_balanced_dispatch_amd as mod
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return mod


def make(m, R, E, B, S, K, H, Hp, pool, seed, planner):
    L = m.MoeLayer(R, E, B, S, K, H, Hp, backward=True, data_grad=True, planner=planner, slot_pool=pool)
    rng = np.random.default_rng(seed)
    L.topk_idx.copy_(torch.as_tensor(random_routing(rng, R, S, K, E, 2.5).astype(np.int32)))
    L.gates.copy_(torch.as_tensor(rng.dirichlet(np.ones(K), size=(R, S)).astype(np.float32)))
    L.X.copy_(rand_tensor((R, S, H), torch.bfloat16, seed=seed + 1))
    L.W_home.copy_(rand_tensor((E, H, Hp), torch.bfloat16, seed=seed + 2, std=H ** -0.5))
    L.dout.copy_(rand_tensor((R, S, Hp), torch.float32, seed=seed + 3))
    return L


def run(La, Lb):
    La.forward()
    Lb.forward()
    for L, refetch in ((Lb, False), (La, True)):
        if refetch:
            L.prefetch()  # the shared pool holds the other layer's slots now
        L.backward_data()
        L.backward()
    torch.cuda.synchronize()


@pytest.mark.parametrize("planner", ["prefix", "mincopy"])
def test_layers_share_one_slot_pool(m, planner):
    R, E, B, S, K, H, Hp = 4, 16, 4, 200, 4, 256, 384
    say("shared slot pool", planner)
    pool = (torch.zeros((R, B, H, Hp), dtype=torch.bfloat16, device=DEV),
            torch.zeros((R, B, H, Hp), dtype=torch.float32, device=DEV))
    shared = [make(m, R, E, B, S, K, H, Hp, pool, seed, planner) for seed in (10, 20)]
    own = [make(m, R, E, B, S, K, H, Hp, None, seed, planner) for seed in (10, 20)]
    assert shared[0].W_slots is shared[1].W_slots and own[0].W_slots is not own[1].W_slots
    run(*shared)
    run(*own)
    for a, b in zip(shared, own):
        assert int(a.stats[1].item()) > 0  # slots are in use
        for name in ("out", "dW_home", "dgates", "dX", "cu_seqlens", "dest_idx"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert float(pool[1].abs().max().item()) == 0.0


def test_slot_pool_shape_is_checked(m):
    with pytest.raises(ValueError, match="slot pool"):
        m.MoeLayer(2, 4, 2, 8, 2, 64, 64, slot_pool=(torch.zeros((2, 1, 64, 64), dtype=torch.bfloat16,
                                                                    device=DEV), None))
