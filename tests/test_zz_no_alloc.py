"""moonep_plan_static, the planner entry point that allocates nothing (GPU): its outputs equal those of
moonep_plan_ex with a caller workspace, bit for bit, on two calls in a row (the second one smaller, so it
runs over scratch the first one left behind), for both planners.  (Sizes beyond its scratch are refused
on the host: tests/test_abi.py.)"""
import pytest
import torch

from synthetic import WORKLOADS
from synthetic.calibrate import alpha_for
from synthetic.router import router_output
from tests.gpu_util import DEV, npi, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import load_balanced_dispatch_amd as mod
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return mod


def outputs(wl, fill):
    dev = dict(device=DEV)
    return dict(counts=torch.full((wl.E,), fill, dtype=torch.int32, **dev),
                mv=torch.full((1,), float(fill), dtype=torch.float64, **dev),
                cu=torch.full((wl.R, wl.E + wl.B + 1), fill, dtype=torch.int32, **dev),
                slots=torch.full((wl.R, max(wl.B, 1)), fill, dtype=torch.int32, **dev),
                dest=torch.full((wl.R, wl.S, wl.K), fill, dtype=torch.int32, **dev),
                src=torch.full((wl.N,), fill, dtype=torch.int32, **dev),
                stats=torch.full((4,), fill, dtype=torch.int32, **dev))


def call(lib, fn, d, planner, topk, o, ws=None):
    args = [d, planner, topk.data_ptr(), o["counts"].data_ptr(), o["mv"].data_ptr(), o["cu"].data_ptr(),
            o["slots"].data_ptr(), o["dest"].data_ptr(), o["src"].data_ptr(), o["stats"].data_ptr()]
    if ws is not None:
        args.append(ws.data_ptr())
    return getattr(lib, fn)(*args, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("planner", [0, 1])
def test_static_plan_equals_plan_with_workspace(m, planner):
    from load_balanced_dispatch_amd import _lib
    lib = _lib.lib()
    cases = [("plan_stress", None), ("mid_fwd", 3.0), ("tiny_f32", None)]  # each call smaller than the last
    for name, target in cases:
        wl = WORKLOADS[name]
        alpha = 0.0 if wl.zipf_s is not None else (wl.alpha if target is None else alpha_for(wl, 0, target))
        idx, _ = router_output(wl.R, wl.S, wl.E, wl.K, 0, alpha=alpha, zipf_s=wl.zipf_s)
        topk = torch.as_tensor(idx).to(DEV)
        d = m.make_dims(wl.R, wl.E, wl.B, wl.S, wl.K)
        assert m.moonep_plan_workspace_bytes(d) <= lib.moonep_plan_static_scratch_bytes()
        say("static plan", name, target, planner)
        ref = outputs(wl, -7)
        ws = torch.empty(m.moonep_plan_workspace_bytes(d), dtype=torch.uint8, device=DEV)
        assert call(lib, "moonep_plan_ex", d, planner, topk, ref, ws) == 0
        got = outputs(wl, -9)
        assert call(lib, "moonep_plan_static", d, planner, topk, got) == 0, m.last_error()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (name, k)
        assert npi(got["cu"])[:, -1].tolist() == [wl.P] * wl.R



def test_static_plan_in_a_captured_graph(m):
    # the use it is for: captured once (after one eager call has looked up the scratch address), replayed
    # with new routings written into the same input buffer, each replay equal to an eager moonep_plan_ex
    from load_balanced_dispatch_amd import _lib
    lib = _lib.lib()
    wl = WORKLOADS["mid_fwd"]
    d = m.make_dims(wl.R, wl.E, wl.B, wl.S, wl.K)
    topk = torch.zeros((wl.R, wl.S, wl.K), dtype=torch.int32, device=DEV)
    got = outputs(wl, -9)
    routings = [router_output(wl.R, wl.S, wl.E, wl.K, 0, alpha=alpha_for(wl, 0, t))[0] for t in (0.0, 1.0, 3.0)]
    topk.copy_(torch.as_tensor(routings[0]))
    say("static plan graph: eager warm-up")
    assert call(lib, "moonep_plan_static", d, 1, topk, got) == 0, m.last_error()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert call(lib, "moonep_plan_static", d, 1, topk, got) == 0, m.last_error()
    torch.cuda.current_stream().wait_stream(s)
    ws = torch.empty(m.moonep_plan_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    for rep, idx in enumerate(routings + routings[:1]):
        say("static plan graph: replay", rep)
        topk.copy_(torch.as_tensor(idx))
        for t in got.values():
            t.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = outputs(wl, -7)
        assert call(lib, "moonep_plan_ex", d, 1, topk, ref, ws) == 0
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (rep, k)
