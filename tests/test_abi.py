"""The C-ABI library loads, exports every symbol include/moonep.h declares, and rejects bad
arguments on the host before enqueuing anything (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import load_balanced_dispatch_amd as m
from load_balanced_dispatch_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moonep.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(moonep_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    syms = declared_symbols()
    for name in ("moonep_plan", "moonep_dispatch", "moonep_prefetch", "moonep_group_gemm", "moonep_combine",
                 "moonep_wgrad", "moonep_reduce_grad", "moonep_combine_backward", "moonep_group_gemm_dgrad",
                 "moonep_dispatch_backward", "moonep_swiglu", "moonep_swiglu_backward"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert sorted(declared_symbols()) == sorted(_lib.SYMBOLS)


def test_workspace_queries():
    d = m.make_dims(8, 64, 8, 4096, 6)
    assert m.moonep_plan_workspace_bytes(d) > 0
    assert m.moonep_group_gemm_workspace_bytes(d) >= 2 * 4 * (8 * 72 + 1)
    assert m.moonep_plan_workspace_bytes(m.make_dims(64, 384, 4, 2048, 8)) > 0


@pytest.mark.parametrize("dims,msg", [
    ((8, 63, 8, 16, 2), "multiple of R"),
    ((0, 64, 8, 16, 2), "R must be"),
    ((8, 64, -1, 16, 2), "B must be"),
    ((8, 64, 8, -1, 2), "S must be"),
    ((8, 64, 8, 16, 0), "K must be"),
    ((8, 64, 8, 16, 65), "K must be"),
    ((1024, 1024, 1, 1 << 20, 8), "2^31"),
])
def test_bad_dims_rejected_everywhere(dims, msg):
    d = m.make_dims(*dims)
    L = _lib.lib()
    null = None
    calls = [
        lambda: L.moonep_plan(d, *([null] * 10)),
        lambda: L.moonep_plan_ex(d, 1, *([null] * 10)),
        lambda: L.moonep_plan_static(d, 0, *([null] * 9)),
        lambda: L.moonep_dispatch(d, 8, 1, null, null, null, null),
        lambda: L.moonep_prefetch(d, 8, 8, 1, null, null, null, null),
        lambda: L.moonep_group_gemm(d, 8, 8, 1, *([null] * 7)),
        lambda: L.moonep_combine(d, 8, 1, null, null, null, null, null),
        lambda: L.moonep_wgrad(d, 8, 8, 1, *([null] * 7)),
        lambda: L.moonep_reduce_grad(d, 8, 8, null, null, null, null),
        lambda: L.moonep_combine_backward(d, 8, 1, *([null] * 7)),
        lambda: L.moonep_group_gemm_dgrad(d, 8, 8, 1, *([null] * 7)),
        lambda: L.moonep_dispatch_backward(d, 8, 1, null, null, null, null),
        lambda: L.moonep_swiglu(d, 8, 1, null, null, null),
        lambda: L.moonep_swiglu_backward(d, 8, 1, null, null, null, null),
    ]
    for c in calls:
        assert c() == _lib.MOONEP_EINVAL
        assert msg in m.last_error()
    assert m.moonep_plan_workspace_bytes(d) == 0
    assert m.moonep_wgrad_workspace_bytes(d) == 0


@pytest.mark.parametrize("R,E,msg", [
    (4096, 4096, "LDS"),        # emit tables 8E + 3R ints = 176 KiB
    (4096, 8192, "exceeds"),    # beyond the expert limit
    (4, 4100, "exceeds"),
])
def test_plan_rejects_sizes_beyond_its_lds_tables(R, E, msg):
    d = m.make_dims(R, E, 8, 1, 2)
    assert _lib.lib().moonep_plan(d, *([None] * 10)) == _lib.MOONEP_EINVAL
    assert msg in m.last_error()


def test_plan_ex_rejects_an_unknown_planner():
    d = m.make_dims(2, 4, 1, 3, 1)
    L = _lib.lib()
    assert L.moonep_plan_ex(d, 2, *([None] * 10)) == _lib.MOONEP_EINVAL
    assert "planner" in m.last_error()
    assert L.moonep_plan_ex(d, -1, *([None] * 10)) == _lib.MOONEP_EINVAL
    assert L.moonep_plan_ex(d, _lib.MOONEP_PLAN_MINCOPY, *([None] * 10)) == _lib.MOONEP_EINVAL
    assert "null" in m.last_error()  # a valid planner gets as far as the pointer checks
    with pytest.raises(ValueError, match="planner"):
        _lib._planner_code("optimal")


def test_static_plan_refuses_sizes_beyond_its_scratch():
    # refused on the host, before the scratch array's device address is looked up
    d = m.make_dims(64, 4096, 4, 65536, 8)  # 4 Mi pairs over 4096 experts: 128 MiB of block histograms
    L = _lib.lib()
    assert m.moonep_plan_workspace_bytes(d) > L.moonep_plan_static_scratch_bytes() == 8 << 20
    assert L.moonep_plan_static(d, 0, *([None] * 8), None) == _lib.MOONEP_EINVAL
    assert "scratch" in m.last_error()
    small = m.make_dims(2, 4, 1, 3, 1)
    assert L.moonep_plan_static(small, 0, *([None] * 8), None) == _lib.MOONEP_EINVAL
    assert "null" in m.last_error()


def test_null_pointers_rejected():
    d = m.make_dims(2, 4, 1, 3, 1)
    L = _lib.lib()
    assert L.moonep_plan(d, *([None] * 10)) == _lib.MOONEP_EINVAL
    assert "null" in m.last_error()
    assert L.moonep_dispatch(d, 8, 1, None, None, None, None) == _lib.MOONEP_EINVAL
    assert L.moonep_group_gemm(d, 8, 8, 1, *([None] * 7)) == _lib.MOONEP_EINVAL
    assert L.moonep_wgrad(d, 8, 8, 1, *([None] * 7)) == _lib.MOONEP_EINVAL
    assert L.moonep_reduce_grad(d, 8, 8, None, None, None, None) == _lib.MOONEP_EINVAL
    assert L.moonep_combine_backward(d, 8, 1, *([None] * 7)) == _lib.MOONEP_EINVAL
    assert L.moonep_group_gemm_dgrad(d, 8, 8, 1, *([None] * 7)) == _lib.MOONEP_EINVAL
    assert L.moonep_dispatch_backward(d, 8, 1, None, None, None, None) == _lib.MOONEP_EINVAL
    assert L.moonep_swiglu(d, 8, 1, None, None, None) == _lib.MOONEP_EINVAL
    assert L.moonep_swiglu_backward(d, 8, 1, None, None, None, None) == _lib.MOONEP_EINVAL


def test_bad_dtype_rejected():
    d = m.make_dims(2, 4, 1, 3, 1)
    L = _lib.lib()
    assert L.moonep_dispatch(d, 8, 7, None, None, None, None) == _lib.MOONEP_EINVAL
    assert "dtype" in m.last_error()
    assert L.moonep_combine_backward(d, 8, 7, *([None] * 7)) == _lib.MOONEP_EINVAL
    assert "dtype" in m.last_error()
    assert L.moonep_group_gemm_dgrad(d, 8, 8, 7, *([None] * 7)) == _lib.MOONEP_EINVAL
    assert "dtype" in m.last_error()


def test_empty_work_is_a_no_op():
    # S == 0: nothing to move or multiply; returns OK without touching any pointer
    d = m.make_dims(2, 4, 1, 0, 1)
    L = _lib.lib()
    assert L.moonep_dispatch(d, 8, 1, None, None, None, None) == _lib.MOONEP_OK
    assert L.moonep_combine(d, 8, 1, None, None, None, None, None) == _lib.MOONEP_OK
    assert L.moonep_group_gemm(d, 8, 8, 1, *([None] * 7)) == _lib.MOONEP_OK
    assert L.moonep_wgrad(d, 8, 8, 1, *([None] * 7)) == _lib.MOONEP_OK
    assert L.moonep_combine_backward(d, 8, 1, *([None] * 7)) == _lib.MOONEP_OK
    assert L.moonep_group_gemm_dgrad(d, 8, 8, 1, *([None] * 7)) == _lib.MOONEP_OK
    assert L.moonep_dispatch_backward(d, 8, 1, None, None, None, None) == _lib.MOONEP_OK
    assert L.moonep_swiglu(d, 8, 1, None, None, None) == _lib.MOONEP_OK
    assert L.moonep_swiglu_backward(d, 8, 1, None, None, None, None) == _lib.MOONEP_OK


def test_binding_refuses_host_tensors():
    import torch
    d = m.make_dims(2, 4, 1, 3, 1)
    with pytest.raises(ValueError, match="device tensor"):
        m.moonep_dispatch(d, 8, torch.zeros(6, 8), torch.zeros(6, dtype=torch.int32), torch.zeros(6, 8))


def test_one_hip_runtime_in_process():
    # the binding loads torch's HIP runtime before libmoonep.so, so only one libamdhip64 is mapped
    import subprocess
    import sys
    code = ("import load_balanced_dispatch_amd, torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout + out.stderr


def test_build_script_loads_without_the_library():
    # build() must work on a fresh checkout: its module is loaded by path, never through the package
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("moonep_build_probe",
                                                  os.path.join(root, "load_balanced_dispatch_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert callable(mod.build) and mod.ARCH == "gfx950"
    assert "-packed-fp32-ops" in mod.FLAGS


@pytest.mark.parametrize("entry", ["moonep_group_gemm", "moonep_group_gemm_dgrad"])
@pytest.mark.parametrize("which,msg", [(0, "input rows"), (5, "output rows"), (1, "weight rows"), (2, "weight rows")])
def test_gemm_rejects_misaligned_rows(entry, which, msg):
    # 16-byte rows move as 16-byte vectors, so an offset view (here 2 bytes) is refused before any launch;
    # the pointers are never dereferenced
    d = m.make_dims(2, 4, 1, 3, 1)
    ptrs = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000]  # A, W_home, W_slots, cu_seqlens, C, ws
    ptrs[{0: 0, 1: 1, 2: 2, 5: 4}[which]] += 2
    rc = getattr(_lib.lib(), entry)(d, 64, 64, _lib.MOONEP_BF16, *ptrs, None)
    assert rc == _lib.MOONEP_EINVAL
    assert msg in m.last_error()
