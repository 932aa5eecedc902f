"""ctypes binding of libmoonep.so: the same entry points, taking torch tensors.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoonep.so.  Tensors must be CUDA (HIP) tensors, contiguous, with the shapes
and dtypes that include/moonep.h documents; calls are enqueued on the current
torch stream (or the one passed) and never synchronise.  A nonzero return code
raises MoonepError carrying the library's message.

There is no fallback: if libmoonep.so is missing or fails to load, importing
this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoonep.so")

MOONEP_F32, MOONEP_BF16 = 0, 1
MOONEP_PLAN_PREFIX, MOONEP_PLAN_MINCOPY = 0, 1
PLANNERS = {"prefix": MOONEP_PLAN_PREFIX, "mincopy": MOONEP_PLAN_MINCOPY}
MOONEP_OK, MOONEP_EINVAL, MOONEP_EHIP, MOONEP_EUNSUPPORTED = 0, -1, -2, -3
_CODES = {MOONEP_EINVAL: "EINVAL", MOONEP_EHIP: "EHIP", MOONEP_EUNSUPPORTED: "EUNSUPPORTED"}


class MoonepError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_CODES.get(code, code)}: {message}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("E", ctypes.c_int32), ("B", ctypes.c_int32),
                ("S", ctypes.c_int32), ("K", ctypes.c_int32)]

    def __repr__(self):
        return f"Dims(R={self.R}, E={self.E}, B={self.B}, S={self.S}, K={self.K})"

    @property
    def P(self):
        return self.S * self.K

    @property
    def N(self):
        return self.R * self.S * self.K


def _load():
    # torch must bring in its HIP runtime first: libmoonep.so then binds to that same
    # libamdhip64 (same soname) instead of loading a second runtime from /opt/rocm,
    # and two HIP runtimes in one process leave the library's launches without a device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python load_balanced_dispatch_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moonep_last_error": (ctypes.c_char_p, []),
        "moonep_plan_workspace_bytes": (sz, [Dims]),
        "moonep_plan": (ctypes.c_int, [Dims, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "moonep_plan_ex": (ctypes.c_int, [Dims, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "moonep_plan_static_scratch_bytes": (sz, []),
        "moonep_plan_static": (ctypes.c_int, [Dims, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "moonep_dispatch": (ctypes.c_int, [Dims, i32, ctypes.c_int, vp, vp, vp, vp]),
        "moonep_prefetch": (ctypes.c_int, [Dims, i32, i32, ctypes.c_int, vp, vp, vp, vp]),
        "moonep_group_gemm_workspace_bytes": (sz, [Dims]),
        "moonep_group_gemm": (ctypes.c_int, [Dims, i32, i32, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]),
        "moonep_combine": (ctypes.c_int, [Dims, i32, ctypes.c_int, vp, vp, vp, vp, vp]),
        "moonep_wgrad_workspace_bytes": (sz, [Dims]),
        "moonep_wgrad": (ctypes.c_int, [Dims, i32, i32, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]),
        "moonep_reduce_grad": (ctypes.c_int, [Dims, i32, i32, vp, vp, vp, vp]),
        "moonep_combine_backward": (ctypes.c_int, [Dims, i32, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]),
        "moonep_group_gemm_dgrad": (ctypes.c_int, [Dims, i32, i32, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]),
        "moonep_dispatch_backward": (ctypes.c_int, [Dims, i32, ctypes.c_int, vp, vp, vp, vp]),
        "moonep_swiglu": (ctypes.c_int, [Dims, i32, ctypes.c_int, vp, vp, vp]),
        "moonep_swiglu_backward": (ctypes.c_int, [Dims, i32, ctypes.c_int, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_LIB = _load()

# exported symbol names, as declared in include/moonep.h
SYMBOLS = ("moonep_last_error", "moonep_plan_workspace_bytes", "moonep_plan", "moonep_plan_ex",
           "moonep_plan_static_scratch_bytes", "moonep_plan_static", "moonep_dispatch", "moonep_prefetch",
           "moonep_group_gemm_workspace_bytes", "moonep_group_gemm", "moonep_combine",
           "moonep_wgrad_workspace_bytes", "moonep_wgrad", "moonep_reduce_grad", "moonep_combine_backward",
           "moonep_group_gemm_dgrad", "moonep_dispatch_backward", "moonep_swiglu", "moonep_swiglu_backward")


def lib():
    return _LIB


def last_error() -> str:
    return _LIB.moonep_last_error().decode()


def _check(rc: int):
    if rc != MOONEP_OK:
        raise MoonepError(rc, last_error())


# ------------------------------------------------------------------ marshalling helpers

def _ptr(t, name, dtype=None, numel=None, optional=False):
    import torch
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements (got {t.numel()})")
    return t.data_ptr()


def _dtype_enum(t):
    import torch
    if t.dtype == torch.bfloat16:
        return MOONEP_BF16
    if t.dtype == torch.float32:
        return MOONEP_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_dims(R, E, B, S, K) -> Dims:
    return Dims(int(R), int(E), int(B), int(S), int(K))


# ------------------------------------------------------------------ entry points

def moonep_plan_workspace_bytes(d: Dims) -> int:
    return int(_LIB.moonep_plan_workspace_bytes(d))


def moonep_group_gemm_workspace_bytes(d: Dims) -> int:
    return int(_LIB.moonep_group_gemm_workspace_bytes(d))


def moonep_wgrad_workspace_bytes(d: Dims) -> int:
    return int(_LIB.moonep_wgrad_workspace_bytes(d))


def moonep_plan(d: Dims, topk_idx, expert_counts, maxvio, cu_seqlens, slot_expert, dest_idx, src_of_row, stats,
                workspace, stream=None):
    moonep_plan_ex(d, MOONEP_PLAN_PREFIX, topk_idx, expert_counts, maxvio, cu_seqlens, slot_expert, dest_idx,
                   src_of_row, stats, workspace, stream)


def _planner_code(planner) -> int:
    if isinstance(planner, str):
        if planner not in PLANNERS:
            raise ValueError(f"unknown planner {planner!r}; one of {sorted(PLANNERS)}")
        return PLANNERS[planner]
    return int(planner)


def moonep_plan_ex(d: Dims, planner, topk_idx, expert_counts, maxvio, cu_seqlens, slot_expert, dest_idx, src_of_row,
                   stats, workspace, stream=None):
    """moonep_plan with a planner: "prefix" (MOONEP_PLAN_PREFIX) or "mincopy" (MOONEP_PLAN_MINCOPY)."""
    import torch
    i32 = torch.int32
    args = (
        _ptr(topk_idx, "topk_idx", i32, d.N),
        _ptr(expert_counts, "expert_counts", i32, d.E),
        _ptr(maxvio, "maxvio", torch.float64, 1),
        _ptr(cu_seqlens, "cu_seqlens", i32, d.R * (d.E + d.B + 1)),
        _ptr(slot_expert, "slot_expert", i32, d.R * d.B, optional=d.B == 0),
        _ptr(dest_idx, "dest_idx", i32, d.N),
        _ptr(src_of_row, "src_of_row", i32, d.N, optional=True),
        _ptr(stats, "stats", i32, 4),
        _ptr(workspace, "workspace"),
    )
    if workspace.numel() * workspace.element_size() < moonep_plan_workspace_bytes(d):
        raise ValueError("plan workspace too small")
    _check(_LIB.moonep_plan_ex(d, _planner_code(planner), *args, _stream(stream)))


def moonep_plan_static_scratch_bytes() -> int:
    return int(_LIB.moonep_plan_static_scratch_bytes())


def moonep_plan_static(d: Dims, planner, topk_idx, expert_counts, maxvio, cu_seqlens, slot_expert, dest_idx,
                       src_of_row, stats, stream=None):
    """moonep_plan_ex without a workspace: the library's own per-GPU scratch array serves instead (calls that
    overlap on one GPU race on it)."""
    import torch
    i32 = torch.int32
    _check(_LIB.moonep_plan_static(
        d, _planner_code(planner), _ptr(topk_idx, "topk_idx", i32, d.N),
        _ptr(expert_counts, "expert_counts", i32, d.E), _ptr(maxvio, "maxvio", torch.float64, 1),
        _ptr(cu_seqlens, "cu_seqlens", i32, d.R * (d.E + d.B + 1)),
        _ptr(slot_expert, "slot_expert", i32, d.R * d.B, optional=d.B == 0), _ptr(dest_idx, "dest_idx", i32, d.N),
        _ptr(src_of_row, "src_of_row", i32, d.N, optional=True), _ptr(stats, "stats", i32, 4), _stream(stream)))


def moonep_dispatch(d: Dims, H: int, X, dest_idx, Xp, stream=None):
    import torch
    t = _dtype_enum(X)
    _check(_LIB.moonep_dispatch(d, int(H), t, _ptr(X, "X", X.dtype, d.R * d.S * H),
                                _ptr(dest_idx, "dest_idx", torch.int32, d.N),
                                _ptr(Xp, "Xp", X.dtype, d.N * H), _stream(stream)))


def moonep_prefetch(d: Dims, H: int, Hp: int, W_home, slot_expert, W_slots, stream=None):
    import torch
    t = _dtype_enum(W_home)
    _check(_LIB.moonep_prefetch(d, int(H), int(Hp), t, _ptr(W_home, "W_home", W_home.dtype, d.E * H * Hp),
                                _ptr(slot_expert, "slot_expert", torch.int32, d.R * d.B, optional=d.B == 0),
                                _ptr(W_slots, "W_slots", W_home.dtype, d.R * d.B * H * Hp, optional=d.B == 0),
                                _stream(stream)))


def moonep_group_gemm(d: Dims, H: int, Hp: int, Xp, W_home, W_slots, cu_seqlens, Yp, workspace, stream=None):
    import torch
    t = _dtype_enum(Xp)
    if workspace.numel() * workspace.element_size() < moonep_group_gemm_workspace_bytes(d):
        raise ValueError("group GEMM workspace too small")
    _check(_LIB.moonep_group_gemm(d, int(H), int(Hp), t, _ptr(Xp, "Xp", Xp.dtype, d.N * H),
                                  _ptr(W_home, "W_home", Xp.dtype, d.E * H * Hp),
                                  _ptr(W_slots, "W_slots", Xp.dtype, d.R * d.B * H * Hp, optional=d.B == 0),
                                  _ptr(cu_seqlens, "cu_seqlens", torch.int32, d.R * (d.E + d.B + 1)),
                                  _ptr(Yp, "Yp", Xp.dtype, d.N * Hp), _ptr(workspace, "workspace"),
                                  _stream(stream)))


def moonep_combine(d: Dims, D: int, Yp, dest_idx, gates, out, stream=None):
    import torch
    t = _dtype_enum(Yp)
    _check(_LIB.moonep_combine(d, int(D), t, _ptr(Yp, "Yp", Yp.dtype, d.N * D),
                               _ptr(dest_idx, "dest_idx", torch.int32, d.N),
                               _ptr(gates, "gates", torch.float32, d.N),
                               _ptr(out, "out", torch.float32, d.R * d.S * D), _stream(stream)))


def moonep_wgrad(d: Dims, H: int, Hp: int, Xp, dY, cu_seqlens, dW_home, dW_slots, workspace, stream=None):
    import torch
    t = _dtype_enum(Xp)
    if workspace.numel() * workspace.element_size() < moonep_wgrad_workspace_bytes(d):
        raise ValueError("wgrad workspace too small")
    _check(_LIB.moonep_wgrad(d, int(H), int(Hp), t, _ptr(Xp, "Xp", Xp.dtype, d.N * H),
                             _ptr(dY, "dY", Xp.dtype, d.N * Hp),
                             _ptr(cu_seqlens, "cu_seqlens", torch.int32, d.R * (d.E + d.B + 1)),
                             _ptr(dW_home, "dW_home", torch.float32, d.E * H * Hp),
                             _ptr(dW_slots, "dW_slots", torch.float32, d.R * d.B * H * Hp, optional=d.B == 0),
                             _ptr(workspace, "workspace"), _stream(stream)))


def moonep_reduce_grad(d: Dims, H: int, Hp: int, slot_expert, dW_home, dW_slots, stream=None):
    import torch
    _check(_LIB.moonep_reduce_grad(d, int(H), int(Hp),
                                   _ptr(slot_expert, "slot_expert", torch.int32, d.R * d.B, optional=d.B == 0),
                                   _ptr(dW_home, "dW_home", torch.float32, d.E * H * Hp),
                                   _ptr(dW_slots, "dW_slots", torch.float32, d.R * d.B * H * Hp, optional=d.B == 0),
                                   _stream(stream)))


def moonep_combine_backward(d: Dims, D: int, dout, Yp, dest_idx, gates, dYp, dgates, stream=None):
    import torch
    t = _dtype_enum(Yp)
    _check(_LIB.moonep_combine_backward(d, int(D), t, _ptr(dout, "dout", torch.float32, d.R * d.S * D),
                                        _ptr(Yp, "Yp", Yp.dtype, d.N * D),
                                        _ptr(dest_idx, "dest_idx", torch.int32, d.N),
                                        _ptr(gates, "gates", torch.float32, d.N),
                                        _ptr(dYp, "dYp", Yp.dtype, d.N * D),
                                        _ptr(dgates, "dgates", torch.float32, d.N), _stream(stream)))


def moonep_group_gemm_dgrad(d: Dims, H: int, Hp: int, dYp, W_home, W_slots, cu_seqlens, dXp, workspace,
                            stream=None):
    import torch
    t = _dtype_enum(dYp)
    if workspace.numel() * workspace.element_size() < moonep_group_gemm_workspace_bytes(d):
        raise ValueError("group GEMM workspace too small")
    _check(_LIB.moonep_group_gemm_dgrad(d, int(H), int(Hp), t, _ptr(dYp, "dYp", dYp.dtype, d.N * Hp),
                                        _ptr(W_home, "W_home", dYp.dtype, d.E * H * Hp),
                                        _ptr(W_slots, "W_slots", dYp.dtype, d.R * d.B * H * Hp, optional=d.B == 0),
                                        _ptr(cu_seqlens, "cu_seqlens", torch.int32, d.R * (d.E + d.B + 1)),
                                        _ptr(dXp, "dXp", dYp.dtype, d.N * H), _ptr(workspace, "workspace"),
                                        _stream(stream)))


def moonep_dispatch_backward(d: Dims, H: int, dXp, dest_idx, dX, stream=None):
    import torch
    t = _dtype_enum(dXp)
    _check(_LIB.moonep_dispatch_backward(d, int(H), t, _ptr(dXp, "dXp", dXp.dtype, d.N * H),
                                         _ptr(dest_idx, "dest_idx", torch.int32, d.N),
                                         _ptr(dX, "dX", torch.float32, d.R * d.S * H), _stream(stream)))


def moonep_swiglu(d: Dims, Hp: int, Ygu, A, stream=None):
    t = _dtype_enum(Ygu)
    _check(_LIB.moonep_swiglu(d, int(Hp), t, _ptr(Ygu, "Ygu", Ygu.dtype, d.N * 2 * Hp),
                              _ptr(A, "A", Ygu.dtype, d.N * Hp), _stream(stream)))


def moonep_swiglu_backward(d: Dims, Hp: int, Ygu, dA, dYgu, stream=None):
    t = _dtype_enum(Ygu)
    _check(_LIB.moonep_swiglu_backward(d, int(Hp), t, _ptr(Ygu, "Ygu", Ygu.dtype, d.N * 2 * Hp),
                                       _ptr(dA, "dA", Ygu.dtype, d.N * Hp),
                                       _ptr(dYgu, "dYgu", Ygu.dtype, d.N * 2 * Hp), _stream(stream)))
