"""Static buffers for one balanced MoE layer and the call sequence through libmoonep.

Every buffer is allocated once, with shapes fixed by (R, E, B, S, K, H, Hp):
nothing depends on the routing, so repeated passes allocate nothing and a
pass can be captured in a HIP graph.  The forward pass is
plan -> prefetch -> dispatch -> group GEMM -> combine (the prefetch needs only
the plan); the weight backward is
wgrad -> reduce_grad; with data_grad=True the data backward is
combine_backward (writes dY and dgates from dout) -> dgrad -> dispatch_backward
(dX).  Each step is one C-ABI call whose kernels do all the work; this class
only owns memory and passes pointers.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import Dims, make_dims


class MoeLayer:
    """One balanced MoE projection layer.

    `slot_pool` = (W_slots [R,B,H,Hp] of the layer dtype, dW_slots [R,B,H,Hp] float32 or None) makes the
    layer use a caller's slot buffers instead of its own: the pages keep one process-wide pool of B
    slots that every layer shares, so the extra memory is B experts in total, not B per layer.  Layers
    sharing a pool run one after another; a layer's backward that follows other layers' forward passes
    re-runs its prefetch first (the pool then holds the other layers' slots), and its reduce_grad leaves
    the slot gradients at zero for the next layer.
    """

    def __init__(self, R, E, B, S, K, H, Hp=None, dtype=torch.bfloat16, device="cuda", backward=False,
                 src_of_row=True, data_grad=False, planner="prefix", slot_pool=None):
        self.d: Dims = make_dims(R, E, B, S, K)
        self.planner = planner  # "prefix" (home-first) or "mincopy" (fewest copies)
        d = self.d
        self.H, self.Hp, self.dtype, self.device = H, Hp, dtype, device
        i32 = dict(dtype=torch.int32, device=device)
        N = d.N
        # routing (inputs)
        self.topk_idx = torch.zeros((R, S, K), **i32)
        self.gates = torch.zeros((R, S, K), dtype=torch.float32, device=device)
        # plan outputs
        self.expert_counts = torch.zeros(E, **i32)
        self.maxvio = torch.zeros(1, dtype=torch.float64, device=device)
        self.cu_seqlens = torch.zeros((R, E + B + 1), **i32)
        self.slot_expert = torch.full((R, max(B, 0)), -1, **i32)
        self.dest_idx = torch.zeros((R, S, K), **i32)
        self.src_of_row = torch.zeros(N, **i32) if src_of_row else None
        self.stats = torch.zeros(4, **i32)
        self.ws_plan = torch.empty(max(1, _lib.moonep_plan_workspace_bytes(d)), dtype=torch.uint8, device=device)
        # activations
        self.X = torch.zeros((R, S, H), dtype=dtype, device=device)
        self.Xp = torch.empty((N, H), dtype=dtype, device=device)
        pool_w, pool_dw = slot_pool if slot_pool is not None else (None, None)
        if Hp is not None:
            self.W_home = torch.zeros((E, H, Hp), dtype=dtype, device=device)
            if pool_w is not None:
                if tuple(pool_w.shape) != (R, B, H, Hp) or pool_w.dtype != dtype:
                    raise ValueError(f"slot pool must be [{R},{B},{H},{Hp}] {dtype}")
                self.W_slots = pool_w
            else:
                self.W_slots = torch.zeros((R, B, H, Hp), dtype=dtype, device=device)
            self.Yp = torch.empty((N, Hp), dtype=dtype, device=device)
            self.ws_gemm = torch.empty(max(1, _lib.moonep_group_gemm_workspace_bytes(d)), dtype=torch.uint8,
                                       device=device)
            self.out = torch.empty((R, S, Hp), dtype=torch.float32, device=device)
            if backward:
                self.dY = torch.zeros((N, Hp), dtype=dtype, device=device)
                self.dW_home = torch.zeros((E, H, Hp), dtype=torch.float32, device=device)
                if pool_dw is not None:
                    if tuple(pool_dw.shape) != (R, B, H, Hp) or pool_dw.dtype != torch.float32:
                        raise ValueError(f"slot gradient pool must be [{R},{B},{H},{Hp}] float32")
                    self.dW_slots = pool_dw
                else:
                    self.dW_slots = torch.zeros((R, B, H, Hp), dtype=torch.float32, device=device)
                self.ws_wgrad = torch.empty(max(1, _lib.moonep_wgrad_workspace_bytes(d)), dtype=torch.uint8,
                                            device=device)
                if data_grad:
                    self.dout = torch.zeros((R, S, Hp), dtype=torch.float32, device=device)
                    self.dgates = torch.zeros((R, S, K), dtype=torch.float32, device=device)
                    self.dXp = torch.empty((N, H), dtype=dtype, device=device)
                    self.dX = torch.empty((R, S, H), dtype=torch.float32, device=device)

    # ---------------------------------------------------------------- steps
    def plan(self, stream=None):
        _lib.moonep_plan_ex(self.d, self.planner, self.topk_idx, self.expert_counts, self.maxvio, self.cu_seqlens,
                            self.slot_expert if self.d.B > 0 else None, self.dest_idx, self.src_of_row, self.stats,
                            self.ws_plan, stream)

    def dispatch(self, stream=None):
        _lib.moonep_dispatch(self.d, self.H, self.X, self.dest_idx, self.Xp, stream)

    def prefetch(self, stream=None):
        _lib.moonep_prefetch(self.d, self.H, self.Hp, self.W_home, self.slot_expert if self.d.B > 0 else None,
                             self.W_slots if self.d.B > 0 else None, stream)

    def group_gemm(self, stream=None):
        _lib.moonep_group_gemm(self.d, self.H, self.Hp, self.Xp, self.W_home,
                               self.W_slots if self.d.B > 0 else None, self.cu_seqlens, self.Yp, self.ws_gemm, stream)

    def combine(self, stream=None):
        _lib.moonep_combine(self.d, self.Hp, self.Yp, self.dest_idx, self.gates, self.out, stream)

    def wgrad(self, stream=None):
        _lib.moonep_wgrad(self.d, self.H, self.Hp, self.Xp, self.dY, self.cu_seqlens, self.dW_home,
                          self.dW_slots if self.d.B > 0 else None, self.ws_wgrad, stream)

    def reduce_grad(self, stream=None):
        _lib.moonep_reduce_grad(self.d, self.H, self.Hp, self.slot_expert if self.d.B > 0 else None, self.dW_home,
                                self.dW_slots if self.d.B > 0 else None, stream)

    def combine_backward(self, stream=None):
        _lib.moonep_combine_backward(self.d, self.Hp, self.dout, self.Yp, self.dest_idx, self.gates, self.dY,
                                     self.dgates, stream)

    def dgrad(self, stream=None):
        _lib.moonep_group_gemm_dgrad(self.d, self.H, self.Hp, self.dY, self.W_home,
                                     self.W_slots if self.d.B > 0 else None, self.cu_seqlens, self.dXp, self.ws_gemm,
                                     stream)

    def dispatch_backward(self, stream=None):
        _lib.moonep_dispatch_backward(self.d, self.H, self.dXp, self.dest_idx, self.dX, stream)

    def backward_data(self, stream=None):
        self.combine_backward(stream)
        self.dgrad(stream)
        self.dispatch_backward(stream)

    def forward(self, stream=None):
        self.plan(stream)
        if self.Hp is None:
            self.dispatch(stream)
            return
        # the weight prefetch needs only the plan, so it runs while (here: before) tokens dispatch
        self.prefetch(stream)
        self.dispatch(stream)
        self.group_gemm(stream)
        self.combine(stream)

    def backward(self, stream=None):
        self.wgrad(stream)
        self.reduce_grad(stream)


class MoeFFN:
    """Static buffers for one balanced MoE layer whose experts are gated FFNs, and the call sequence.

    Forward: plan -> dispatch -> prefetch (both projections) -> group GEMM with the gate|up weights
    [E+B, H, 2H'] -> swiglu -> group GEMM with the down weights [E+B, H', H] -> combine to [R, S, H].
    Backward (backward=True): combine backward -> dgrad and wgrad of the down projection -> swiglu
    backward -> dgrad and wgrad of the gate|up projection -> dispatch backward -> reduce_grad of both
    projections.  Every buffer has a shape fixed by (R, E, B, S, K, H, H'); nothing depends on the
    routing, so passes allocate nothing.
    """

    def __init__(self, R, E, B, S, K, H, Hp, dtype=torch.bfloat16, device="cuda", backward=False):
        self.d: Dims = make_dims(R, E, B, S, K)
        d = self.d
        self.H, self.Hp, self.dtype, self.device = H, Hp, dtype, device
        i32 = dict(dtype=torch.int32, device=device)
        act = dict(dtype=dtype, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        N = d.N
        self.topk_idx = torch.zeros((R, S, K), **i32)
        self.gates = torch.zeros((R, S, K), **f32)
        self.expert_counts = torch.zeros(E, **i32)
        self.maxvio = torch.zeros(1, dtype=torch.float64, device=device)
        self.cu_seqlens = torch.zeros((R, E + B + 1), **i32)
        self.slot_expert = torch.full((R, max(B, 0)), -1, **i32)
        self.dest_idx = torch.zeros((R, S, K), **i32)
        self.stats = torch.zeros(4, **i32)
        self.ws_plan = torch.empty(max(1, _lib.moonep_plan_workspace_bytes(d)), dtype=torch.uint8, device=device)
        self.ws_gemm = torch.empty(max(1, _lib.moonep_group_gemm_workspace_bytes(d)), dtype=torch.uint8,
                                   device=device)
        self.X = torch.zeros((R, S, H), **act)
        self.Xp = torch.empty((N, H), **act)
        self.W_gu_home = torch.zeros((E, H, 2 * Hp), **act)
        self.W_gu_slots = torch.zeros((R, B, H, 2 * Hp), **act)
        self.W_down_home = torch.zeros((E, Hp, H), **act)
        self.W_down_slots = torch.zeros((R, B, Hp, H), **act)
        self.Ygu = torch.empty((N, 2 * Hp), **act)
        self.A = torch.empty((N, Hp), **act)
        self.Zp = torch.empty((N, H), **act)
        self.out = torch.empty((R, S, H), **f32)
        if backward:
            self.ws_wgrad = torch.empty(max(1, _lib.moonep_wgrad_workspace_bytes(d)), dtype=torch.uint8,
                                        device=device)
            self.dout = torch.zeros((R, S, H), **f32)
            self.dgates = torch.zeros((R, S, K), **f32)
            self.dZp = torch.empty((N, H), **act)
            self.dA = torch.empty((N, Hp), **act)
            self.dYgu = torch.empty((N, 2 * Hp), **act)
            self.dXp = torch.empty((N, H), **act)
            self.dX = torch.empty((R, S, H), **f32)
            self.dW_gu_home = torch.zeros((E, H, 2 * Hp), **f32)
            self.dW_gu_slots = torch.zeros((R, B, H, 2 * Hp), **f32)
            self.dW_down_home = torch.zeros((E, Hp, H), **f32)
            self.dW_down_slots = torch.zeros((R, B, Hp, H), **f32)

    def _slots(self, t):
        return t if self.d.B > 0 else None

    def forward_calls(self):
        d, H, Hp, L = self.d, self.H, self.Hp, _lib
        sl = self._slots
        return [
            ("plan", lambda: L.moonep_plan(d, self.topk_idx, self.expert_counts, self.maxvio, self.cu_seqlens,
                                           sl(self.slot_expert), self.dest_idx, None, self.stats, self.ws_plan)),
            ("prefetch", lambda: (L.moonep_prefetch(d, H, 2 * Hp, self.W_gu_home, sl(self.slot_expert),
                                                    sl(self.W_gu_slots)),
                                  L.moonep_prefetch(d, Hp, H, self.W_down_home, sl(self.slot_expert),
                                                    sl(self.W_down_slots)))),
            ("dispatch", lambda: L.moonep_dispatch(d, H, self.X, self.dest_idx, self.Xp)),
            ("gemm_gate_up", lambda: L.moonep_group_gemm(d, H, 2 * Hp, self.Xp, self.W_gu_home, sl(self.W_gu_slots),
                                                         self.cu_seqlens, self.Ygu, self.ws_gemm)),
            ("swiglu", lambda: L.moonep_swiglu(d, Hp, self.Ygu, self.A)),
            ("gemm_down", lambda: L.moonep_group_gemm(d, Hp, H, self.A, self.W_down_home, sl(self.W_down_slots),
                                                      self.cu_seqlens, self.Zp, self.ws_gemm)),
            ("combine", lambda: L.moonep_combine(d, H, self.Zp, self.dest_idx, self.gates, self.out)),
        ]

    def backward_calls(self):
        d, H, Hp, L = self.d, self.H, self.Hp, _lib
        sl = self._slots
        return [
            ("combine_backward", lambda: L.moonep_combine_backward(d, H, self.dout, self.Zp, self.dest_idx,
                                                                   self.gates, self.dZp, self.dgates)),
            ("dgrad_down", lambda: L.moonep_group_gemm_dgrad(d, Hp, H, self.dZp, self.W_down_home,
                                                             sl(self.W_down_slots), self.cu_seqlens, self.dA,
                                                             self.ws_gemm)),
            ("wgrad_down", lambda: L.moonep_wgrad(d, Hp, H, self.A, self.dZp, self.cu_seqlens, self.dW_down_home,
                                                  sl(self.dW_down_slots), self.ws_wgrad)),
            ("swiglu_backward", lambda: L.moonep_swiglu_backward(d, Hp, self.Ygu, self.dA, self.dYgu)),
            ("dgrad_gate_up", lambda: L.moonep_group_gemm_dgrad(d, H, 2 * Hp, self.dYgu, self.W_gu_home,
                                                                sl(self.W_gu_slots), self.cu_seqlens, self.dXp,
                                                                self.ws_gemm)),
            ("wgrad_gate_up", lambda: L.moonep_wgrad(d, H, 2 * Hp, self.Xp, self.dYgu, self.cu_seqlens,
                                                     self.dW_gu_home, sl(self.dW_gu_slots), self.ws_wgrad)),
            ("dispatch_backward", lambda: L.moonep_dispatch_backward(d, H, self.dXp, self.dest_idx, self.dX)),
            ("reduce_grad", lambda: (L.moonep_reduce_grad(d, H, 2 * Hp, sl(self.slot_expert), self.dW_gu_home,
                                                          sl(self.dW_gu_slots)),
                                     L.moonep_reduce_grad(d, Hp, H, sl(self.slot_expert), self.dW_down_home,
                                                          sl(self.dW_down_slots)))),
        ]

    def forward(self):
        for _, f in self.forward_calls():
            f()

    def backward(self):
        for _, f in self.backward_calls():
            f()
