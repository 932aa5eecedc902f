"""Balanced expert-parallel MoE layer on one MI355X (gfx950): Python binding of libmoonep.so.

The C ABI (include/moonep.h) has the seven calls of the layer -- moonep_plan
(and moonep_plan_ex, which also offers the fewest-copies planner),
moonep_dispatch, moonep_prefetch, moonep_group_gemm, moonep_combine,
moonep_wgrad, moonep_reduce_grad -- three for the backward of the data path --
moonep_combine_backward, moonep_group_gemm_dgrad, moonep_dispatch_backward --
and two for the activation of the gated expert FFN -- moonep_swiglu,
moonep_swiglu_backward -- exposed here under the same names, taking torch
tensors.  Importing this
package loads libmoonep.so and raises if it is missing; there is no CPU or
PyTorch fallback.
"""
from ._lib import (  # noqa: F401
    Dims, MoonepError, LIB_PATH, SYMBOLS, MOONEP_F32, MOONEP_BF16, MOONEP_PLAN_PREFIX, MOONEP_PLAN_MINCOPY,
    PLANNERS, make_dims, last_error,
    moonep_plan_workspace_bytes, moonep_group_gemm_workspace_bytes, moonep_wgrad_workspace_bytes, moonep_plan,
    moonep_plan_ex, moonep_plan_static, moonep_plan_static_scratch_bytes,
    moonep_dispatch, moonep_prefetch, moonep_group_gemm, moonep_combine, moonep_wgrad, moonep_reduce_grad,
    moonep_combine_backward, moonep_group_gemm_dgrad, moonep_dispatch_backward, moonep_swiglu,
    moonep_swiglu_backward,
)
from .layer import MoeFFN  # noqa: F401
from .layer import MoeLayer  # noqa: F401
