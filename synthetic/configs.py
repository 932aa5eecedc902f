"""The five workloads of the balanced expert-parallel MoE layer, with their sizes.

Notation (after the memory-contract section of "Moonshot open-sources MoonEP: an
expert-parallel communication library for MoE training", umios.umi6.com):
R virtual expert-parallel ranks, E routed experts (E/R home experts per rank),
B prefetch slots per rank, S tokens per rank, K experts per token, H hidden
size, Hp = H' the expert FFN width.  P = S*K pairs per rank, N = R*S*K pairs.

The router recipe follows the same article's "core problem" section (maxvio as
the skew measure); the skew is produced synthetically: logits are N(0,1) noise
plus ``alpha * z_e`` with ``z_e ~ N(0,1)`` per expert, or, for the
planner-stress workload, a Zipf(s) popularity bias over a seeded expert
permutation.  ``alpha`` is chosen per sweep point so that the measured maxvio
lands near a target (table in ``alpha_table.json``, written by
``calibrate.py``).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    R: int
    E: int
    K: int
    S: int
    H: int
    Hp: Optional[int]  # None: no expert projection (planner/dispatch stress)
    B: int
    dtype: str  # "f32" or "bf16"
    backward: bool = False
    alpha: Optional[float] = None  # fixed skew (tiny workload)
    maxvio_targets: Tuple[float, ...] = ()
    zipf_s: Optional[float] = None
    description: str = ""

    @property
    def P(self) -> int:
        return self.S * self.K

    @property
    def N(self) -> int:
        return self.R * self.S * self.K

    @property
    def experts_per_rank(self) -> int:
        return self.E // self.R

    def with_dims(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", R=4, E=16, K=2, S=64, H=128, Hp=256, B=4, dtype="f32",
        alpha=1.0,
        description="tiny forward, fp32 throughout (R4 E16 K2 S64 H128 H'256 B4)"),
    "mid_fwd": Workload(
        name="mid_fwd", R=8, E=64, K=6, S=4096, H=2048, Hp=1408, B=8, dtype="bf16",
        maxvio_targets=(0.0, 1.0, 3.0),
        description="mid forward sweep, bf16 (R8 E64 K6 S4096 H2048 H'1408 B8)"),
    "large_fwd": Workload(
        name="large_fwd", R=8, E=256, K=8, S=4096, H=7168, Hp=2048, B=32, dtype="bf16",
        maxvio_targets=(0.5, 1.0, 2.0, 4.0),
        description="large forward, bf16, training slot budget B=E/R (R8 E256 K8 S4096 H7168 H'2048 B32)"),
    "mid_bwd": Workload(
        name="mid_bwd", R=8, E=64, K=6, S=4096, H=2048, Hp=1408, B=8, dtype="bf16",
        backward=True, maxvio_targets=(2.0,),
        description="backward, bf16 in / fp32 grads (R8 E64 K6 S4096 H2048 H'1408 B8)"),
    "plan_stress": Workload(
        name="plan_stress", R=64, E=384, K=8, S=2048, H=7168, Hp=None, B=4, dtype="bf16",
        zipf_s=1.2,
        description="planner/dispatch stress, bf16, Zipf(1.2) popularity (R64 E384 K8 S2048 H7168 B4)"),
}

# The workloads in their published order (tiny, mid sweep, large, backward, stress).
ORDER = ("tiny_f32", "mid_fwd", "large_fwd", "mid_bwd", "plan_stress")
