"""CPU oracle for the balanced expert-parallel MoE layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation (int64 indices, float64
arithmetic) of what the GPU path computes.  It shares no code with the HIP
library and imports nothing from it.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does.

Sources (web pages about MoonEP):
  [P1] "Valhalla static engineering review #004 -- MoonshotAI MoonEP" (wsisp.com),
       section 2 "Project background".
  [P2] "Moonshot open-sources MoonEP: an expert-parallel communication library
       for MoE training" (umios.umi6.com), sections "Core problem",
       "Core technique: dynamic redundant experts", "Memory contract and weight
       layout".
  [P3] "Moonshot AI Open-Sources MoonEP for Expert Parallelism"
       (interestana.com), paragraphs two (maxvio) and three (the S*K invariant).

Modules:
  planner   -- histogram, maxvio, and the home-first prefix-sum planner, step by
               step (a heuristic, so the oracle follows its steps).
  layer     -- dispatch, prefetch, group GEMM, combine, wgrad, reduce_grad, the
               backward of the data path (combine backward, group-GEMM dgrad,
               dispatch backward), the gated expert FFN's activation (silu,
               swiglu and its gradient), and the plain MoE definitions (forward
               and gradients, single projection and full FFN) they must reproduce.
  mincopies -- brute-force minimum number of redundant copies on tiny inputs.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against hand-worked examples, closed forms, invariants or brute force (see
tests/test_oracle_*.py).  No function is parity-unpinned.
"""
from . import planner, layer, mincopies  # noqa: F401
