"""Seeded synthetic inputs (router output, activations, weights, output grads) and workload sizes.

Shared by the tests, the benchmark and the oracle's callers; holds none of the
layer's arithmetic.
"""
from .configs import WORKLOADS, ORDER, Workload  # noqa: F401
