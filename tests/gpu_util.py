"""Helpers for the GPU parity tests: uploads, float64 views, tolerance checks.

Inputs given to both sides come from the seeded generators (synthetic/) or
from the oracle; nothing the HIP path returns is ever fed to the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda"


def say(*a):
    """Names the case before each GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def i32(a):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=DEV)


def f32(a):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32), device=DEV)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def npi(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def rand_tensor(shape, dtype, seed, std=1.0):
    """Seeded CPU normal tensor rounded to dtype (test inputs), then moved to the device."""
    g = torch.Generator().manual_seed(seed)
    t = torch.randn(shape, generator=g, dtype=torch.float32) * std
    return t.to(dtype).to(DEV)


def assert_gemm_close(gpu, ref, rel=1e-2, what="gemm"):
    """|gpu - ref| <= rel * (1 + |ref|), elementwise."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = rel * (1.0 + np.abs(ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside {rel}*(1+|ref|); worst at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r}")


def assert_sum_close(gpu, ref, scale, rel=1e-5, what="sum"):
    """|gpu - ref| <= rel * scale (+ a denormal floor), scale = sum of |terms|."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = rel * np.asarray(scale, dtype=np.float64) + 1e-30
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside; worst at {i}: gpu={gpu[i]!r} "
                             f"ref={ref[i]!r} scale={np.asarray(scale)[i]!r}")


def bf16_round_np(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via torch, round-to-nearest-even) and return float64."""
    return torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16).float().numpy().astype(np.float64)
