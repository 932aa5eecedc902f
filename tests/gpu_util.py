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


# ------------------------------------------------------------------ lazy host views of generated inputs
#
# At the workloads' full sizes the float64 host copies of the inputs would be tens of GB, so the oracle
# receives objects that fetch what it indexes.  They hold generator outputs (device tensors drawn by the
# seeded generators, never written by the library) and the oracle's own index maps.

class DeviceExperts:
    """W_home[e] of a device weight tensor as float64 on the host, fetched when indexed (two cached)."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)
        self._cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self._cache:
            if len(self._cache) >= 2:
                self._cache.pop(next(iter(self._cache)))
            self._cache[e] = np64(self.t[e])
        return self._cache[e]


class OracleSlots:
    """W_slots[r, j] as the oracle's prefetch defines it: the home weights of slot_expert[r, j]."""

    def __init__(self, W: DeviceExperts, slot_expert: np.ndarray):
        self.W, self.slot = W, slot_expert

    def __getitem__(self, rj):
        r, j = rj
        e = int(self.slot[r, j])
        assert e >= 0, "read of an unused slot"
        return self.W[e]


class DispatchedRows:
    """Xp as the oracle's dispatch defines it: row i is token src_of_row[i] // K of the device tensor X
    ([R*S, H] view); rows are gathered on the device and returned as float64."""

    def __init__(self, Xf: torch.Tensor, src_of_row: np.ndarray, K: int):
        self.Xf, self.src, self.K = Xf, src_of_row, K
        self.shape = (len(src_of_row), Xf.shape[1])

    def __getitem__(self, rows):
        tok = np.asarray(self.src[rows]) // self.K
        return np64(self.Xf[torch.as_tensor(tok, device=self.Xf.device)])


class DeviceRows:
    """Rows of a device tensor (a generator output such as dY), fetched as float64 when indexed; with
    `index`, item i is row index[i] of the tensor (e.g. the gradient row of pair i, index = dest_idx)."""

    def __init__(self, t: torch.Tensor, index=None):
        self.t = t
        self.index = None if index is None else np.asarray(index)
        n = t.shape[0] if index is None else len(self.index)
        self.shape = (n,) + tuple(t.shape[1:])

    def __getitem__(self, rows):
        ids = np.arange(self.shape[0])[rows] if isinstance(rows, slice) else np.asarray(rows)
        if self.index is not None:
            ids = self.index[ids]
        return np64(self.t[torch.as_tensor(ids, device=self.t.device)])


class Guarded:
    """A device buffer of `shape` inside a larger allocation whose guard regions before and after it hold a
    fixed bit pattern; intact() tells whether anything wrote outside the buffer."""

    PATTERN = {2: 0x5A5B, 4: 0x5A5B5C5D}

    def __init__(self, shape, dtype, guard_bytes=64 * 1024):
        es = torch.empty((), dtype=dtype).element_size()
        self.g = guard_bytes // es
        self.n = int(np.prod(shape))
        self.buf = torch.empty(self.n + 2 * self.g, dtype=dtype, device=DEV)
        self.view = self.buf[self.g:self.g + self.n].view(shape)
        self.ity = {2: torch.int16, 4: torch.int32}[es]
        self.pat = self.PATTERN[es]
        self.buf[:self.g].view(self.ity).fill_(self.pat)
        self.buf[self.g + self.n:].view(self.ity).fill_(self.pat)

    def intact(self) -> bool:
        lo = self.buf[:self.g].view(self.ity)
        hi = self.buf[self.g + self.n:].view(self.ity)
        return bool((lo == self.pat).all().item()) and bool((hi == self.pat).all().item())
