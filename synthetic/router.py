"""Seeded synthetic router output and tensors for the balanced expert-parallel MoE layer.

This module only draws inputs.  It holds none of the layer's arithmetic: the
histogram, planner, permute, GEMMs, combine and gradient reduction live in the
HIP library and, independently, in the CPU oracle.  Both sides receive the
arrays made here.

Router recipe (a stand-in for "router output under skew"; the skew measure is
the maxvio of "Moonshot AI Open-Sources MoonEP for Expert Parallelism",
second paragraph):
  * logits[t, e] = N(0,1) + bias_e, one row per token t in rank-major order
    (t = r*S + s);
  * bias_e = alpha * z_e with z_e ~ N(0,1) per expert, or, for Zipf skew,
    bias = log(i^-s) for popularity rank i = 1..E assigned to experts through a
    seeded permutation;
  * top-K by logit, k = 0 the largest; equal logits go to the lower expert id;
  * gates = softmax over the K selected logits (max-subtracted, computed in
    float64, stored as float32).

Tensors: X ~ N(0,1) [R,S,H]; W ~ N(0, 1/H) [E,H,H']; dY ~ N(0,1) [N,H'];
rounded to the workload dtype (round-to-nearest-even for bf16).
"""
from __future__ import annotations

import numpy as np

# Stream tags: every tensor draws from its own seeded stream.
TAG_SKEW, TAG_LOGITS, TAG_PERM, TAG_X, TAG_W, TAG_DY, TAG_MISC = 1, 2, 3, 4, 5, 6, 7
TAG_WD = 8  # second projection's weights (the down projection of the gated FFN)


def _rng(seed: int, tag: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), int(sub)])


def expert_bias(E: int, seed: int, alpha: float = 0.0, zipf_s: float | None = None) -> np.ndarray:
    """Per-expert logit bias (float64 [E])."""
    if zipf_s is not None:
        perm = _rng(seed, TAG_PERM).permutation(E)
        bias = np.empty(E, dtype=np.float64)
        ranks = np.arange(1, E + 1, dtype=np.float64)
        bias[perm] = -zipf_s * np.log(ranks)  # expert perm[i-1] has popularity rank i
        return bias
    z = _rng(seed, TAG_SKEW).standard_normal(E)
    return alpha * z


def topk_route(logits: np.ndarray, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-K expert ids (descending logit, ties -> lower id) and softmax gates."""
    T, E = logits.shape
    cand = np.argpartition(-logits, K - 1, axis=1)[:, :K] if K < E else np.tile(np.arange(E), (T, 1))
    vals = np.take_along_axis(logits, cand, axis=1)
    # order the K candidates: larger logit first, then lower expert id
    order = np.lexsort((cand, -vals), axis=1)
    idx = np.take_along_axis(cand, order, axis=1)
    v = np.take_along_axis(vals, order, axis=1).astype(np.float64)
    v = v - v[:, :1]
    g = np.exp(v)
    g /= g.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), g.astype(np.float32)


def router_output(R: int, S: int, E: int, K: int, seed: int, alpha: float = 0.0,
                  zipf_s: float | None = None, chunk: int = 16384):
    """Returns (topk_idx int32 [R,S,K], gates float32 [R,S,K])."""
    bias = expert_bias(E, seed, alpha, zipf_s).astype(np.float32)
    T = R * S
    idx = np.empty((T, K), dtype=np.int32)
    gates = np.empty((T, K), dtype=np.float32)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        noise = _rng(seed, TAG_LOGITS, c0 // chunk).standard_normal((c1 - c0, E), dtype=np.float32)
        i, g = topk_route(noise + bias, K)
        idx[c0:c1] = i
        gates[c0:c1] = g
    return idx.reshape(R, S, K), gates.reshape(R, S, K)


def measured_maxvio(topk_idx: np.ndarray, E: int) -> float:
    """maxvio of a routing, used only to steer the skew calibration."""
    counts = np.bincount(topk_idx.reshape(-1), minlength=E)
    return float(E * int(counts.max())) / float(topk_idx.size) - 1.0


# ---------------------------------------------------------------- tensors (torch)

def _torch_seed(seed: int, tag: int, sub: int = 0) -> int:
    return (int(seed) * 1_000_003 + int(tag) * 10_007 + int(sub)) & 0x7FFF_FFFF_FFFF


def normal_tensor(shape, std: float, dtype: str, seed: int, tag: int, device="cpu", slices: int = 1):
    """N(0, std^2) tensor of `shape`, drawn in float32 on `device` and rounded to `dtype`.

    With ``slices > 1`` the leading dimension is drawn slice by slice, each
    from its own stream, to bound the float32 temporary.
    """
    import torch
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    out = torch.empty(shape, dtype=tdt, device=device)
    n0 = shape[0]
    per = max(1, (n0 + slices - 1) // slices)
    for i, a in enumerate(range(0, n0, per)):
        b = min(n0, a + per)
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(seed, tag, i))
        t = torch.randn((b - a,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[a:b].copy_(t)  # float32 -> bf16 copy rounds to nearest even
        del t
    return out


def layer_inputs(wl, seed: int, device="cpu", alpha: float | None = None, with_weights: bool = True,
                 with_dy: bool | None = None):
    """All inputs of one layer pass of workload `wl` (a synthetic.configs.Workload).

    Returns a dict with numpy routing (topk_idx, gates) and torch tensors
    X [R,S,H], W_home [E,H,Hp], dY [N,Hp] on `device`.
    """
    if alpha is None:
        alpha = wl.alpha if wl.alpha is not None else 0.0
    idx, gates = router_output(wl.R, wl.S, wl.E, wl.K, seed, alpha=alpha, zipf_s=wl.zipf_s)
    out = {"topk_idx": idx, "gates": gates, "alpha": alpha}
    out["X"] = normal_tensor((wl.R, wl.S, wl.H), 1.0, wl.dtype, seed, TAG_X, device, slices=wl.R)
    if with_weights and wl.Hp is not None:
        out["W_home"] = normal_tensor((wl.E, wl.H, wl.Hp), 1.0 / np.sqrt(wl.H), wl.dtype, seed, TAG_W,
                                      device, slices=wl.E)
    if with_dy is None:
        with_dy = wl.backward
    if with_dy and wl.Hp is not None:
        out["dY"] = normal_tensor((wl.N, wl.Hp), 1.0, wl.dtype, seed, TAG_DY, device, slices=wl.R)
    return out
