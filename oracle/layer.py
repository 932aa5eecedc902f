"""Oracle: the data-moving and arithmetic stages of the layer, forward and backward, and the full
gated expert FFN built from them (test infrastructure).

Plain numpy, float64 arithmetic on whatever values the caller passes (the
tests pass bf16-rounded inputs converted to float64).

The method only relocates work: a slot row is a bitwise copy of a home row
and a direct read of a home row gives the same numbers ([P2] "Core technique"
and "Memory contract and weight layout"), so every float result here also has
a plan-independent definition (``moe_forward``, ``expert_weight_grad``) that
the tests hold the planned chain to.

Layout contract ([P2] "Memory contract and weight layout"):
  * Xp, Yp, dY: [R*S*K, D] rows; rank r owns rows [r*P, (r+1)*P), P = S*K;
    inside a rank, group g owns rows [cu[r,g], cu[r,g+1]).
  * Rank r's weight row g is W_home[g] for g < E and W_slots[r, g-E] for
    g >= E.
  * Gradients are float32 buffers of the same shapes; rows [E, E+B) of each
    rank are its reduce buffers, viewed together as [R, B, H, H'].
"""
from __future__ import annotations

import numpy as np


def dispatch(X: np.ndarray, dest_idx: np.ndarray) -> np.ndarray:
    """Fused permute: row dest_idx[r,s,k] of the output is token (r, s) of X ([P2] "Core technique")."""
    R, S, H = X.shape
    K = dest_idx.shape[2]
    Xp = np.empty((R * S * K, H), dtype=X.dtype)
    Xp[np.asarray(dest_idx).reshape(-1)] = np.repeat(X.reshape(R * S, H), K, axis=0)
    return Xp


def prefetch(W_home: np.ndarray, slot_expert: np.ndarray, W_slots: np.ndarray | None = None) -> np.ndarray:
    """Slot j of rank r receives a copy of home expert slot_expert[r, j]; -1 leaves it as is."""
    R, B = slot_expert.shape
    E, H, Hp = W_home.shape
    out = np.zeros((R, B, H, Hp), dtype=W_home.dtype) if W_slots is None else W_slots.copy()
    for r in range(R):
        for j in range(B):
            if slot_expert[r, j] >= 0:
                out[r, j] = W_home[slot_expert[r, j]]
    return out


def rank_weight(W_home, W_slots, r: int, g: int):
    """Weight row g of rank r's logical [E+B, H, H'] tensor."""
    E = W_home.shape[0]
    return W_home[g] if g < E else W_slots[r, g - E]


def row_group(cu_seqlens: np.ndarray, P: int, rows: np.ndarray):
    """(rank, group) of each dispatched row."""
    rows = np.asarray(rows, dtype=np.int64)
    ranks = rows // P
    local = rows % P
    groups = np.array([np.searchsorted(cu_seqlens[r], l, side="right") - 1 for r, l in zip(ranks, local)],
                      dtype=np.int64)
    return ranks, groups


def group_gemm(Xp, W_home, W_slots, cu_seqlens, P: int, rows=None, ranks=None) -> np.ndarray:
    """Yp[rows of group g on rank r] = Xp[those rows] @ W_r[g] ([P2] "Memory contract": VM group GEMM).

    With ``rows`` given, returns only those output rows (Xp must then be the full
    buffer or any array indexable by the row ids).  With ``ranks`` given, returns
    the whole buffers of those ranks, one after the other ([len(ranks)*P, H']).
    """
    R = cu_seqlens.shape[0]
    G = cu_seqlens.shape[1] - 1
    Hp = W_home.shape[2]
    if rows is None:
        rs = range(R) if ranks is None else list(ranks)
        Y = np.zeros((len(rs) * P, Hp), dtype=np.float64)
        for i, r in enumerate(rs):
            for g in range(G):
                a, b = r * P + cu_seqlens[r, g], r * P + cu_seqlens[r, g + 1]
                if b > a:
                    o = i * P + cu_seqlens[r, g]
                    Y[o:o + b - a] = (np.asarray(Xp[a:b], dtype=np.float64)
                                      @ np.asarray(rank_weight(W_home, W_slots, r, g), dtype=np.float64))
        return Y
    ranks, groups = row_group(cu_seqlens, P, rows)
    Y = np.zeros((len(rows), Hp), dtype=np.float64)
    for i, (row, r, g) in enumerate(zip(rows, ranks, groups)):
        Y[i] = Xp[row].astype(np.float64) @ rank_weight(W_home, W_slots, r, g).astype(np.float64)
    return Y


def combine(Yp: np.ndarray, dest_idx: np.ndarray, gates: np.ndarray, tokens=None) -> np.ndarray:
    """Fused unpermute: out[r,s] = sum_k gate[r,s,k] * Yp[dest_idx[r,s,k]] ([P2] "Core technique").

    ``tokens`` (flat r*S+s ids) restricts the result to those tokens.
    """
    R, S, K = dest_idx.shape
    D = Yp.shape[1]
    dflat = np.asarray(dest_idx).reshape(R * S, K)
    gflat = np.asarray(gates, dtype=np.float64).reshape(R * S, K)
    tok = np.arange(R * S) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(tok), D), dtype=np.float64)
    for k in range(K):
        out += gflat[tok, k:k + 1] * Yp[dflat[tok, k]].astype(np.float64)
    return out if tokens is not None else out.reshape(R, S, D)


def combine_abs(Yp, dest_idx, gates, tokens=None) -> np.ndarray:
    """sum_k |gate * y|: the scale of the combine sum, used for its error bound."""
    return combine(np.abs(np.asarray(Yp, dtype=np.float64)), dest_idx, np.abs(gates), tokens)


def wgrad(Xp, dY, cu_seqlens, P: int, dW_home, dW_slots, dtype=np.float64):
    """dW_r[g] += Xp[rows_g]^T @ dY[rows_g] for every rank and group ([P2] "Memory contract").

    Groups g < E add into dW_home[g] (ranks in ascending order: the home rank's
    kept rows and other ranks' direct reads of that home row); slot groups add
    into that rank's reduce buffer dW_slots[r, g-E].  Works in place.
    """
    R = cu_seqlens.shape[0]
    E = dW_home.shape[0]
    G = cu_seqlens.shape[1] - 1
    for g in range(G):
        for r in range(R):
            a, b = r * P + cu_seqlens[r, g], r * P + cu_seqlens[r, g + 1]
            if b <= a:
                continue
            contrib = (Xp[a:b].astype(np.float64).T @ dY[a:b].astype(np.float64)).astype(dtype)
            if g < E:
                dW_home[g] += contrib
            else:
                dW_slots[r, g - E] += contrib
    return dW_home, dW_slots


def reduce_grad(slot_expert, dW_home, dW_slots, dtype=np.float64):
    """Fold every consumed reduce-buffer slot into its home expert's gradient, then zero it.

    For each expert, ranks are visited in ascending order and the running value
    starts from the home gradient ([P2] "Memory contract": reduce_grad reads the
    slots of all ranks, accumulates into the parameter gradient and clears the
    consumed slots).  With dtype=float32 the additions are float32 in exactly
    this order.  Works in place.
    """
    R, B = slot_expert.shape
    E = dW_home.shape[0]
    for e in range(E):
        acc = None
        for r in range(R):
            for j in range(B):
                if slot_expert[r, j] == e:
                    if acc is None:
                        acc = dW_home[e].astype(dtype)
                    acc = (acc + dW_slots[r, j].astype(dtype)).astype(dtype)
                    dW_slots[r, j] = 0
        if acc is not None:
            dW_home[e] = acc
    return dW_home, dW_slots


# ------------------------------------------------------------------ backward of the data path
#
# The pages say the backward pass runs through the same buffers and that the gradients of the
# redundant experts are folded back to their home experts ([P2] "Core technique"; [P3] third
# paragraph); they say nothing more about the data gradients.  Read plainly, these are the chain
# rule of dispatch -> group GEMM -> combine, each the transpose of its forward stage.

def combine_backward(dout: np.ndarray, Yp: np.ndarray, dest_idx: np.ndarray, gates: np.ndarray):
    """Gradients of out = combine(Yp, dest_idx, gates) given dout = d(loss)/d(out):

    dYp[dest_idx[r,s,k]] = gate[r,s,k] * dout[r,s]   (every row of Yp is the destination of one pair)
    dgate[r,s,k] = sum_n dout[r,s,n] * Yp[dest_idx[r,s,k], n]
    """
    R, S, K = dest_idx.shape
    D = dout.shape[2]
    dflat = np.asarray(dest_idx).reshape(R * S, K)
    gf = np.asarray(gates, dtype=np.float64).reshape(R * S, K)
    do = np.asarray(dout, dtype=np.float64).reshape(R * S, D)
    dYp = np.zeros((Yp.shape[0], D), dtype=np.float64)
    dgate = np.zeros((R * S, K), dtype=np.float64)
    for k in range(K):
        dYp[dflat[:, k]] = gf[:, k:k + 1] * do
        dgate[:, k] = np.sum(do * Yp[dflat[:, k]].astype(np.float64), axis=1)
    return dYp, dgate.reshape(R, S, K)


def group_gemm_dgrad(dYp, W_home, W_slots, cu_seqlens, P: int, rows=None, ranks=None) -> np.ndarray:
    """dXp[rows of group g on rank r] = dYp[those rows] @ W_r[g]^T: the gradient of the VM group GEMM
    with respect to its input, through the same groups and the same weight rows (home or slot).

    With ``rows`` given, returns only those output rows; with ``ranks`` given, the whole buffers of
    those ranks, one after the other ([len(ranks)*P, H]).
    """
    R = cu_seqlens.shape[0]
    G = cu_seqlens.shape[1] - 1
    H = W_home.shape[1]
    if rows is None:
        rs = range(R) if ranks is None else list(ranks)
        dX = np.zeros((len(rs) * P, H), dtype=np.float64)
        for i, r in enumerate(rs):
            for g in range(G):
                a, b = r * P + cu_seqlens[r, g], r * P + cu_seqlens[r, g + 1]
                if b > a:
                    o = i * P + cu_seqlens[r, g]
                    dX[o:o + b - a] = (np.asarray(dYp[a:b], dtype=np.float64)
                                       @ np.asarray(rank_weight(W_home, W_slots, r, g), dtype=np.float64).T)
        return dX
    ranks, groups = row_group(cu_seqlens, P, rows)
    dX = np.zeros((len(rows), H), dtype=np.float64)
    for i, (row, r, g) in enumerate(zip(rows, ranks, groups)):
        dX[i] = rank_weight(W_home, W_slots, r, g).astype(np.float64) @ dYp[row].astype(np.float64)
    return dX


def dispatch_backward(dXp: np.ndarray, dest_idx: np.ndarray, tokens=None) -> np.ndarray:
    """Gradient of the fused permute: dX[r,s] = sum_k dXp[dest_idx[r,s,k]], k ascending.

    ``tokens`` (flat r*S+s ids) restricts the result to those tokens.
    """
    R, S, K = dest_idx.shape
    H = dXp.shape[1]
    dflat = np.asarray(dest_idx).reshape(R * S, K)
    tok = np.arange(R * S) if tokens is None else np.asarray(tokens)
    dX = np.zeros((len(tok), H), dtype=np.float64)
    for k in range(K):
        dX += dXp[dflat[tok, k]].astype(np.float64)
    return dX if tokens is not None else dX.reshape(R, S, H)


# ------------------------------------------------------------------ full expert FFN
#
# The pages call the weight tensor one "expert projection" and ask for one such tensor per
# projection ([P2] "Memory contract and weight layout"); they do not name the FFN.  Read plainly
# (the usual gated MoE expert): a gate|up projection [E+B, H, 2H'] whose first H' output columns are
# the gate and last H' the up projection, act = silu(gate) * up, and a down projection
# [E+B, H', H]; each projection runs through the same plan, slots and group GEMM.

def silu(g):
    """g * sigmoid(g), from exp of a non-positive argument only (no overflow)."""
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig


def swiglu(Ygu: np.ndarray) -> np.ndarray:
    """act = silu(gate) * up for rows [gate (H') | up (H')]."""
    Y = np.asarray(Ygu, dtype=np.float64)
    Hp = Y.shape[1] // 2
    return silu(Y[:, :Hp]) * Y[:, Hp:]


def swiglu_backward(Ygu: np.ndarray, dA: np.ndarray) -> np.ndarray:
    """Gradient of swiglu: d gate = dA * up * s * (1 + g * (1 - s)) with s = sigmoid(g), d up = dA * silu(g);
    returned as rows [d gate | d up]."""
    Y = np.asarray(Ygu, dtype=np.float64)
    Hp = Y.shape[1] // 2
    g, u = Y[:, :Hp], Y[:, Hp:]
    d = np.asarray(dA, dtype=np.float64)
    e = np.exp(-np.abs(g))
    s = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return np.concatenate([d * u * s * (1.0 + g * (1.0 - s)), d * g * s], axis=1)


# ------------------------------------------------------------------ plain definitions

def moe_forward(X, W_home, topk_idx, gates, tokens=None) -> np.ndarray:
    """Plain MoE projection: out[r,s] = sum_k gate[r,s,k] * X[r,s] @ W[topk_idx[r,s,k]]."""
    R, S, H = X.shape
    K = topk_idx.shape[2]
    Xf = X.reshape(R * S, H)
    ids = np.asarray(topk_idx).reshape(R * S, K)
    gf = np.asarray(gates, dtype=np.float64).reshape(R * S, K)
    tok = np.arange(R * S) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(tok), W_home.shape[2]), dtype=np.float64)
    for i, t in enumerate(tok):
        x = Xf[t].astype(np.float64)
        for k in range(K):
            out[i] += gf[t, k] * (x @ W_home[ids[t, k]].astype(np.float64))
    return out if tokens is not None else out.reshape(R, S, -1)


def expert_weight_grad(X, dY_of_pair, topk_idx, E: int, experts=None) -> np.ndarray:
    """Plain expert weight gradient: dW[e] = sum over pairs (t,k) with expert e of x_t^T dy_(t,k).

    ``experts`` restricts the result to those experts ([len(experts), H, H'], in that order); dY_of_pair
    then needs only row indexing by pair ids.
    """
    R, S, H = X.shape
    K = topk_idx.shape[2]
    Xf = X.reshape(R * S, H)
    ids = np.asarray(topk_idx).reshape(R * S * K)
    sel = range(E) if experts is None else list(experts)
    dW = np.zeros((len(sel), H, dY_of_pair.shape[1]), dtype=np.float64)
    for i, e in enumerate(sel):
        q = np.nonzero(ids == e)[0]
        if len(q):
            dW[i] = np.asarray(Xf[q // K], dtype=np.float64).T @ np.asarray(dY_of_pair[q], dtype=np.float64)
    return dW


def moe_forward_rows(Xt, W_home, ids, gates):
    """moe_forward for a block of tokens given as rows: out[i] = sum over k ascending of
    gate[i,k] * Xt[i] @ W[ids[i,k]], and the scale sum_k |gate[i,k] * Xt[i] @ W[ids[i,k]]| of that sum.

    Each (i, k) term is one row of a matmul over the tokens that chose the same expert (each expert's
    weights are read once); the terms are kept apart until the k-ascending sum.
    """
    Xt = np.asarray(Xt, dtype=np.float64)
    ids = np.asarray(ids)
    g = np.asarray(gates, dtype=np.float64)
    n, K = ids.shape
    terms = np.zeros((K, n, W_home.shape[2]), dtype=np.float64)
    for e in np.unique(ids):
        i, k = np.nonzero(ids == e)
        terms[k, i] = g[i, k][:, None] * (Xt[i] @ np.asarray(W_home[e], dtype=np.float64))
    out = terms[0].copy()
    for k in range(1, K):
        out += terms[k]
    return out, np.abs(terms).sum(axis=0)


def moe_input_grad_rows(dY_rows, W_home, ids):
    """Gradient of the planned layer's input for a block of tokens, through dgrad and the permute's
    backward: dX[i] = sum over k ascending of dY_rows[i,k] @ W[ids[i,k]]^T, where dY_rows[i,k] is the
    gradient row of pair (i, k) in the dispatched buffer; also the scale sum_k |that term|.  One matmul
    per expert over the pairs that chose it; terms kept apart until the k-ascending sum."""
    dY_rows = np.asarray(dY_rows, dtype=np.float64)
    ids = np.asarray(ids)
    n, K = ids.shape
    terms = np.zeros((K, n, W_home.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        i, k = np.nonzero(ids == e)
        terms[k, i] = dY_rows[i, k] @ np.asarray(W_home[e], dtype=np.float64).T
    out = terms[0].copy()
    for k in range(1, K):
        out += terms[k]
    return out, np.abs(terms).sum(axis=0)


def moe_backward(X, W_home, topk_idx, gates, dout):
    """Plain gradients of moe_forward given dout:

    dX[r,s] = sum_k gate[r,s,k] * W[e] @ dout[r,s]      (e = topk_idx[r,s,k])
    dgate[r,s,k] = dout[r,s] . (X[r,s] @ W[e])
    """
    R, S, H = X.shape
    K = topk_idx.shape[2]
    Xf = X.reshape(R * S, H).astype(np.float64)
    ids = np.asarray(topk_idx).reshape(R * S, K)
    gf = np.asarray(gates, dtype=np.float64).reshape(R * S, K)
    do = np.asarray(dout, dtype=np.float64).reshape(R * S, -1)
    dX = np.zeros((R * S, H), dtype=np.float64)
    dgate = np.zeros((R * S, K), dtype=np.float64)
    for t in range(R * S):
        for k in range(K):
            w = W_home[ids[t, k]].astype(np.float64)
            dX[t] += gf[t, k] * (w @ do[t])
            dgate[t, k] = do[t] @ (Xf[t] @ w)
    return dX.reshape(R, S, H), dgate.reshape(R, S, K)


def moe_ffn_forward(X, W_gu, W_down, topk_idx, gates) -> np.ndarray:
    """Plain gated-expert MoE: out[r,s] = sum_k gate * ffn_e(X[r,s]),
    ffn_e(x) = swiglu(x @ W_gu[e]) @ W_down[e]."""
    R, S, H = X.shape
    K = topk_idx.shape[2]
    Xf = X.reshape(R * S, H).astype(np.float64)
    ids = np.asarray(topk_idx).reshape(R * S, K)
    gf = np.asarray(gates, dtype=np.float64).reshape(R * S, K)
    out = np.zeros((R * S, W_down.shape[2]), dtype=np.float64)
    for t in range(R * S):
        for k in range(K):
            e = ids[t, k]
            a = swiglu((Xf[t] @ W_gu[e].astype(np.float64))[None, :])[0]
            out[t] += gf[t, k] * (a @ W_down[e].astype(np.float64))
    return out.reshape(R, S, -1)
