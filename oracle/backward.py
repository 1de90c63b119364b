"""Gradients of masked softmax attention, float64.  TEST INFRASTRUCTURE.

The backward pass the pages describe (page "Derive online softmax, prove it
is exact", section "What interviewers probe next": the forward keeps one
log-sum-exp per query and the backward recomputes P block by block from Q,
K and that scalar; page "Online softmax for a whole query tile, matrix
form", section "What interviewers probe next": the backward rebuilds the
normalized P = exp(S - LSE) with no running maximum; page "Online softmax",
section "Trade-offs and edge cases") computes the gradients of the forward
output.  Recomputing P block by block changes only the order of the sums, so
the oracle is the plain definition: for one (b, h) with O = P V,
P = softmax(sigma Q K^T) over the visible keys of each row, and an incoming
gradient dO,
    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)      (the softmax Jacobian)
    dQ = sigma dS K,   dK = sigma dS^T Q.
A row that sees no key has P = 0 and contributes nothing.  The masks and the
scale follow ``attention.attention_ref`` (sigma is the float32 scale the
library receives, widened exactly).
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask


def _probs(q: np.ndarray, k: np.ndarray, sigma: float, vis: np.ndarray) -> np.ndarray:
    """Row softmax of the visible scaled scores (zeros for rows with no key)."""
    s = np.where(vis, sigma * (q @ k.T), -np.inf)
    m = s.max(axis=1)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    return p / np.where(l > 0, l, 1.0)[:, None]


def attention_bwd_ref(Q, K, V, dO, scale: float, causal: bool = False, window: int = 0, kv_len=None,
                      heads=None):
    """dQ, dK, dV of masked softmax attention for the incoming gradient dO, float64.

    Q, K, V, dO: [B, H, N, d] (any float dtype, widened exactly).  ``heads``:
    None for every (b, h), or a list of (b, h) pairs (the others stay zero).
    Returns (dQ, dK, dV), each [B, H, N, d] float64.
    """
    Q, K, V, dO = (np.asarray(a) for a in (Q, K, V, dO))
    B, H, N, d = Q.shape
    sigma = float(np.float32(scale))
    dQ = np.zeros((B, H, N, d))
    dK = np.zeros((B, H, N, d))
    dV = np.zeros((B, H, N, d))
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    idx = np.arange(N)
    for b, h in pairs:
        klen = N if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        q, k, v, g = (a[b, h].astype(np.float64) for a in (Q, K, V, dO))
        p = _probs(q, k, sigma, visible_mask(idx, idx, N, klen, causal, window))
        dV[b, h] = p.T @ g
        dp = g @ v.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dQ[b, h] = sigma * (ds @ k)
        dK[b, h] = sigma * (ds.T @ q)
    return dQ, dK, dV


def attention_bwd_delta(O, dO):
    """D_i = sum_d dO_id O_id per query, float64 ([B, H, N]): equals sum_k P_ik dP_ik."""
    return (np.asarray(O, np.float64) * np.asarray(dO, np.float64)).sum(axis=-1)


def attention_bwd_error_bound(Q, K, V, dO, scale: float, causal: bool = False, window: int = 0, kv_len=None,
                              heads=None, u_operand: float = 2.0 ** -8, u_o: float = 2.0 ** -8,
                              u_out: float = 2.0 ** -8):
    """First-order bound on |computed - exact| of dQ, dK, dV, float64 (a tolerance, not a result).

    For a backward pass that (a) forms D_i = sum_c dO_ic O_ic from O rounded
    with relative error <= u_o, (b) rounds P (for dV) and dS (for dQ, dK)
    with relative error <= u_operand before the products, and (c) rounds
    each gradient once more with relative error <= u_out:
        dD_i      = u_o sum_c |dO_ic| |O_ic|
        err dV_jc <= u_operand sum_i P_ij |dO_ic| + u_out |dV_jc|
        err dQ_ic <= sigma (u_operand sum_j |dS_ij| |K_jc| + dD_i sum_j P_ij |K_jc|) + u_out |dQ_ic|
        err dK_jc <= sigma (u_operand sum_i |dS_ij| |Q_ic| + sum_i P_ij dD_i |Q_ic|) + u_out |dK_jc|
    (the error dD_i of D reaches dS_ij = P_ij (dP_ij - D_i) as P_ij dD_i).
    The defaults are bfloat16's unit roundoff 2^-8 (8 significand bits,
    round to nearest).  Accumulation error of the sums is not included: the
    caller adds its margin.  Bound is 0 exactly where the gradient is 0 for every input (a
    query that sees no key, a key no query sees).  Same arguments as
    attention_bwd_ref; returns (bQ, bK, bV), each [B, H, N, d].
    """
    Q, K, V, dO = (np.asarray(a) for a in (Q, K, V, dO))
    B, H, N, d = Q.shape
    sigma = float(np.float32(scale))
    bQ = np.zeros((B, H, N, d))
    bK = np.zeros((B, H, N, d))
    bV = np.zeros((B, H, N, d))
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    idx = np.arange(N)
    for b, h in pairs:
        klen = N if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        q, k, v, g = (a[b, h].astype(np.float64) for a in (Q, K, V, dO))
        p = _probs(q, k, sigma, visible_mask(idx, idx, N, klen, causal, window))
        o = p @ v
        dp = g @ v.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dd = u_o * (np.abs(g) * np.abs(o)).sum(axis=1)
        aq, ak, ads = np.abs(q), np.abs(k), np.abs(ds)
        bV[b, h] = u_operand * (p.T @ np.abs(g)) + u_out * np.abs(p.T @ g)
        bQ[b, h] = sigma * (u_operand * (ads @ ak) + dd[:, None] * (p @ ak)) + u_out * np.abs(sigma * (ds @ k))
        bK[b, h] = sigma * (u_operand * (ads.T @ aq) + p.T @ (dd[:, None] * aq)) + u_out * np.abs(sigma * (ds.T @ q))
    return bQ, bK, bV
