"""Direct (non-streaming) softmax attention in float64.  TEST INFRASTRUCTURE.

Follows page "Derive online softmax, prove it is exact", section "A strong
answer": for one query, o is the softmax-weighted sum of the value rows,
with scores s_i = q . k_i scaled by 1/sqrt(d) (here by the caller's scale),
and the maximum subtracted before exponentiating, which changes nothing
mathematically and keeps every exponent <= 0.  The method on the pages
reaches exactly this result (same page, the induction argument; page
"Online softmax for a whole query tile, matrix form", section "A strong
answer": each row of the tile is the single-query recurrence), so the
oracle is the definition itself, not the recurrence.

Masks (page "Online softmax for a whole query tile, matrix form", sections
"How to approach it" and "A strong answer": causal, sliding window and
padding) use these readings where the pages name a mask without fixing its
convention:
  * causal: key j is visible to query i iff j <= i;
  * sliding window W > 0: visible iff |i - j| < W (the diagonal counts; with
    causal masking this is the W most recent keys including the query's own);
    W <= 0 disables the window;
  * right padding: keys j >= kv_len[b] are masked; queries at padded
    positions are still computed from whatever keys they see;
  * a query that sees no key at all has O = 0 and LSE = -inf (an empty sum).

LSE is the natural log of the row's sum of exp(score), in the units of the
scaled score (page "Derive online softmax, prove it is exact", section "What
interviewers probe next": the backward pass keeps m + log l per query).
"""
from __future__ import annotations

import numpy as np


def visible_mask(rows: np.ndarray, cols: np.ndarray, N: int, kv_len_b: int,
                 causal: bool, window: int) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: may query ``rows[a]`` see key ``cols[c]``?"""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    vis = (j >= 0) & (j < N) & (j < kv_len_b) & (i == i)  # (i == i) broadcasts to [rows, cols]
    if causal:
        vis = vis & (j <= i)
    if window > 0:
        vis = vis & (np.abs(i - j) < window)
    return vis


def visible_count(N: int, kv_len_b: int, causal: bool, window: int) -> int:
    """Number of visible (query, key) pairs of one (b, h) slice, by enumeration."""
    total = 0
    cols = np.arange(N)
    for r0 in range(0, N, 1024):
        rows = np.arange(r0, min(N, r0 + 1024))
        total += int(visible_mask(rows, cols, N, kv_len_b, causal, window).sum())
    return total


def _attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, sigma: float,
                 vis: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Safe softmax attention of the query rows ``q`` over all keys, masked by ``vis``.

    q [R, d], k and v [N, d] (float64), vis [R, N] bool.  Returns O [R, d]
    and LSE [R].
    """
    s = sigma * (q @ k.T)  # [R, N] scores
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)  # -inf for rows with no visible key
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    l = p.sum(axis=1)
    o = p @ v
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(empty[:, None], 0.0, o / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return o, lse


def attention_ref(Q, K, V, scale: float, causal: bool = False, window: int = 0,
                  kv_len=None, rows=None, chunk: int = 512):
    """O and LSE of masked softmax attention, float64.

    Q, K, V: [B, H, N, d] arrays of any float dtype; each element is widened
    exactly to float64.  ``scale`` is used as the float32 number the library
    receives (sigma = float64(float32(scale))).  ``kv_len``: None or [B]
    integers.  ``rows``: None for every query, or a 1-D array of query
    indices (the same for every (b, h)).  Returns ``(O, LSE)`` with shapes
    [B, H, R, d] and [B, H, R].
    """
    Q = np.asarray(Q)
    K = np.asarray(K)
    V = np.asarray(V)
    B, H, N, d = Q.shape
    sigma = float(np.float32(scale))
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, H, len(rows), d), np.float64)
    LSE = np.zeros((B, H, len(rows)), np.float64)
    cols = np.arange(N)
    for b in range(B):
        klen = N if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        for h in range(H):
            k = K[b, h].astype(np.float64)
            v = V[b, h].astype(np.float64)
            for c0 in range(0, len(rows), chunk):
                r = rows[c0:c0 + chunk]
                vis = visible_mask(r, cols, N, klen, causal, window)
                o, lse = _attend_rows(Q[b, h, r].astype(np.float64), k, v, sigma, vis)
                O[b, h, c0:c0 + chunk] = o
                LSE[b, h, c0:c0 + chunk] = lse
    return O, LSE


def decode_ref(q, K, V, heads=None):
    """Single-query attention per (b, h), non-causal, unmasked, float64.

    q [B, H, d], K, V [B, H, Nkv, d].  The scale is 1/sqrt(d) rounded once to
    float32 (page "Derive online softmax, prove it is exact", section "A
    strong answer": scores are q . k / sqrt(d)).  Splitting the keys into
    chunks and merging partial (m, l, a) triples reaches exactly this value
    (same page, the batch-1 decoding follow-up), so the oracle does not
    split.  ``heads``: None for all, or a list of (b, h) pairs.  Returns o
    [B, H, d] (zeros for heads not requested).
    """
    q = np.asarray(q)
    B, H, d = q.shape
    Nkv = K.shape[2]
    sigma = float(np.float32(1.0 / np.sqrt(d)))
    o = np.zeros((B, H, d), np.float64)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    vis = np.ones((1, Nkv), dtype=bool)
    for b, h in pairs:
        ob, _ = _attend_rows(q[b, h][None, :].astype(np.float64), np.asarray(K[b, h], np.float64),
                             np.asarray(V[b, h], np.float64), sigma, vis)
        o[b, h] = ob[0]
    return o
