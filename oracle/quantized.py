"""Error model of FP8 (e4m3) attention, float64.  TEST INFRASTRUCTURE.

The pages name FP8 as FA3's precision step (page "Derive online softmax,
prove it is exact", "What interviewers probe next"; article "Online
softmax", "Trade-offs and edge cases") without fixing its numerics.  What
FP8 attention computes is the attention of the dequantized inputs
(``attention.attention_ref`` on code x descale), except that P is rounded to
e4m3 before P V and the matrix core accumulates its products with less than
float32 precision.  This module bounds that difference; it computes no
attention output itself.

For one query i with normalized probabilities p_ij (sum_j p_ij = 1) over
its visible keys, output O_i = sum_j p_ij v_j and score s_ij = sigma q_i.k_j:

  * P rounding: each P_j is rounded with relative error <= u_p (e4m3, round
    to nearest: 2^-4), or absolute error <= a_p max_{k in block(j)} P_k
    where it falls below e4m3's normal range.  The FP8 path rounds P in a
    power-of-two frame per (query, key block of 64 aligned at multiples of
    64) that maps the block's largest P into (128, 256], so a_p = 2^-17 (half
    of the 2^-9 subnormal step over 2^7), relative to the block's maximum.  Dividing by
    the sum of the rounded P, dO_c = sum_j dp_j (v_jc - O_c) to first order.
  * matrix-core accumulation: each product-sum has error <= kappa x the sum
    of |terms|; on the scores that is ds_ij = kappa sigma sum_c |q_ic k_jc|
    (dp_j = p_j ds_ij), on P V and on the sum of P it adds
    kappa (sum_j p_ij |v_jc| + |O_ic|).
  * the bf16 output: u_out |O_ic|.

worst-case  bO_ic = sum_j (u_p p_ij + a_p pblk_ij + p_ij ds_ij) |v_jc - O_ic|
                    + kappa (sum_j p_ij |v_jc| + |O_ic|) + u_out |O_ic|
statistical sO_ic = sqrt(sum_j (u_p^2 / 3) p_ij^2 (v_jc - O_ic)^2)
                    (the P rounding as independent errors uniform in +-u_p)
LSE         bL_i  = max_j (ds_ij + 2^-20 |s_ij|) + 1e-5
                    (LSE is formed from float32 P: only the score errors and
                    float32 rounding reach it).
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask


def attention_fp8_error_model(Q, K, V, scale: float, causal: bool = False, window: int = 0, kv_len=None,
                              heads=None, u_p: float = 2.0 ** -4, a_p: float = 2.0 ** -17,
                              kappa: float = 2.0 ** -13, u_out: float = 2.0 ** -8):
    """(bO, sO, bL): worst-case and statistical bounds on O, bound on LSE ([B, H, N, d], [B, H, N, d], [B, H, N]).

    Q, K, V: dequantized values [B, H, N, d].  Rows with no visible key get 0
    (their O and LSE are exact: 0 and -inf).  ``heads`` as in attention_bwd_ref.
    """
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    B, H, N, d = Q.shape
    sigma = float(np.float32(scale))
    bO = np.zeros((B, H, N, d))
    sO = np.zeros((B, H, N, d))
    bL = np.zeros((B, H, N))
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    idx = np.arange(N)
    for b, h in pairs:
        klen = N if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        q, k, v = Q[b, h], K[b, h], V[b, h]
        vis = visible_mask(idx, idx, N, klen, causal, window)
        s = np.where(vis, sigma * (q @ k.T), -np.inf)
        m = s.max(axis=1)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.where(vis, np.exp(s - m[:, None]), 0.0)
        l = e.sum(axis=1)
        p = e / np.where(l > 0, l, 1.0)[:, None]
        o = p @ v
        ds = np.where(vis, kappa * sigma * (np.abs(q) @ np.abs(k).T), 0.0)
        pblk = np.zeros((N, N))  # max of p over the 64-key block of each key
        for j0 in range(0, N, 64):
            pblk[:, j0:j0 + 64] = p[:, j0:j0 + 64].max(axis=1, keepdims=True)
        av = np.abs(v)
        # sum_j w_ij |v_jc - O_ic| for the weights w = u_p p + a_p pblk + p ds (zero where not visible)
        wgt = np.where(vis, u_p * p + a_p * pblk + p * ds, 0.0)
        dev = np.zeros((N, d))
        var = np.zeros((N, d))
        for r0 in range(0, N, 64):  # [rows, keys, d] over the visible key span of 64 rows
            r1 = min(N, r0 + 64)
            cols = np.nonzero(vis[r0:r1].any(axis=0))[0]
            if cols.size == 0:
                continue
            c0, c1 = cols[0], cols[-1] + 1
            diff = np.abs(v[None, c0:c1, :] - o[r0:r1, None, :])
            dev[r0:r1] = np.einsum("ij,ijc->ic", wgt[r0:r1, c0:c1], diff)
            var[r0:r1] = np.einsum("ij,ijc->ic", (u_p ** 2 / 3.0) * p[r0:r1, c0:c1] ** 2, diff ** 2)
        bO[b, h] = dev + kappa * (p @ av + np.abs(o)) + u_out * np.abs(o)
        sO[b, h] = np.sqrt(var)
        seen = vis.any(axis=1)
        bL[b, h] = np.where(seen, np.where(vis, ds + 2.0 ** -20 * np.abs(np.where(vis, s, 0.0)), 0.0).max(axis=1) + 1e-5,
                            0.0)
    return bO, sO, bL
