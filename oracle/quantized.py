"""Error bounds of FP8 (e4m3) attention, float64.  TEST INFRASTRUCTURE.

The pages name FP8 as FA3's precision step (page "Derive online softmax,
prove it is exact", "What interviewers probe next"; article "Online
softmax", "Trade-offs and edge cases") without fixing its numerics.  What
FP8 attention computes is the attention of the dequantized inputs
(``attention.attention_ref`` on code x descale), except that P is rounded to
e4m3 before P V and the matrix core accumulates its products with less than
float32 precision.  This module bounds that difference; it computes no
attention output itself.

For one query i with normalized probabilities p_ij (sum_j p_ij = 1) over
its visible keys, output O_i = sum_j p_ij v_j and score s_ij = sigma q_i.k_j,
a first-order bound per output element:

  bO_ic = sum_j (u_p p_ij + a_p r_ij + p_ij ds_ij) |v_jc - O_ic|
          + kappa (sum_j p_ij |v_jc| + |O_ic|) + u_out |O_ic|
  sO_ic = sqrt(sum_j (u_p^2 / 3) p_ij^2 (v_jc - O_ic)^2)   (statistical: the P
          roundings as independent errors uniform in +-u_p)
  bL_i  = max_j (ds_ij + 2^-20 |s_ij|) + 1e-5               (LSE is formed from
          float32 P: only score errors and float32 rounding reach it)
  with ds_ij = kappa sigma sum_c |q_ic k_jc| (dp_ij = p_ij ds_ij).

Terms: u_p is the relative rounding of P where it is a normal e4m3 value;
a_p r_ij its absolute rounding where it falls below the normal range (r_ij
is the probability that sets the rounding frame of p_ij); kappa the
matrix core's accumulation error as a fraction of the sum of |terms|; u_out
the bf16 rounding of O.  Dividing O by the sum of the rounded P, a P error
dp_j moves O_c by dp_j (v_jc - O_c) to first order.

Two parameter sets:

``attention_fp8_error_bound`` -- the parity gate.  Every term follows from
the e4m3 and bf16 formats and one stated reading, none from a kernel's
design or a measurement:
  * u_p = 2^-4: e4m3 keeps 3 fraction bits, so round-to-nearest of a normal
    value errs by at most half a unit in the 4th significant bit;
  * a_p = 2^-10, r_ij = max_k p_ik: e4m3's smallest step is 2^-9 (its
    subnormal spacing), so rounding errs by at most 2^-10 in code units.  A
    kernel that rounds P = exp(s - m) with its running reference m mapped to
    at least 1 code unit (the plainest reading: P in (0, 1] rounded as it
    is) errs by at most 2^-10 x the reference's P, and the reference never
    exceeds the row's largest P;
  * kappa = 2^-8 (reading R20): FP8 matrix cores do not promise float32
    accumulation; the bar takes each product sum to be at least as accurate
    as one rounding of its sum of |terms| to bf16 precision (8 significant
    bits).  Float32 accumulation (64 terms: 2^-18) meets it with room;
  * u_out = 2^-8: the bf16 output's unit roundoff.

``attention_fp8_error_model`` -- a diagnostic, tighter bound for the frame
that attn_fwd_fp8 chooses (each 64-key block aligned at multiples of 64 is
scaled so its largest P lands in (128, 256], so a_p = 2^-17 of that block's
largest p) and kappa = 2^-13.  It is reported beside the gate, never used
as the gate.
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask


def _fp8_bounds(Q, K, V, scale, causal, window, kv_len, heads, u_p, a_p, kappa, u_out, frame):
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
        if frame == "row":
            ref = np.broadcast_to(p.max(axis=1, keepdims=True), p.shape)
        else:  # the largest p of each 64-key block aligned at multiples of 64
            ref = np.zeros((N, N))
            for j0 in range(0, N, 64):
                ref[:, j0:j0 + 64] = p[:, j0:j0 + 64].max(axis=1, keepdims=True)
        av = np.abs(v)
        # sum_j w_ij |v_jc - O_ic| for the weights w = u_p p + a_p ref + p ds (zero where not visible)
        wgt = np.where(vis, u_p * p + a_p * ref + p * ds, 0.0)
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


def attention_fp8_error_bound(Q, K, V, scale: float, causal: bool = False, window: int = 0, kv_len=None,
                              heads=None, u_p: float = 2.0 ** -4, a_p: float = 2.0 ** -10,
                              kappa: float = 2.0 ** -8, u_out: float = 2.0 ** -8):
    """(bO, sO, bL) of the gate: worst-case and statistical bounds on O, bound on LSE.

    Shapes [B, H, N, d], [B, H, N, d], [B, H, N].  Q, K, V are the
    dequantized values.  Rows with no visible key get 0 (their O and LSE
    are exact: 0 and -inf).  ``heads``: None (all) or a list of (b, h).
    The defaults are the format-derived terms of the module docstring.
    """
    return _fp8_bounds(Q, K, V, scale, causal, window, kv_len, heads, u_p, a_p, kappa, u_out, "row")


def attention_fp8_error_model(Q, K, V, scale: float, causal: bool = False, window: int = 0, kv_len=None,
                              heads=None, u_p: float = 2.0 ** -4, a_p: float = 2.0 ** -17,
                              kappa: float = 2.0 ** -13, u_out: float = 2.0 ** -8):
    """Diagnostic (bO, sO, bL) for a per-(query, 64-key block) frame with the block's largest P in (128, 256]."""
    return _fp8_bounds(Q, K, V, scale, causal, window, kv_len, heads, u_p, a_p, kappa, u_out, "block")
