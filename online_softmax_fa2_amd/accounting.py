"""Algorithmic work of each workload, used to turn kernel times into rates.

Attention forward: 4 d FLOPs per visible (query, key) pair (2 d for the
score q . k, 2 d for adding p v), summed over the pairs the masks leave
visible; masked pairs a kernel may still touch are not counted.  Decode and
softmax: compulsory HBM bytes (every input element read once, every output
element written once).
"""
from __future__ import annotations

import numpy as np

# MI355X published peaks.
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA
NOMINAL_CLOCK_GHZ = 2.4     # the shader clock the published peaks assume
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3    # fp32 vector
PEAK_HBM_GBS = 8000.0       # HBM3E


def visible_pairs(N: int, kv_len: int | None, causal: bool, window: int) -> int:
    """Visible (query, key) pairs of one (b, h) slice: key j < kv_len, j <= i if causal, |i - j| < window."""
    L = N if kv_len is None else max(0, min(N, int(kv_len)))
    i = np.arange(N, dtype=np.int64)
    lo = np.zeros(N, np.int64) if window <= 0 else np.maximum(0, i - window + 1)
    hi = np.full(N, L - 1, np.int64)
    if causal:
        hi = np.minimum(hi, i)
    elif window > 0:
        hi = np.minimum(hi, i + window - 1)
    return int(np.maximum(0, hi - lo + 1).sum())


def attn_flops(B: int, H: int, N: int, d: int, causal: bool, window: int, kv_len=None) -> float:
    total = 0
    for b in range(B):
        kl = None if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        total += visible_pairs(N, kl, causal, window)
    return 4.0 * d * H * total


def attn_bwd_flops(B: int, H: int, N: int, d: int, causal: bool, window: int, kv_len=None) -> float:
    """Five d-long products per visible pair (S, dP, dV, dQ, dK): 10 d FLOPs, 2.5x the forward.

    The recomputation of S and dP that a split backward makes is not counted.
    """
    return 2.5 * attn_flops(B, H, N, d, causal, window, kv_len)


def decode_bytes(B: int, H: int, Nkv: int, d: int, elem: int = 2) -> int:
    """K and V read once (the q read and the float32 o write are < 0.01 % and not counted)."""
    return 2 * B * H * Nkv * d * elem


def softmax_bytes(rows: int, cols: int) -> int:
    """x read once and y written once, float32."""
    return 2 * rows * cols * 4


def topk_bytes(rows: int, cols: int, k: int) -> int:
    """x read once, float32, plus the k values and indices written per row."""
    return rows * cols * 4 + rows * k * 8


def fwd_bf16_d128_grid(B: int, H: int, N: int) -> int:
    """Work-items of one bf16 d = 128 forward launch: a 256-thread workgroup per 128-query tile of every head,
    the workgroup count rounded up to a multiple of the 8 XCDs.  Selects that launch's profile record."""
    tiles = B * H * ((N + 127) // 128)
    return (tiles + 7) // 8 * 8 * 256
