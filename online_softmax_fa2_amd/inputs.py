"""Seeded synthetic inputs for the attention, decode and row-softmax workloads.

This module is shared by the GPU tests, the benchmark and the CPU oracle's
tests, so it deliberately holds none of the method's arithmetic: only random
draws, the round-to-nearest-even conversion of inputs to bfloat16, the
scaling of a fixed key subset by 8 (exact in bfloat16) and the workload
shapes.  Nothing here computes a score, a maximum, an exponential or a sum.

Recipe (every draw is reproducible from the seed list alone):
  * attention: for each (b, h) slice, ``numpy.random.default_rng([seed, b, h])``
    draws Q, K, V in that order with ``standard_normal(dtype=float32)``;
  * extra draws (the key subset that is scaled by 8) use
    ``default_rng([seed, 1000])``;
  * the incoming gradient dO of the backward pass: for each (b, h) slice,
    ``default_rng([seed, 2000, b, h])`` draws ``standard_normal(float32)``;
  * FP8 attention: the float32 Q, K, V of the attention recipe (big keys
    included), each tensor divided by its descale max|x| / 448 (float32,
    nudged up until no quotient exceeds 448) and rounded to e4m3 (OCP e4m3fn,
    round to nearest even); the oracle sees code x descale in float64;
  * row softmax: ``default_rng([seed, r // 256])`` draws blocks of 256 rows of
    ``standard_normal(float32)`` which are multiplied by the workload's sigma
    (4, a power of two, so the product is exact).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# bfloat16 conversion of inputs (host side, round to nearest even)
# ---------------------------------------------------------------------------


def bf16_round(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round finite float32 values to bfloat16, ties to even.

    Returns ``(bits, values)``: the bfloat16 bit patterns as uint16 and the
    same numbers widened back to float32 (exactly representable).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    bits = ((u + bias) >> 16).astype(np.uint16)
    values = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits, values


def e4m3_round(y: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round finite values with |y| <= 448 to OCP e4m3fn, ties to even: (codes uint8, values float64).

    e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals below
    2^-6 in steps of 2^-9; 448 is the largest finite value (0x7E).
    """
    y = np.asarray(y, np.float64)
    if not np.all(np.isfinite(y)) or np.abs(y).max(initial=0.0) > 448.0:
        raise ValueError("e4m3_round: values must be finite with |y| <= 448")
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3.0)
    q = np.rint(a / quantum) * quantum  # exact division by a power of two; rint ties to even
    E = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    sub = q < 2.0 ** -6
    mant = np.where(sub, q / 2.0 ** -9, q / np.exp2(E) * 8.0 - 8.0)
    field = np.where(sub, 0.0, E + 7.0)
    codes = (np.where(y < 0, 128, 0) + field.astype(np.int64) * 8 + mant.astype(np.int64)).astype(np.uint8)
    codes = np.where(q == 0, 0, codes).astype(np.uint8)
    return codes, np.where(y < 0, -q, q)


def e4m3_descale(x: np.ndarray) -> float:
    """float32 d with |x| / d <= 448 for every element (d = max|x| / 448, nudged up)."""
    amax = float(np.abs(np.asarray(x, np.float64)).max(initial=0.0))
    if amax == 0.0:
        return 1.0
    d = np.float32(amax / 448.0)
    while amax / float(d) > 448.0:
        d = np.nextafter(d, np.float32(np.inf))
    return float(d)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 values exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Attention inputs
# ---------------------------------------------------------------------------


@dataclass
class AttnInputs:
    """Q, K, V as float32 values (bf16-representable when dtype == 'bf16')."""

    q: np.ndarray  # [B, H, N, d] float32
    k: np.ndarray
    v: np.ndarray
    dtype: str  # 'f32' or 'bf16'
    scale: float  # the float32 scale the library receives
    causal: bool = False
    window: int = 0
    kv_len: np.ndarray | None = None  # [B] int32 or None
    big_keys: np.ndarray | None = None  # key positions scaled by 8, if any
    q_bits: np.ndarray | None = field(default=None, repr=False)  # uint16 when bf16
    k_bits: np.ndarray | None = field(default=None, repr=False)
    v_bits: np.ndarray | None = field(default=None, repr=False)


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded once to float32."""
    return float(np.float32(1.0 / math.sqrt(d)))


def attn_inputs(B: int, H: int, N: int, d: int, *, dtype: str = "bf16", seed: int = 0,
                causal: bool = False, window: int = 0, kv_len=None,
                n_big_keys: int = 0, scale: float | None = None,
                q_shift: float = 0.0, k_shift: float = 0.0, std: float = 1.0) -> AttnInputs:
    """Draw Q, K, V of shape [B, H, N, d] from N(0, std^2) per (b, h) slice.

    ``n_big_keys`` key positions (shared by all batches and heads, drawn
    without replacement from ``default_rng([seed, 1000])``) are multiplied by
    8 after rounding, which is exact in bfloat16.  ``q_shift``/``k_shift``
    add a constant to every element before rounding (used to build rows whose
    scores sit far from zero).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    shape = (B, H, N, d)
    q = np.empty(shape, np.float32)
    k = np.empty(shape, np.float32)
    v = np.empty(shape, np.float32)
    for b in range(B):
        for h in range(H):
            rng = np.random.default_rng([seed, b, h])
            q[b, h] = rng.standard_normal((N, d), dtype=np.float32) * np.float32(std) + np.float32(q_shift)
            k[b, h] = rng.standard_normal((N, d), dtype=np.float32) * np.float32(std) + np.float32(k_shift)
            v[b, h] = rng.standard_normal((N, d), dtype=np.float32) * np.float32(std)
    out = AttnInputs(q=q, k=k, v=v, dtype=dtype,
                     scale=default_scale(d) if scale is None else float(np.float32(scale)),
                     causal=causal, window=window)
    if dtype == "bf16":
        out.q_bits, out.q = bf16_round(q)
        out.k_bits, out.k = bf16_round(k)
        out.v_bits, out.v = bf16_round(v)
    if n_big_keys:
        pos = np.sort(np.random.default_rng([seed, 1000]).choice(N, size=n_big_keys, replace=False))
        out.big_keys = pos
        out.k[:, :, pos, :] *= np.float32(8.0)
        if dtype == "bf16":
            out.k_bits, _ = bf16_round(out.k)  # exact: a power-of-two multiple
    if kv_len is not None:
        out.kv_len = np.asarray(kv_len, dtype=np.int32).reshape(B)
    return out


@dataclass
class Fp8AttnInputs:
    """e4m3 codes of Q, K, V with their float32 descales, and the dequantized values (float64)."""

    q8: np.ndarray  # [B, H, N, d] uint8
    k8: np.ndarray
    v8: np.ndarray
    qd: float
    kd: float
    vd: float
    q: np.ndarray  # code value x descale, float64 (exact)
    k: np.ndarray
    v: np.ndarray
    scale: float
    causal: bool = False
    window: int = 0
    kv_len: np.ndarray | None = None


def attn_fp8_inputs(B: int, H: int, N: int, d: int, *, seed: int = 0, causal: bool = False, window: int = 0,
                    kv_len=None, n_big_keys: int = 0) -> Fp8AttnInputs:
    """The float32 attention recipe (same draws as ``attn_inputs``), quantized per tensor to e4m3."""
    src = attn_inputs(B, H, N, d, dtype="f32", seed=seed, causal=causal, window=window, kv_len=kv_len,
                      n_big_keys=n_big_keys)
    out = {}
    for name in ("q", "k", "v"):
        x = getattr(src, name)
        dsc = e4m3_descale(x)
        codes, vals = e4m3_round(x.astype(np.float64) / dsc)
        out[name + "8"], out[name + "d"], out[name] = codes, dsc, vals * dsc
    return Fp8AttnInputs(scale=src.scale, causal=causal, window=window, kv_len=src.kv_len, **out)


def grad_inputs(B: int, H: int, N: int, d: int, *, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """dO [B, H, N, d] from N(0, 1) per (b, h) slice, rounded to bfloat16: (bits, float32 values)."""
    do = np.empty((B, H, N, d), np.float32)
    for b in range(B):
        for h in range(H):
            do[b, h] = np.random.default_rng([seed, 2000, b, h]).standard_normal((N, d), dtype=np.float32)
    return bf16_round(do)


def decode_inputs(B: int, H: int, Nkv: int, d: int, *, seed: int = 0, dtype: str = "bf16"):
    """One query per (b, h) plus K, V of length Nkv; same per-slice recipe."""
    q = np.empty((B, H, d), np.float32)
    k = np.empty((B, H, Nkv, d), np.float32)
    v = np.empty((B, H, Nkv, d), np.float32)
    for b in range(B):
        for h in range(H):
            rng = np.random.default_rng([seed, b, h])
            q[b, h] = rng.standard_normal(d, dtype=np.float32)
            k[b, h] = rng.standard_normal((Nkv, d), dtype=np.float32)
            v[b, h] = rng.standard_normal((Nkv, d), dtype=np.float32)
    res = {"q": q, "k": k, "v": v, "dtype": dtype}
    if dtype == "bf16":
        for name in ("q", "k", "v"):
            bits, vals = bf16_round(res[name])
            res[name] = vals
            res[name + "_bits"] = bits
    return res


def decode_slice(seed: int, b: int, h: int, Nkv: int, d: int, dtype: str = "bf16"):
    """The (b, h) slice of :func:`decode_inputs`, drawn on its own (bounded memory)."""
    rng = np.random.default_rng([seed, b, h])
    q = rng.standard_normal(d, dtype=np.float32)
    k = rng.standard_normal((Nkv, d), dtype=np.float32)
    v = rng.standard_normal((Nkv, d), dtype=np.float32)
    if dtype == "bf16":
        qb, q = bf16_round(q)
        kb, k = bf16_round(k)
        vb, v = bf16_round(v)
        return q, k, v, qb, kb, vb
    return q, k, v, None, None, None


def attn_bits_large(B: int, H: int, N: int, d: int, regions, *, seed: int = 0, count: int = 3) -> list[np.ndarray]:
    """``count`` bfloat16 tensors [B, H, N, d] (Q, K, V, then dO) as bit patterns, for the largest shapes.

    Zero except the row ranges ``regions`` = [(b, h, r0, r1), ...], whose
    elements are a random sign, a binade drawn uniformly from [1/8, 1/4),
    [1/4, 1/2), [1/2, 1), [1, 2) and a uniform 7-bit mantissa (integer
    operations on one uniform 16-bit draw), so that tensors of 10^9 elements
    cost only their allocation; range i is drawn from rng([seed, 3000, t, i]).
    """
    out = []
    for t in range(count):
        bits = np.zeros((B, H, N, d), np.uint16)
        for i, (b, h, r0, r1) in enumerate(regions):
            rng = np.random.default_rng([seed, 3000, t, i])
            r = rng.integers(0, 1 << 16, size=(r1 - r0, d), dtype=np.uint16)
            e = ((r >> 7) & np.uint16(3)) + np.uint16(124)  # biased exponents 124..127
            bits[b, h, r0:r1] = (r & np.uint16(0x807F)) | (e << np.uint16(7))
        out.append(bits)
    return out


def softmax_rows_inputs(rows: int, cols: int, *, seed: int = 0, sigma: float = 4.0) -> np.ndarray:
    """x[rows, cols] float32, i.i.d. N(0, sigma^2), drawn in blocks of 256 rows."""
    x = np.empty((rows, cols), np.float32)
    for r0 in range(0, rows, 256):
        r1 = min(rows, r0 + 256)
        rng = np.random.default_rng([seed, r0 // 256])
        x[r0:r1] = rng.standard_normal((r1 - r0, cols), dtype=np.float32) * np.float32(sigma)
    return x


# ---------------------------------------------------------------------------
# The five workloads (shapes, masks, seeds)
# ---------------------------------------------------------------------------

WORKLOADS = {
    # FP32 attention, N not a multiple of any tile, no mask.
    "attn_f32_b1h1_n1000_d64": dict(kind="attn", B=1, H=1, N=1000, d=64, dtype="f32",
                                     causal=False, window=0, kv_len=None, n_big_keys=0, seed=1),
    # Row softmax and the fused top-5 variant, N(0, 4^2).
    "softmax_rows_4096x4000": dict(kind="softmax", rows=4096, cols=4000, sigma=4.0, seed=2),
    "softmax_top5_1024x25000": dict(kind="topk", rows=1024, cols=25000, k=5, sigma=4.0, seed=20),
    # bf16 causal attention.
    "attn_bf16_causal_b4h32_n2048_d128": dict(kind="attn", B=4, H=32, N=2048, d=128, dtype="bf16",
                                               causal=True, window=0, kv_len=None, n_big_keys=0, seed=3),
    # bf16 causal + sliding window 1024 + last 512 keys padded; 1% of keys x8.
    "attn_bf16_causal_w1024_pad512_b1h64_n8192_d128": dict(
        kind="attn", B=1, H=64, N=8192, d=128, dtype="bf16", causal=True, window=1024,
        kv_len=[8192 - 512], n_big_keys=82, seed=4),
    # Split-KV decode: one query per head, 131072 keys, 64 splits.
    "decode_bf16_b1h32_nkv131072_d128_split64": dict(kind="decode", B=1, H=32, Nkv=131072, d=128,
                                                      nsplit=64, dtype="bf16", seed=5),
}


def workload_attn_inputs(name: str, **override) -> AttnInputs:
    w = dict(WORKLOADS[name])
    w.update(override)
    return attn_inputs(w["B"], w["H"], w["N"], w["d"], dtype=w["dtype"], seed=w["seed"],
                       causal=w["causal"], window=w["window"], kv_len=w["kv_len"],
                       n_big_keys=w["n_big_keys"])
