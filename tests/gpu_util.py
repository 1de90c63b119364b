"""Helpers for the GPU parity tests: uploads, guard-band canaries, tolerances.

Tolerances (the bar the tests apply):
  * float32 paths: relative error <= 1e-5.  O is compared normwise per
    (b, h) slice, max|O - O_ref| / max|O_ref|, because elementwise relative
    error is unbounded where O_ref passes through zero; LSE, softmax values
    and top-k values elementwise, |g - r| <= 1e-5 |r| (values below the
    float32 normal range, 1.18e-38, are compared absolutely at that size).
    LSE is measured relative to max(|LSE|, 1): its rounding error is
    absolute in the units of the scores, so near LSE = 0 a purely relative
    measure is undefined.
  * bfloat16-input attention (float32 statistics, bf16 O): |O - O_ref| <=
    1e-2 + half a bf16 ulp of O_ref elementwise (the output format's own
    rounding is charged to the format), LSE |g - r| <= 1e-3.
  * integer outputs (top-k indices): bit-exact.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

PAD = 4096  # canary elements on each side of every output
CANARY_F32 = -123456.0


def dev():
    return torch.device("cuda:0")


def upload_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def upload_f32(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


class Guarded:
    """An output tensor with patterned guard bands on both sides."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape))
        self.buf = torch.empty(n + 2 * PAD, dtype=dtype, device=dev())
        if dtype.is_floating_point:
            self.buf.fill_(CANARY_F32 if dtype == torch.float32 else -777.0)
        else:
            self.buf.fill_(-1234567)
        self.ref = self.buf.clone()
        self.t = self.buf[PAD:PAD + n].view(shape)

    def check(self):
        lo_ok = torch.equal(self.buf[:PAD], self.ref[:PAD])
        hi_ok = torch.equal(self.buf[-PAD:], self.ref[-PAD:])
        assert lo_ok and hi_ok, "write outside the output tensor (guard band changed)"


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 0.0)


def assert_f32_rel(got, ref, tol=1e-5, what="", floor=0.0):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    same_inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), same_inf) and np.all(got[same_inf] == ref[same_inf]), f"{what}: inf mismatch"
    g, r = got[~same_inf], ref[~same_inf]
    err = np.abs(g - r)
    bound = np.maximum(tol * np.maximum(np.abs(r), floor), 1.18e-38 * 2)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements over rel {tol}; worst rel "
                           f"{np.max(err / np.maximum(np.abs(r), 1e-300)):.3e}")


def assert_normwise(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if den == 0:
        assert num == 0, f"{what}: expected zeros, max |err| {num}"
    else:
        assert num / den <= tol, f"{what}: normwise rel error {num / den:.3e} > {tol}"


def assert_bf16_out(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    err = np.abs(got - ref)
    bound = 1e-2 + bf16_half_ulp(ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements over 1e-2 + half ulp; max abs err {err.max():.4e}"
    return float(err.max()) if err.size else 0.0


def assert_lse_abs(got, ref, tol=1e-3, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in LSE"
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.all(got[inf] == ref[inf]), f"{what}: -inf rows differ"
    err = np.abs(got[~inf] - ref[~inf])
    assert err.size == 0 or err.max() <= tol, f"{what}: LSE max abs err {err.max():.3e} > {tol}"


def oracle_map(fn, items, workers: int = 8):
    """[fn(x) for x in items], run on a thread pool (NumPy releases the GIL in its array kernels)."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))
