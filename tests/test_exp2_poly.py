"""CPU checks of the FMA-pipe exponential (exp2_fma in csrc/device_common.h).

* Its cubic's coefficients are the ones the stated method gives: the float32
  rounding of the minimax (relative error) cubic for 2^f on [-1/2, 1/2],
  re-derived here by ``exp2_poly.minimax_exp2_coeffs``.
* The whole function, emulated step by step in float32 (clamp at -200,
  nearest integer n, f = x - n, Horner with fused multiply-adds, 2^n by
  ldexp), stays within 7.6e-5 relative of 2^x over the range the attention
  kernels feed it ([-126, 32]: P <= 2^32 under the lazy rescale) and gives
  exactly 0 for -inf (masked scores).
"""
import os
import re

import numpy as np

from online_softmax_fa2_amd.exp2_poly import minimax_exp2_coeffs

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "online_softmax_fa2_amd", "csrc",
                   "device_common.h")


def _kernel_coeffs():
    text = open(SRC).read()
    vals = dict(re.findall(r"constexpr float kExp2C(\d) = ([0-9.eE+-]+)f;", text))
    return np.array([float(vals[str(i)]) for i in range(4)], np.float32)


def _fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _exp2_fma(x):
    c = _kernel_coeffs()
    x = np.maximum(np.asarray(x, np.float32), np.float32(-200.0))
    n = np.rint(x).astype(np.float32)
    f = (x - n).astype(np.float32)
    p = _fma32(_fma32(_fma32(np.full_like(f, c[3]), f, np.full_like(f, c[2])), f, np.full_like(f, c[1])), f,
               np.full_like(f, c[0]))
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def test_coefficients_are_the_minimax_cubic():
    c, err = minimax_exp2_coeffs(3)
    assert np.array_equal(c.astype(np.float32), _kernel_coeffs())
    assert err < 7.5e-5


def test_exp2_fma_accuracy_and_masked_scores():
    rng = np.random.default_rng(5)
    x = np.concatenate([np.linspace(-126, 32, 400001), rng.uniform(-126, 32, 200000), np.arange(-126, 33) + 0.5,
                        np.arange(-126, 33) - 0.5, [0.0, -1e-30, 1e-30]]).astype(np.float32)
    got = _exp2_fma(x).astype(np.float64)
    want = np.exp2(x.astype(np.float64))
    assert np.max(np.abs(got / want - 1.0)) < 7.6e-5
    z = _exp2_fma(np.array([-np.inf, -200.0, -1e30, -250.5], np.float32))
    assert np.all(z == 0.0)
