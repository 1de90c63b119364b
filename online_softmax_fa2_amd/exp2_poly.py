"""Coefficients of the cubic that gives 2^f on [-1/2, 1/2] for the FMA-pipe exponential.

``exp2_fma`` (csrc/device_common.h) computes 2^x as 2^n * p(x - n) with n the
nearest integer to x.  p is the cubic with the smallest maximum relative error
|p(f) / 2^f - 1| over [-1/2, 1/2], found as a linear program on a dense grid
of f (minimize t subject to -t 2^f <= p(f) - 2^f <= t 2^f).  Usage:
``python -m online_softmax_fa2_amd.exp2_poly`` prints the float32 constants.
"""
from __future__ import annotations

import numpy as np


def minimax_exp2_coeffs(degree: int = 3, points: int = 4001) -> tuple[np.ndarray, float]:
    """(c_0 .. c_degree, max relative error on the grid) of the minimax polynomial for 2^f, |f| <= 1/2."""
    from scipy.optimize import linprog

    f = np.linspace(-0.5, 0.5, points)
    y = np.exp2(f)
    vander = np.vander(f, degree + 1, increasing=True)
    a_ub = np.vstack([np.hstack([vander, -y[:, None]]), np.hstack([-vander, -y[:, None]])])
    b_ub = np.concatenate([y, -y])
    cost = np.zeros(degree + 2)
    cost[-1] = 1.0
    res = linprog(cost, A_ub=a_ub, b_ub=b_ub, bounds=[(None, None)] * (degree + 1) + [(0, None)], method="highs")
    if not res.success:
        raise RuntimeError(res.message)
    return res.x[:-1], float(res.x[-1])


if __name__ == "__main__":
    c, err = minimax_exp2_coeffs()
    for i, v in enumerate(c.astype(np.float32)):
        print(f"constexpr float kExp2C{i} = {float(v)!r}f;")
    print(f"// max relative error on the grid: {err:.3e}")
