"""Direct row softmax and its top-k in float64.  TEST INFRASTRUCTURE.

Row softmax follows article "Online softmax", section "Step 1" (safe
softmax): subtract the row maximum, exponentiate, divide by the sum.  The
online normalizer (Steps 2-3 of the same article) returns exactly these
values; the oracle is the definition.

Top-k follows the same article, section "Step 3" (softmax fused with a
top-k selection): the k largest probabilities of the row and their column
indices.  Reading where the article is silent: ties in x are broken by the
lower column index, so the order is (x descending, index ascending), and the
values returned are the k probabilities (not the full row).  Softmax is
strictly increasing in x, so ranking by x is ranking by probability.
"""
from __future__ import annotations

import numpy as np


def softmax_ref(x) -> np.ndarray:
    """y[r, :] = exp(x[r, :] - max_r) / sum(exp(x[r, :] - max_r)), float64."""
    x = np.asarray(x).astype(np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def topk_order(x, k: int) -> np.ndarray:
    """Column indices [rows, k] ordered by (x descending, index ascending)."""
    x = np.asarray(x)
    rows, cols = x.shape
    idx = np.empty((rows, k), np.int64)
    col = np.arange(cols)
    for r in range(rows):
        xr = x[r].astype(np.float64)
        # Sort keys: primary -x (descending x), secondary column index.
        order = sorted(range(cols), key=lambda c: (-xr[c], c)) if cols <= 64 else \
            np.lexsort((col, -xr))
        idx[r] = np.asarray(order[:k])
    return idx


def topk_ref(x, k: int) -> tuple[np.ndarray, np.ndarray]:
    """(values [rows, k] float64, indices [rows, k] int64) of the row softmax."""
    y = softmax_ref(x)
    idx = topk_order(x, k)
    vals = np.take_along_axis(y, idx, axis=1)
    return vals, idx
