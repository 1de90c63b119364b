"""Pins of the FP64 backward oracle (oracle.backward) against things it does
not compute itself: central finite differences of the forward definition
(oracle.attention_ref) on tiny inputs, closed forms and exact invariants.

The gradient formulas are the softmax Jacobian written out; the pages fix
what the backward pass computes (the gradients of the forward output,
recomputed from the per-row log-sum-exp: page "Derive online softmax, prove
it is exact", section "What interviewers probe next").
"""
import numpy as np
import pytest

import oracle.backward as ob
from oracle import attention_bwd_delta, attention_bwd_ref, attention_ref

MASKS = [
    dict(causal=False, window=0, kv_len=None),
    dict(causal=True, window=0, kv_len=None),
    dict(causal=True, window=2, kv_len=None),
    dict(causal=False, window=2, kv_len=None),
    dict(causal=False, window=0, kv_len=[3]),
    dict(causal=True, window=2, kv_len=[2]),  # rows 4.. see no key
    dict(causal=False, window=0, kv_len=[0]),  # nothing visible
]


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _loss(Q, K, V, dO, scale, m):
    O, _ = attention_ref(Q, K, V, scale, **m)
    return float((O * dO).sum())


def _fd(Q, K, V, dO, scale, m, h=1e-5):
    grads = []
    for which in range(3):
        X = [Q.copy(), K.copy(), V.copy()]
        g = np.zeros_like(X[which])
        for idx in np.ndindex(*X[which].shape):
            Xp = [x.copy() for x in X]
            Xm = [x.copy() for x in X]
            Xp[which][idx] += h
            Xm[which][idx] -= h
            g[idx] = (_loss(*Xp, dO, scale, m) - _loss(*Xm, dO, scale, m)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("m", MASKS, ids=[str(i) for i in range(len(MASKS))])
def test_gradients_match_finite_differences(m):
    N, d = 6, 4
    Q, K, V, dO = (_rand((1, 1, N, d), s) for s in (1, 2, 3, 4))
    scale = 0.7
    dQ, dK, dV = attention_bwd_ref(Q, K, V, dO, scale, **m)
    fQ, fK, fV = _fd(Q, K, V, dO, scale, m)
    for a, f in ((dQ, fQ), (dK, fK), (dV, fV)):
        assert np.max(np.abs(a - f)) < 1e-7 * max(1.0, np.max(np.abs(f)))


def test_planted_mistake_is_caught():
    """Dropping the row term of the softmax Jacobian (dS = P * dP) fails the finite-difference pin."""
    N, d = 5, 3
    Q, K, V, dO = (_rand((1, 1, N, d), s) for s in (5, 6, 7, 8))
    good = attention_bwd_ref(Q, K, V, dO, 0.9)[0]
    sigma = float(np.float32(0.9))
    p = ob._probs(Q[0, 0], K[0, 0], sigma, np.ones((N, N), bool))
    dp = dO[0, 0] @ V[0, 0].T
    wrong = sigma * ((p * dp) @ K[0, 0])
    fQ = _fd(Q, K, V, dO, 0.9, dict(causal=False, window=0, kv_len=None))[0]
    assert np.max(np.abs(good[0, 0] - fQ[0, 0])) < 1e-7
    assert np.max(np.abs(wrong - fQ[0, 0])) > 1e-3


def test_invariants_and_closed_forms():
    rng = np.random.default_rng(11)
    B, H, N, d = 2, 2, 37, 8
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    m = dict(causal=True, window=9, kv_len=[30, 37])
    dQ, dK, dV = attention_bwd_ref(Q, K, V, dO, 0.35, **m)
    # every row sees at least its own key or keys before the padding here
    # sum over keys of dS is zero in every row: dK sums to zero over keys
    assert np.max(np.abs(dK.sum(axis=2))) < 1e-12
    # rows of P sum to one: dV sums to the sum of dO over rows that see a key
    _, L = attention_ref(Q, K, V, 0.35, **m)
    seen = np.isfinite(L)[..., None]
    assert np.max(np.abs(dV.sum(axis=2) - (dO * seen).sum(axis=2))) < 1e-11
    # translating every key by u leaves dQ (and dV) unchanged
    u = rng.standard_normal(d)
    dQ2, dK2, dV2 = attention_bwd_ref(Q, K + u, V, dO, 0.35, **m)
    assert np.max(np.abs(dQ2 - dQ)) < 1e-11 and np.max(np.abs(dV2 - dV)) < 1e-11
    # equal value rows: O does not depend on Q or K
    Vc = np.broadcast_to(rng.standard_normal(d), V.shape)
    dQ3, dK3, _ = attention_bwd_ref(Q, K, Vc, dO, 0.35, **m)
    assert np.max(np.abs(dQ3)) < 1e-12 and np.max(np.abs(dK3)) < 1e-12


def test_single_key_and_masked_rows():
    Q, K, V, dO = (_rand((1, 1, 1, 4), s) for s in (21, 22, 23, 24))
    dQ, dK, dV = attention_bwd_ref(Q, K, V, dO, 0.5)
    assert np.allclose(dV, dO, atol=0, rtol=0) and not dQ.any() and not dK.any()
    # a row with no visible key contributes nothing; kv_len = 0 gives all zeros
    Q, K, V, dO = (_rand((1, 1, 9, 4), s) for s in (31, 32, 33, 34))
    z = attention_bwd_ref(Q, K, V, dO, 0.5, causal=True, kv_len=[0])
    assert all(not g.any() for g in z)


def test_delta_is_row_sum_of_p_times_dp():
    rng = np.random.default_rng(3)
    N, d = 23, 6
    Q, K, V, dO = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    O, _ = attention_ref(Q, K, V, 0.4, causal=True)
    D = attention_bwd_delta(O, dO)[0, 0]
    sigma = float(np.float32(0.4))
    idx = np.arange(N)
    p = ob._probs(Q[0, 0], K[0, 0], sigma, idx[None, :] <= idx[:, None])
    dp = dO[0, 0] @ V[0, 0].T
    assert np.max(np.abs(D - (p * dp).sum(axis=1))) < 1e-12
