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


# ---------------------------------------------------------------------------
# The rounding-error bound used as the GPU tolerance: it must cover a
# simulated bf16 pipeline (O, P, dS and the outputs rounded to bf16 with
# round-to-nearest-even, everything else exact), every one of its terms must
# be needed, and it must not be vacuous.
# ---------------------------------------------------------------------------

def _bf(x):
    from online_softmax_fa2_amd.inputs import bf16_round
    return bf16_round(np.asarray(x, np.float32))[1].astype(np.float64)


def _sim_bf16_bwd(Q, K, V, dO, scale, m, mistake=None):
    """The bf16 pipeline, optionally with one planted mistake (to show the bound would catch it)."""
    B, H, N, d = Q.shape
    sigma = float(np.float32(scale))
    out = [np.zeros((B, H, N, d)) for _ in range(3)]
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            klen = N if m["kv_len"] is None else m["kv_len"][b]
            q, k, v, g = Q[b, h], K[b, h], V[b, h], dO[b, h]
            vis = ob.visible_mask(idx, idx, N, klen, m["causal"], m["window"])
            if mistake == "mask_off_by_one":
                vis = ob.visible_mask(idx, idx, N, klen - 1, m["causal"], m["window"] + (m["window"] > 0))
            p = ob._probs(q, k, sigma, vis)
            o = _bf(p @ v)
            dp = g @ v.T
            dd = (g * o).sum(axis=1, keepdims=True)
            if mistake == "no_delta":
                dd = 0.0 * dd
            ds = _bf(p * (dp - dd))
            if mistake == "ds_transposed_block":
                ds[:32, :32] = ds[:32, :32].T.copy()
            out[0][b, h] = _bf(sigma * (ds @ k))
            out[1][b, h] = _bf((1.0 if mistake == "dk_unscaled" else sigma) * (ds.T @ q))
            out[2][b, h] = _bf(_bf(p).T @ g)
    return out


def _bf_inputs(N, d, seed, big=()):
    Q, K, V, dO = (_bf(_rand((1, 1, N, d), seed + i)) for i in range(4))
    K[:, :, list(big), :] *= 8.0
    return Q, K, V, dO


@pytest.mark.parametrize("big", [(), (3, 77, 120)], ids=["plain", "big_keys"])
@pytest.mark.parametrize("m", MASKS[:-1] + [dict(causal=True, window=40, kv_len=[100])], ids=str)
def test_bound_covers_simulated_bf16(m, big):
    """The bound holds for every element, and four plausible mistakes each break it."""
    Q, K, V, dO = _bf_inputs(160, 16, 40, big=big)
    sc = 0.25
    ref = attention_bwd_ref(Q, K, V, dO, sc, **m)
    bnd = ob.attention_bwd_error_bound(Q, K, V, dO, sc, **m)
    sim = _sim_bf16_bwd(Q, K, V, dO, sc, m)
    for name, s, r, bd in zip("QKV", sim, ref, bnd):
        assert np.all(np.abs(s - r) <= 1.01 * bd + 1e-300), f"d{name}: simulated error exceeds the bound"
    # Not vacuous: each planted mistake escapes it.
    for mistake in ("no_delta", "mask_off_by_one", "ds_transposed_block", "dk_unscaled"):
        bad = _sim_bf16_bwd(Q, K, V, dO, sc, m, mistake)
        assert any(np.any(np.abs(s - r) > 1.01 * bd) for s, r, bd in zip(bad, ref, bnd)), mistake


def test_bound_terms_are_needed():
    """Drop the D term or the operand term (planted mistakes in the bound) and the simulated error escapes it.

    (The output-rounding term is kept for rigour; with the worst-case sums of
    the other two it is never the one that decides.)
    """
    m = dict(causal=False, window=0, kv_len=None)
    Q, K, V, dO = _bf_inputs(160, 16, 41, big=(5, 90))
    sc = 0.25
    ref = attention_bwd_ref(Q, K, V, dO, sc, **m)
    sim = _sim_bf16_bwd(Q, K, V, dO, sc, m)

    def escapes(**u):
        bnd = ob.attention_bwd_error_bound(Q, K, V, dO, sc, **m, **u)
        return [bool(np.any(np.abs(s - r) > 1.01 * bd)) for s, r, bd in zip(sim, ref, bnd)]

    assert escapes() == [False, False, False]
    assert escapes(u_o=0.0)[0]                # D's rounding reaches dQ
    assert escapes(u_operand=0.0)[2]          # P's rounding reaches dV


def test_bound_zero_where_gradient_vanishes():
    m = dict(causal=True, window=2, kv_len=[2])
    Q, K, V, dO = _bf_inputs(8, 4, 42)
    bQ, bK, bV = ob.attention_bwd_error_bound(Q, K, V, dO, 0.5, **m)
    assert np.all(bQ[0, 0, 3:] == 0)          # queries 3.. see no key
    assert np.all(bK[0, 0, 2:] == 0) and np.all(bV[0, 0, 2:] == 0)  # keys 2.. are padding
