"""CPU pins for the attention and decode oracle, and for the pages' claims.

The direct oracle (``oracle.attention_ref``) is pinned by closed forms,
invariants, a pure-Python brute force that subtracts no maximum, and exact
mask counts.  The pages' streaming algorithms (``oracle.models``) are then
checked against it on the pages' own test cases, and each mistake the pages
list is planted in the model to show that some pin fails for it.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_ref, decode_ref, visible_count, visible_mask
from oracle.models import (MUTATIONS, blockwise_attention, blockwise_attention_full,
                           single_query_blockwise, split_kv_merge, split_kv_partials)
from online_softmax_fa2_amd.inputs import attn_inputs, decode_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FACTS = json.load(open(os.path.join(GOLDEN, "page_facts.json")))


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# --- brute force ---------------------------------------------------------------------

def _brute_attention(q, k, v, sigma, causal, window, kv_len):
    """Pure-Python loops, no maximum subtracted, exactly rounded sums (math.fsum)."""
    N, d = q.shape
    O = np.zeros((N, d))
    L = np.zeros(N)
    for i in range(N):
        ws, js = [], []
        for j in range(N):
            ok = j < kv_len and (not causal or j <= i) and (window <= 0 or abs(i - j) < window)
            if ok:
                s = sigma * math.fsum(float(q[i, t]) * float(k[j, t]) for t in range(d))
                ws.append(math.exp(s))
                js.append(j)
        if not ws:
            L[i] = -math.inf
            continue
        z = math.fsum(ws)
        for t in range(d):
            O[i, t] = math.fsum(w * float(v[j, t]) for w, j in zip(ws, js)) / z
        L[i] = math.log(z)
    return O, L


@pytest.mark.parametrize("case", [
    dict(N=7, d=4, causal=False, window=0, kv_len=7),
    dict(N=9, d=3, causal=True, window=0, kv_len=9),
    dict(N=10, d=5, causal=True, window=3, kv_len=10),
    dict(N=10, d=2, causal=False, window=4, kv_len=10),
    dict(N=12, d=4, causal=True, window=5, kv_len=8),   # padding + window: empty rows
    dict(N=6, d=3, causal=False, window=0, kv_len=0),   # every row empty
    dict(N=11, d=6, causal=True, window=2, kv_len=4),
])
def test_direct_equals_brute_force(case):
    N, d = case["N"], case["d"]
    rng = np.random.default_rng(N * 100 + d)
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    sigma = float(np.float32(0.7))
    O, L = attention_ref(q[None, None], k[None, None], v[None, None], 0.7, causal=case["causal"],
                         window=case["window"], kv_len=[case["kv_len"]])
    Ob, Lb = _brute_attention(q, k, v, sigma, case["causal"], case["window"], case["kv_len"])
    assert np.max(np.abs(O[0, 0] - Ob)) < 1e-13
    fin = np.isfinite(Lb)
    assert np.array_equal(fin, np.isfinite(L[0, 0]))
    assert np.max(np.abs(L[0, 0][fin] - Lb[fin]), initial=0.0) < 1e-13
    assert np.all(O[0, 0][~fin] == 0.0)


# --- closed forms -------------------------------------------------------------------

def test_single_key_gives_value_and_score():
    q, k, v = _rand((1, 1, 1, 8), 1), _rand((1, 1, 1, 8), 2), _rand((1, 1, 1, 8), 3)
    O, L = attention_ref(q, k, v, 0.25)
    assert np.max(np.abs(O[0, 0, 0] - v[0, 0, 0])) < 1e-15
    assert L[0, 0, 0] == pytest.approx(float(np.float32(0.25)) * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-14)


@pytest.mark.parametrize("causal,window,klen", [(False, 0, 40), (True, 0, 40), (True, 7, 33), (False, 5, 40)])
def test_constant_values_give_constant_output(causal, window, klen):
    q, k = _rand((1, 1, 40, 16), 4), _rand((1, 1, 40, 16), 5)
    v = np.ones((1, 1, 40, 16))
    O, L = attention_ref(q, k, v, 0.25, causal=causal, window=window, kv_len=[klen])
    nonempty = np.isfinite(L[0, 0])
    assert np.max(np.abs(O[0, 0][nonempty] - 1.0)) < 1e-14


@pytest.mark.parametrize("causal,window,klen", [(True, 0, 30), (True, 6, 30), (False, 4, 25), (True, 3, 12)])
def test_identical_keys_give_mean_of_visible_values(causal, window, klen):
    """Equal scores: O is the mean of the visible values, LSE = s + ln |visible|."""
    N, d = 30, 8
    q = _rand((1, 1, N, d), 6)
    k = np.broadcast_to(_rand((1, 1, 1, d), 7), (1, 1, N, d)).copy()
    v = _rand((1, 1, N, d), 8)
    O, L = attention_ref(q, k, v, 0.5, causal=causal, window=window, kv_len=[klen])
    for i in range(N):
        js = [j for j in range(min(N, klen)) if (not causal or j <= i) and (window <= 0 or abs(i - j) < window)]
        if not js:
            assert L[0, 0, i] == -np.inf and np.all(O[0, 0, i] == 0)
            continue
        assert np.max(np.abs(O[0, 0, i] - v[0, 0, js].mean(axis=0))) < 1e-14
        s = float(np.float32(0.5)) * float(q[0, 0, i] @ k[0, 0, 0])
        assert L[0, 0, i] == pytest.approx(s + math.log(len(js)), abs=1e-13)


def test_causal_window_one_is_identity():
    q, k, v = _rand((2, 3, 17, 8), 9), _rand((2, 3, 17, 8), 10), _rand((2, 3, 17, 8), 11)
    O, L = attention_ref(q, k, v, 0.3, causal=True, window=1)
    assert np.max(np.abs(O - v)) < 1e-15
    s = float(np.float32(0.3)) * np.einsum("bhnd,bhnd->bhn", q, k)
    assert np.max(np.abs(L - s)) < 1e-14


def test_huge_score_gap_is_exact_one_hot():
    """Scores 1e4 apart: exact one-hot, no NaN (page 'Derive online softmax, prove it is exact')."""
    N, d = 50, 4
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 1.0
    k = _rand((1, 1, N, d), 12); k[..., 0] = 0.0
    k[0, 0, 31, 0] = 1.0e4
    v = _rand((1, 1, N, d), 13)
    qq = np.zeros((1, 1, N, d)); qq[0, 0, 0] = q[0, 0, 0]
    O, L = attention_ref(qq, k, v, 1.0, rows=[0])
    assert np.all(O[0, 0, 0] == v[0, 0, 31])
    assert L[0, 0, 0] == 1.0e4


# --- invariants ---------------------------------------------------------------------

def test_key_translation_shifts_lse_only():
    q, k, v = _rand((1, 2, 20, 8), 14), _rand((1, 2, 20, 8), 15), _rand((1, 2, 20, 8), 16)
    u = _rand((8,), 17)
    O1, L1 = attention_ref(q, k, v, 0.4, causal=True)
    O2, L2 = attention_ref(q, k + u, v, 0.4, causal=True)
    sig = float(np.float32(0.4))
    assert np.max(np.abs(O1 - O2)) < 1e-13
    assert np.max(np.abs(L2 - (L1 + sig * (q @ u)))) < 1e-12


def test_key_permutation_invariance():
    q, k, v = _rand((1, 1, 25, 8), 18), _rand((1, 1, 25, 8), 19), _rand((1, 1, 25, 8), 20)
    perm = np.random.default_rng(21).permutation(25)
    O1, L1 = attention_ref(q, k, v, 0.4)
    O2, L2 = attention_ref(q, k[:, :, perm], v[:, :, perm], 0.4)
    assert np.max(np.abs(O1 - O2)) < 1e-14 and np.max(np.abs(L1 - L2)) < 1e-14


def test_lse_bracket():
    q, k, v = _rand((1, 1, 64, 16), 22), _rand((1, 1, 64, 16), 23), _rand((1, 1, 64, 16), 24)
    O, L = attention_ref(q, k, v, 0.25, causal=True, window=9, kv_len=[60])
    s = float(np.float32(0.25)) * (q[0, 0] @ k[0, 0].T)
    vis = visible_mask(np.arange(64), np.arange(64), 64, 60, True, 9)
    for i in range(64):
        if not vis[i].any():
            assert L[0, 0, i] == -np.inf
            continue
        mx = s[i][vis[i]].max()
        assert mx - 1e-12 <= L[0, 0, i] <= mx + math.log(vis[i].sum()) + 1e-12


def test_output_is_convex_combination():
    q, k, v = _rand((1, 1, 50, 8), 25), _rand((1, 1, 50, 8), 26), _rand((1, 1, 50, 8), 27)
    O, _ = attention_ref(q, k, v, 0.25, causal=True, window=6)
    for i in range(50):
        lo, hi = max(0, i - 5), i + 1
        assert np.all(O[0, 0, i] <= v[0, 0, lo:hi].max(axis=0) + 1e-14)
        assert np.all(O[0, 0, i] >= v[0, 0, lo:hi].min(axis=0) - 1e-14)


# --- mask counts (closed forms) -------------------------------------------------------

def test_visible_counts_closed_forms():
    N = 300
    assert visible_count(N, N, False, 0) == N * N
    assert visible_count(N, N, True, 0) == N * (N + 1) // 2
    W = 40  # causal window: row i sees min(i + 1, W) keys
    assert visible_count(N, N, True, W) == sum(min(i + 1, W) for i in range(N))
    # non-causal symmetric window: row i sees keys in [i-W+1, i+W-1] within [0, N)
    assert visible_count(N, N, False, W) == sum(min(N - 1, i + W - 1) - max(0, i - W + 1) + 1 for i in range(N))
    # right padding with causal: rows >= L see exactly L keys
    L = 200
    assert visible_count(N, L, True, 0) == L * (L + 1) // 2 + (N - L) * L
    assert visible_count(N, 0, True, 5) == 0


def test_fully_masked_rows_are_zero_and_neg_inf_without_nan():
    """Window 4 + padding at 20: rows >= 23 see nothing (page 'Online softmax for a whole query tile')."""
    inp = attn_inputs(1, 2, 40, 16, dtype="f32", seed=28, causal=True, window=4, kv_len=[20])
    O, L = attention_ref(inp.q, inp.k, inp.v, inp.scale, causal=True, window=4, kv_len=inp.kv_len)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    assert np.all(O[:, :, 23:] == 0.0) and np.all(L[:, :, 23:] == -np.inf)
    assert np.all(np.isfinite(L[:, :, :23]))


# --- the pages' claims: the recurrence equals the direct softmax ------------------------

def test_single_query_blockwise_exact():
    """1,000 keys in blocks of 128 (page 'Derive online softmax, prove it is exact')."""
    c = FACTS["exactness_claims"]
    n, d = c["single_query_keys"], 64
    q, K, V = _rand(d, 30), _rand((n, d), 31), _rand((n, d), 32)
    o = single_query_blockwise(q, K, V, block=c["single_query_block"])
    Q = np.zeros((1, 1, n, d)); Q[0, 0, 0] = q
    O, _ = attention_ref(Q, K[None, None], V[None, None], 1.0 / math.sqrt(d), rows=[0])
    # the oracle rounds the scale to float32; compare at the same scale
    o32 = single_query_blockwise(q, K, V, block=c["single_query_block"], scale=float(np.float32(1 / math.sqrt(d))))
    assert np.max(np.abs(o32 - O[0, 0, 0])) < c["single_query_max_err"]
    assert np.max(np.abs(o - o32)) < 1e-6  # only the scale's float32 rounding differs
    # magnitudes of 1e4: exact, where unshifted exp overflows
    Kb = K * 1e4 / np.abs(K @ q).max() * math.sqrt(d)
    ob = single_query_blockwise(q, Kb, V, block=128, scale=float(np.float32(1 / math.sqrt(d))))
    Ob, _ = attention_ref(Q, Kb[None, None], V[None, None], 1.0 / math.sqrt(d), rows=[0])
    assert np.max(np.abs(ob - Ob[0, 0, 0])) == 0.0
    with np.errstate(over="ignore", invalid="ignore"):
        s = float(np.float32(1 / math.sqrt(d))) * (Kb @ q)
        e = np.exp(s)
        assert np.isnan((e @ V) / e.sum()).any()


def _tile_cases():
    c = FACTS["exactness_claims"]
    N, Br, d = c["tile_N"], c["tile_Br"], c["tile_d"]
    yield "noncausal", N, Br, d, False, 0, None
    for off in c["tile_causal_offsets"]:
        yield f"causal@{off}", N, Br, d, True, off, None
    yield "late_max", N, Br, d, False, 0, c["tile_late_max_keys"]


@pytest.mark.parametrize("name,N,Br,d,causal,q0,late", list(_tile_cases()))
def test_tile_recurrence_exact(name, N, Br, d, causal, q0, late):
    """N = 1,000, Br = 128, d = 64 (page 'Online softmax for a whole query tile, matrix form')."""
    rng = np.random.default_rng(40)
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    if late:
        K[-late:] *= 6.0  # the largest scores arrive in the last keys
    scale = float(np.float32(1 / math.sqrt(d)))
    rows = np.arange(q0, min(N, q0 + Br))
    o, lse = blockwise_attention(Q[rows], K, V, scale, q0=q0, N=N, Bc=64, causal=causal)
    O, L = attention_ref(Q[None, None], K[None, None], V[None, None], scale, causal=causal, rows=rows)
    assert np.max(np.abs(o - O[0, 0])) < FACTS["exactness_claims"]["tile_max_err"]
    assert np.max(np.abs(lse - L[0, 0])) < 1e-12


@pytest.mark.parametrize("causal,window,klen", [(True, 64, 900), (True, 300, 1000), (False, 100, 700), (True, 1, 1000)])
def test_tile_recurrence_exact_with_window_and_padding(causal, window, klen):
    rng = np.random.default_rng(41)
    N, d = 1000, 32
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    O1, L1 = blockwise_attention_full(Q, K, V, float(np.float32(0.2)), Br=128, Bc=64, causal=causal, window=window, kv_len=klen)
    O2, L2 = attention_ref(Q[None, None], K[None, None], V[None, None], 0.2, causal=causal,
                           window=window, kv_len=[klen])
    assert not np.isnan(O1).any()
    assert np.max(np.abs(O1 - O2[0, 0])) < 1e-13
    fin = np.isfinite(L2[0, 0])
    assert np.array_equal(fin, np.isfinite(L1))
    assert np.max(np.abs(L1[fin] - L2[0, 0][fin])) < 1e-12


# --- planted mistakes: each must be caught by some pin --------------------------------

def _pin_suite(mutation):
    """Run the pins that the pages say catch each listed mistake; return the failures."""
    failures = []
    rng = np.random.default_rng(50)
    N, d = 1000, 32
    scale = float(np.float32(1 / math.sqrt(d)))

    def check(name, Q, K, V, **kw):
        O1, L1 = blockwise_attention_full(Q, K, V, scale, Br=128, Bc=64, mutation=mutation, **kw)
        O2, L2 = attention_ref(Q[None, None], K[None, None], V[None, None], scale,
                               kv_len=[kw.get("kv_len") or Q.shape[0]],
                               causal=kw.get("causal", False), window=kw.get("window", 0))
        with np.errstate(invalid="ignore"):
            bad = (np.isnan(O1).any() or np.isnan(L1).any() or np.max(np.abs(O1 - O2[0, 0])) > 1e-12)
        if bad:
            failures.append(name)

    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Kl = K.copy(); Kl[-5:] *= 6.0
    check("late_max", Q, Kl, V)
    check("causal_partial_block", Q, K, V, causal=True)
    # all-negative rows: scores near -1000
    Qn = np.abs(Q) + 1.0; Kn = -np.abs(K) * 0 - 1.0
    check("all_negative", Qn * 30, Kn * 30 + rng.standard_normal((N, d)), V)
    # rows far apart in one tile: +1000 and -1000
    Qf = Q.copy(); Qf[::2] *= 0.0; Qf[::2, 0] = 1e4 / scale / 3; Qf[1::2, 0] = -1e4 / scale / 3
    Kf = K.copy(); Kf[:, 0] = np.abs(Kf[:, 0]) * 0.1 + 0.3
    check("rows_far_apart", Qf, Kf, V)
    check("window_padding", Q, K, V, causal=True, window=100, kv_len=700)
    return failures


def test_correct_model_passes_every_pin():
    assert _pin_suite(None) == []


@pytest.mark.parametrize("mutation", [m for m in MUTATIONS if m is not None])
def test_each_planted_mistake_is_caught(mutation):
    assert _pin_suite(mutation), f"no pin caught {mutation}"


# --- decode ---------------------------------------------------------------------------

@pytest.mark.parametrize("nsplit", [1, 2, 7, 64, 300])
def test_split_kv_merge_equals_direct(nsplit):
    inp = decode_inputs(1, 2, 300, 32, seed=60)
    o = decode_ref(inp["q"], inp["k"], inp["v"])
    for h in range(2):
        parts = split_kv_partials(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h], nsplit)
        om, _ = split_kv_merge(parts)
        assert np.max(np.abs(om - o[0, h])) < 1e-14


def test_decode_brute_force():
    inp = decode_inputs(1, 1, 40, 6, seed=61, dtype="f32")
    o = decode_ref(inp["q"], inp["k"], inp["v"])
    q, k, v = inp["q"][0, 0], inp["k"][0, 0], inp["v"][0, 0]
    sigma = float(np.float32(1 / math.sqrt(6)))
    ws = [math.exp(sigma * math.fsum(float(q[t]) * float(k[j, t]) for t in range(6))) for j in range(40)]
    z = math.fsum(ws)
    want = [math.fsum(w * float(v[j, t]) for j, w in enumerate(ws)) / z for t in range(6)]
    assert np.max(np.abs(o[0, 0] - np.array(want))) < 1e-14


def test_decode_equal_keys_is_mean():
    q = _rand((1, 1, 16), 62)
    k = np.broadcast_to(_rand((1, 1, 1, 16), 63), (1, 1, 333, 16)).copy()
    v = _rand((1, 1, 333, 16), 64)
    o = decode_ref(q, k, v)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(axis=0))) < 1e-14


def test_empty_split_contributes_nothing():
    q, k, v = _rand(8, 65), _rand((5, 8), 66), _rand((5, 8), 67)
    parts = split_kv_partials(q, k, v, 8)  # L = 1: chunks 5..7 empty
    assert parts[6][0] == -np.inf and parts[6][1] == 0.0
    o1, _ = split_kv_merge(parts)
    o2, _ = split_kv_merge(split_kv_partials(q, k, v, 1))
    assert np.max(np.abs(o1 - o2)) < 1e-15
