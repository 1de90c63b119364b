"""Pins of the FP8 input conversion and of the FP8 attention error model (CPU).

* ``inputs.e4m3_round`` against a brute-force nearest search over the 254
  finite e4m3fn codes decoded from the format's definition (1 sign, 4
  exponent bits with bias 7, 3 mantissa bits, subnormals, 0x7F/0xFF NaN),
  ties to the even code.
* ``oracle.attention_fp8_error_model``: a simulated FP8 pipeline (P rounded
  to e4m3 in a per-(query, 64-key block) power-of-two frame whose block
  maximum lands in (128, 256], O divided by the sum of the rounded P) stays
  inside the worst-case bound everywhere and inside the statistical bound in
  RMS; planted mistakes (a dropped key block, a mask off by one, O not
  multiplied by the V descale, one frame per row instead of per block on a
  row dominated by one key) escape one of them.
"""
import numpy as np
import pytest

from online_softmax_fa2_amd.inputs import attn_fp8_inputs, e4m3_descale, e4m3_round
from oracle import attention_fp8_error_model, attention_ref, visible_mask


def _e4m3_table():
    vals = np.empty(256)
    for c in range(256):
        sgn = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sgn * m * 2.0 ** -9
        else:
            vals[c] = sgn * (1 + m / 8) * 2.0 ** (e - 7)
    return vals


TAB = _e4m3_table()


def _nearest_even(y):
    fin = np.nonzero(np.isfinite(TAB))[0]
    d = np.abs(TAB[fin] - y)
    best = fin[d == d.min()]
    even = [c for c in best if (c & 1) == 0]
    c = (even or list(best))[0]
    return TAB[c]


def test_e4m3_round_matches_brute_force():
    rng = np.random.default_rng(0)
    y = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-12, 9, 3000)),
        np.array([448.0, -448.0, 0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 1.0625, 1.1875, 15.5, 240.0, 232.0]),
        (np.arange(1, 40) + 0.5) * 2.0 ** -9,  # subnormal ties
    ])
    y = np.clip(y, -448, 448)
    codes, vals = e4m3_round(y)
    for yi, ci, vi in zip(y, codes, vals):
        want = _nearest_even(yi)
        assert vi == want or (vi == 0 and want == 0), (yi, vi, want)
        assert TAB[ci] == vi or (TAB[ci] == 0 and vi == 0)
    with pytest.raises(ValueError):
        e4m3_round(np.array([449.0]))


def test_e4m3_descale_fits_range():
    rng = np.random.default_rng(1)
    for scale in (1e-3, 1.0, 37.0, 1e4):
        x = rng.standard_normal(5000).astype(np.float32) * scale
        d = e4m3_descale(x)
        assert np.float32(d) == d and np.abs(x.astype(np.float64) / d).max() <= 448.0
        assert np.abs(x.astype(np.float64) / d).max() > 447.0


# ---------------------------------------------------------------------------
# The error model against a simulated FP8 pipeline
# ---------------------------------------------------------------------------

def _sim_fp8(inp, mistake=None):
    """O of the dequantized inputs with P rounded to e4m3 as the FP8 path does (float64 elsewhere)."""
    B, H, N, d = inp.q.shape
    sigma = float(np.float32(inp.scale))
    out = np.zeros((B, H, N, d))
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            klen = N if inp.kv_len is None else int(inp.kv_len[b])
            vis = visible_mask(idx, idx, N, klen, inp.causal, inp.window)
            if mistake == "mask_off_by_one":  # causal j < i, or the last key dropped
                vis = vis & (idx[None, :] < idx[:, None]) if inp.causal else visible_mask(idx, idx, N, klen - 1,
                                                                                           False, inp.window)
            q, k, v = inp.q[b, h], inp.k[b, h], inp.v[b, h]
            if mistake == "no_v_descale":
                v = v / inp.vd
            s = np.where(vis, sigma * (q @ k.T), -np.inf)
            m = s.max(axis=1)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            pq = np.zeros_like(e)
            blocks = [(0, N)] if mistake == "row_frame" else [(j0, min(N, j0 + 64)) for j0 in range(0, N, 64)]
            for j0, j1 in blocks:
                bm = e[:, j0:j1].max(axis=1)
                u = np.where(bm > 0, 8 - np.ceil(np.log2(np.where(bm > 0, bm, 1.0))), 0.0)
                frame = np.exp2(u)[:, None]
                pq[:, j0:j1] = e4m3_round(np.minimum(e[:, j0:j1] * frame, 448.0))[1] / frame
            if mistake == "drop_block":
                pq[:, 64:128] = 0.0
            lq = pq.sum(axis=1)
            out[b, h] = (pq @ v) / np.where(lq > 0, lq, 1.0)[:, None]
    return out


def _check(inp, o, bO, sO, bdet, Oref):
    """(worst-case holds everywhere, RMS within 2 x statistical + deterministic) per (b, h) slice."""
    err = np.abs(o - Oref)
    worst_ok = bool(np.all(err <= 1.01 * bO + 1e-300))
    B, H = inp.q.shape[:2]
    rms_ok = True
    for b in range(B):
        for h in range(H):
            lim = 2 * np.sqrt(np.mean(sO[b, h] ** 2)) + np.sqrt(np.mean(bdet[b, h] ** 2))
            rms_ok &= bool(np.sqrt(np.mean(err[b, h] ** 2)) <= lim)
    return worst_ok, rms_ok


CASES = [
    dict(B=1, H=2, N=300, causal=False, window=0, kv_len=None, n_big_keys=0),
    dict(B=1, H=1, N=400, causal=True, window=0, kv_len=None, n_big_keys=4),
    dict(B=2, H=1, N=333, causal=True, window=70, kv_len=[333, 120], n_big_keys=3),
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_fp8_model_covers_simulated_pipeline(case):
    c = dict(case)
    inp = attn_fp8_inputs(c.pop("B"), c.pop("H"), c.pop("N"), 128, seed=50, **c)
    Oref, _ = attention_ref(inp.q, inp.k, inp.v, inp.scale, causal=inp.causal, window=inp.window, kv_len=inp.kv_len)
    bO, sO, _ = attention_fp8_error_model(inp.q, inp.k, inp.v, inp.scale, causal=inp.causal, window=inp.window,
                                          kv_len=inp.kv_len)
    bdet, _, _ = attention_fp8_error_model(inp.q, inp.k, inp.v, inp.scale, causal=inp.causal, window=inp.window,
                                           kv_len=inp.kv_len, u_p=0.0)
    assert _check(inp, _sim_fp8(inp), bO, sO, bdet, Oref) == (True, True)
    for mistake in ("drop_block", "mask_off_by_one", "no_v_descale"):
        assert _check(inp, _sim_fp8(inp, mistake), bO, sO, bdet, Oref) != (True, True), mistake


def test_fp8_model_catches_a_row_wide_frame():
    """A frame per row flushes many small P far below one dominant key (here 1.1 % of the mass); the
    per-block frame keeps them, and the bound (block maxima) tells the two apart."""
    inp = attn_fp8_inputs(1, 1, 2048, 128, seed=51)
    sigma = float(np.float32(inp.scale))
    inp.q[:] = 0.0
    inp.k[:] = 0.0
    inp.q[0, 0, 0, 0] = 17.5 * np.log(2.0) / sigma  # key 0 beats every other key by 2^17.5
    inp.k[0, 0, 0, 0] = 1.0
    inp.v[:] = 1.0
    inp.v[0, 0, 0] = 0.0
    Oref, _ = attention_ref(inp.q, inp.k, inp.v, inp.scale)
    bO, sO, _ = attention_fp8_error_model(inp.q, inp.k, inp.v, inp.scale)
    bdet, _, _ = attention_fp8_error_model(inp.q, inp.k, inp.v, inp.scale, u_p=0.0)
    assert Oref[0, 0, 0, 0] > 0.01
    assert _check(inp, _sim_fp8(inp), bO, sO, bdet, Oref)[0]
    assert not _check(inp, _sim_fp8(inp, "row_frame"), bO, sO, bdet, Oref)[0]


def test_fp8_model_zero_for_rows_without_keys():
    inp = attn_fp8_inputs(2, 1, 100, 128, seed=52, causal=True, kv_len=[0, 100])
    bO, sO, bL = attention_fp8_error_model(inp.q, inp.k, inp.v, inp.scale, causal=True, kv_len=inp.kv_len)
    assert np.all(bO[0] == 0) and np.all(sO[0] == 0) and np.all(bL[0] == 0)
    assert np.all(bL[1] > 0)
