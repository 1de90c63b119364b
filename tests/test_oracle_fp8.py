"""Pins of the FP8 input conversion and of the FP8 attention error model (CPU).

* ``inputs.e4m3_round`` against a brute-force nearest search over the 254
  finite e4m3fn codes decoded from the format's definition (1 sign, 4
  exponent bits with bias 7, 3 mantissa bits, subnormals, 0x7F/0xFF NaN),
  ties to the even code.
* ``oracle.attention_fp8_error_bound`` (the gate, format-derived terms):
  simulated FP8 pipelines for every legal way of rounding P (no frame, a
  frame per row, a frame per 64-key block) and with scores carrying a bf16
  rounding stay inside the worst-case bound everywhere and inside the
  statistical bound in RMS; planted mistakes (a dropped key block, a mask
  off by one, O not multiplied by the V descale) escape it; dropping its
  a_p or kappa term lets a legal pipeline escape.
* ``oracle.attention_fp8_error_model`` (diagnostic, the block frame's own
  tighter bound): covers the block-frame pipeline, is never looser than
  the gate, and rejects a row-wide frame on a row dominated by one key.
"""
import numpy as np
import pytest

from online_softmax_fa2_amd.inputs import attn_fp8_inputs, e4m3_descale, e4m3_round
from oracle import attention_fp8_error_bound, attention_fp8_error_model, attention_ref, visible_mask


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
# The gate and the diagnostic model against simulated FP8 pipelines
# ---------------------------------------------------------------------------

def _bf16(x):
    """Round float64 to the nearest bf16 value (ties to even), via float32."""
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _sim_fp8(inp, design="block_frame", mistake=None):
    """O of the dequantized inputs with P rounded to e4m3 (float64 elsewhere).

    design: "block_frame" -- each 64-key block scaled so that its largest P
    lands in (128, 256] (the frame attn_fwd_fp8 uses); "plain" -- P =
    exp(s - max) in (0, 1] rounded as it is; "row_frame" -- one frame per
    row; "bf16_scores" -- block frame with every score rounded to bf16
    precision (an accumulation error of one bf16 rounding of the sum).
    """
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
            s = sigma * (q @ k.T)
            if design == "bf16_scores":
                s = _bf16(s)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            pq = np.zeros_like(e)
            if design == "plain":
                pq = e4m3_round(e)[1]
            else:
                blocks = [(0, N)] if design == "row_frame" else [(j0, min(N, j0 + 64)) for j0 in range(0, N, 64)]
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


def _bounds(fn, inp, **kw):
    a = (inp.q, inp.k, inp.v, inp.scale)
    m = dict(causal=inp.causal, window=inp.window, kv_len=inp.kv_len)
    bO, sO, bL = fn(*a, **m, **kw)
    bdet, _, _ = fn(*a, **m, **dict(kw, u_p=0.0))
    return bO, sO, bdet, bL


@pytest.mark.parametrize("case", CASES, ids=str)
def test_fp8_gate_covers_every_design_and_rejects_mistakes(case):
    """The gate (format-derived terms) holds for each legal way of rounding P and for bf16-accurate score
    accumulation; a dropped key block, a mask off by one and a missing V descale escape it."""
    c = dict(case)
    inp = attn_fp8_inputs(c.pop("B"), c.pop("H"), c.pop("N"), 128, seed=50, **c)
    Oref, _ = attention_ref(inp.q, inp.k, inp.v, inp.scale, causal=inp.causal, window=inp.window, kv_len=inp.kv_len)
    bO, sO, bdet, _ = _bounds(attention_fp8_error_bound, inp)
    for design in ("block_frame", "plain", "row_frame", "bf16_scores"):
        assert _check(inp, _sim_fp8(inp, design), bO, sO, bdet, Oref) == (True, True), design
    for mistake in ("drop_block", "mask_off_by_one", "no_v_descale"):
        assert _check(inp, _sim_fp8(inp, mistake=mistake), bO, sO, bdet, Oref) != (True, True), mistake


@pytest.mark.parametrize("case", CASES, ids=str)
def test_fp8_diagnostic_model_covers_the_block_frame(case):
    """The tighter model of the kernel's own frame covers that frame and rejects the same mistakes."""
    c = dict(case)
    inp = attn_fp8_inputs(c.pop("B"), c.pop("H"), c.pop("N"), 128, seed=50, **c)
    Oref, _ = attention_ref(inp.q, inp.k, inp.v, inp.scale, causal=inp.causal, window=inp.window, kv_len=inp.kv_len)
    bO, sO, bdet, _ = _bounds(attention_fp8_error_model, inp)
    assert _check(inp, _sim_fp8(inp), bO, sO, bdet, Oref) == (True, True)
    for mistake in ("drop_block", "mask_off_by_one", "no_v_descale"):
        assert _check(inp, _sim_fp8(inp, mistake=mistake), bO, sO, bdet, Oref) != (True, True), mistake
    gO = attention_fp8_error_bound(inp.q, inp.k, inp.v, inp.scale, causal=inp.causal, window=inp.window,
                                   kv_len=inp.kv_len)[0]
    assert np.all(bO <= gO + 1e-300)  # the diagnostic is never looser than the gate


def _dominant_key_case():
    """Key 0 beats every other key by 2^17.5; the other 2047 keys carry 1.1 % of the mass."""
    inp = attn_fp8_inputs(1, 1, 2048, 128, seed=51)
    sigma = float(np.float32(inp.scale))
    inp.q[:] = 0.0
    inp.k[:] = 0.0
    inp.q[0, 0, 0, 0] = 17.5 * np.log(2.0) / sigma
    inp.k[0, 0, 0, 0] = 1.0
    inp.v[:] = 1.0
    inp.v[0, 0, 0] = 0.0
    return inp


def test_fp8_frames_on_a_row_dominated_by_one_key():
    """A row-wide frame (or no frame) flushes the small P: legal under the gate, whose a_p term is what
    covers it (drop that term and the plain design escapes); the diagnostic model of the block frame tells
    the two designs apart."""
    inp = _dominant_key_case()
    Oref, _ = attention_ref(inp.q, inp.k, inp.v, inp.scale)
    assert Oref[0, 0, 0, 0] > 0.01
    gate = _bounds(attention_fp8_error_bound, inp)[:3]
    for design in ("block_frame", "plain", "row_frame"):
        assert _check(inp, _sim_fp8(inp, design), *gate, Oref)[0], design
    no_ap = _bounds(attention_fp8_error_bound, inp, a_p=0.0)[:3]
    assert not _check(inp, _sim_fp8(inp, "plain"), *no_ap, Oref)[0]
    diag = _bounds(attention_fp8_error_model, inp)[:3]
    assert _check(inp, _sim_fp8(inp), *diag, Oref)[0]
    assert not _check(inp, _sim_fp8(inp, "row_frame"), *diag, Oref)[0]


def test_fp8_gate_kappa_covers_bf16_accumulation():
    """Scores carrying one bf16 rounding stay inside the gate; with kappa at float32 level they escape."""
    inp = attn_fp8_inputs(1, 1, 512, 128, seed=53, causal=True)
    Oref, _ = attention_ref(inp.q, inp.k, inp.v, inp.scale, causal=True)
    o = _sim_fp8(inp, "bf16_scores")
    gate = _bounds(attention_fp8_error_bound, inp)[:3]
    assert _check(inp, o, *gate, Oref)[0]
    tight = _bounds(attention_fp8_error_bound, inp, kappa=2.0 ** -24, u_p=0.0, a_p=0.0)[:3]
    assert not _check(inp, o, *tight, Oref)[0]


def test_fp8_model_zero_for_rows_without_keys():
    inp = attn_fp8_inputs(2, 1, 100, 128, seed=52, causal=True, kv_len=[0, 100])
    for fn in (attention_fp8_error_bound, attention_fp8_error_model):
        bO, sO, bL = fn(inp.q, inp.k, inp.v, inp.scale, causal=True, kv_len=inp.kv_len)
        assert np.all(bO[0] == 0) and np.all(sO[0] == 0) and np.all(bL[0] == 0)
        assert np.all(bL[1] > 0)
