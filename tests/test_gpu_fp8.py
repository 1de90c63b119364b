"""GPU parity: attn_fwd_fp8 (e4m3 Q, K, V, d = 128) against the FP64 oracle.

The oracle is the exact attention of the dequantized inputs (code x
descale), ``oracle.attention_ref``.  The FP8 path differs from it by the
e4m3 rounding of P and the matrix core's accumulation, which
``oracle.attention_fp8_error_bound`` bounds from the e4m3 and bf16 formats
alone (pinned on the CPU against simulated FP8 pipelines and planted
mistakes); no term of it comes from this kernel's design or from a
measurement.  Per (b, h) slice:

  * every element: |O - O_ref| <= 1.5 x the worst-case bound bO;
  * RMS over the slice: rms(O - O_ref) <= 2 rms(sO) + 1.5 rms(bO with the P
    rounding term removed) -- the P roundings behave as independent errors,
    so a systematic mistake (a lost block, a wrong mask) shows here long
    before it breaks the worst case;
  * LSE: |LSE - LSE_ref| <= 1.5 x bL (score accumulation error);
  * a query with no visible key: O = 0 and LSE = -inf exactly.
The factor 1.5 covers the second-order terms the first-order model drops.
The ratio to ``oracle.attention_fp8_error_model`` (the tighter bound of the
kernel's own per-block frame) is printed as a diagnostic, not asserted.
"""
import numpy as np
import pytest
import torch

import online_softmax_fa2_amd as osfa
from online_softmax_fa2_amd.inputs import WORKLOADS, attn_fp8_inputs, bf16_round
from oracle import attention_fp8_error_bound, attention_fp8_error_model, attention_ref
from tests.gpu_util import Guarded

pytestmark = pytest.mark.gpu


def run_fp8(inp):
    dev = torch.device("cuda:0")
    q8, k8, v8 = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (inp.q8, inp.k8, inp.v8))
    B, H, N, d = inp.q.shape
    o = Guarded((B, H, N, d), torch.bfloat16)
    lse = Guarded((B, H, N), torch.float32)
    kvl = None if inp.kv_len is None else torch.from_numpy(inp.kv_len).to(dev)
    osfa.attn_fwd_fp8(q8, k8, v8, inp.qd, inp.kd, inp.vd, scale=inp.scale, causal=inp.causal, window=inp.window,
                      kv_len=kvl, out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    o.check()
    lse.check()
    return o.t.float().cpu().numpy(), lse.t.cpu().numpy()


def check(inp, O, L, heads=None):
    B, H, N, d = inp.q.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = (inp.q[sl], inp.k[sl], inp.v[sl], inp.scale)
        kw = dict(causal=inp.causal, window=inp.window, kv_len=None if inp.kv_len is None else inp.kv_len[b:b + 1])
        Or, Lr = attention_ref(*args, **kw)
        bO, sO, bL = attention_fp8_error_bound(*args, **kw)
        bdet, _, _ = attention_fp8_error_bound(*args, **kw, u_p=0.0)
        dO = attention_fp8_error_model(*args, **kw)[0][0, 0]
        og, lg = O[b, h], L[b, h]
        Or, Lr, bO, sO, bL, bdet = Or[0, 0], Lr[0, 0], bO[0, 0], sO[0, 0], bL[0, 0], bdet[0, 0]
        what = f"b={b} h={h}"
        assert not np.isnan(og).any() and not np.isnan(lg).any(), f"{what}: NaN"
        err = np.abs(og - Or)
        bad = err > 1.5 * bO
        assert not bad.any(), (f"{what}: {int(bad.sum())} O elements over 1.5 x bound; worst ratio "
                               f"{(err / np.maximum(bO, 1e-300)).max():.3g}")
        print(f"{what}: worst err / gate {(err / np.maximum(bO, 1e-300)).max():.3f}, "
              f"worst err / block-frame model {(err / np.maximum(dO, 1e-300)).max():.3f}")
        rms, lim = np.sqrt(np.mean(err ** 2)), 2 * np.sqrt(np.mean(sO ** 2)) + 1.5 * np.sqrt(np.mean(bdet ** 2))
        assert rms <= lim, f"{what}: O rms error {rms:.3e} > {lim:.3e}"
        inf = np.isinf(Lr)
        assert np.array_equal(np.isinf(lg), inf) and np.all(lg[inf] == Lr[inf]), f"{what}: -inf rows differ"
        assert np.all(og[inf] == 0), f"{what}: O of a row with no key"
        le = np.abs(lg[~inf] - Lr[~inf])
        assert le.size == 0 or np.all(le <= 1.5 * bL[~inf]), f"{what}: LSE error {le.max():.3e} over bound"


CASES = [
    # (B, H, N, causal, window, kv_len, n_big)
    (1, 1, 1, False, 0, None, 0),
    (1, 2, 65, False, 0, None, 0),
    (2, 1, 129, True, 0, None, 0),
    (1, 2, 1000, True, 0, None, 0),
    (1, 1, 1000, False, 0, None, 0),
    (2, 2, 300, True, 7, None, 0),
    (1, 2, 700, True, 100, [650], 3),
    (2, 1, 500, False, 60, [430, 500], 0),
    (2, 1, 333, True, 0, [0, 200], 0),        # batch 0: every row fully masked
    (1, 1, 256, True, 64, [100], 0),          # window + padding: rows 163.. see nothing
    (1, 3, 513, False, 0, [257], 4),
    (1, 1, 200, False, 2**31 - 1, None, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_fp8_parity(case):
    B, H, N, causal, window, kv_len, nbig = case
    print(f"attn_fwd_fp8 B={B} H={H} N={N} d=128 causal={causal} window={window} kv_len={kv_len}", flush=True)
    inp = attn_fp8_inputs(B, H, N, 128, seed=N + B + 11, causal=causal, window=window, kv_len=kv_len, n_big_keys=nbig)
    O, L = run_fp8(inp)
    check(inp, O, L)


def test_fp8_self_only_closed_form():
    """Causal window 1: P = 1 for the query's own key, so O = bf16(v_i) exactly and LSE = s_ii."""
    inp = attn_fp8_inputs(1, 2, 300, 128, seed=95, causal=True, window=1)
    O, L = run_fp8(inp)
    assert np.array_equal(O, bf16_round(inp.v.astype(np.float32))[1])
    s = np.float32(inp.scale) * np.einsum("bhnd,bhnd->bhn", inp.q, inp.k)
    assert np.abs(L - s).max() <= 1e-3 * max(1.0, np.abs(s).max())


def test_fp8_full_window_pad_8192():
    w = WORKLOADS["attn_bf16_causal_w1024_pad512_b1h64_n8192_d128"]
    print("attn_fwd_fp8 full workload (window + padding, 8192)", flush=True)
    inp = attn_fp8_inputs(w["B"], w["H"], w["N"], w["d"], seed=w["seed"], causal=w["causal"], window=w["window"],
                          kv_len=w["kv_len"], n_big_keys=w["n_big_keys"])
    O, L = run_fp8(inp)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    check(inp, O, L, heads=[(0, 0), (0, 63)])
