"""GPU parity: attn_bwd (bf16, d = 128) against the FP64 oracle's gradients.

The forward runs first on the GPU (attn_fwd gives O and LSE, as a training
step would), then attn_bwd; dQ, dK, dV are compared with
``oracle.attention_bwd_ref`` computed from the same bf16 Q, K, V, dO.

Tolerance, per element: |g - r| <= 1.5 x the first-order rounding bound of
``oracle.attention_bwd_error_bound`` with bfloat16's unit roundoff 2^-8
for the three roundings this path makes: P (for dV) and dS (for dQ, dK)
become bf16 matrix-core operands, D = rowsum(dO * O) is formed from the
forward's bf16 O, and each gradient is rounded to bf16.  The bound is pinned
on the CPU against a simulated bf16 pipeline, including planted mistakes it
must reject.  The factor 1.5 covers what the bound leaves out: float32
accumulation over at most 8192 terms (n 2^-24 < 2^-8 / 7 of the same sums)
and the float32 error of P = exp2(S log2(e) - LSE log2(e)), ~1e-6 relative.
Where the bound is 0 (a query that sees no key, a key that no query sees)
the gradient must be exactly 0.

attn_bwd has two ways to dQ, chosen by the workspace size: storing dS in
the workspace and multiplying it with K, or recomputing S and dP; the
parity cases run both.
"""
import numpy as np
import pytest
import torch

import online_softmax_fa2_amd as osfa
from online_softmax_fa2_amd.inputs import (WORKLOADS, attn_bits_large, attn_inputs, bf16_bits_to_f32, grad_inputs,
                                          workload_attn_inputs)
from oracle import attention_bwd_error_bound, attention_bwd_ref, visible_mask
from tests.gpu_util import Guarded, upload_bf16

pytestmark = pytest.mark.gpu

MARGIN = 1.5


def assert_grad(got, ref, bound, what):
    got = np.asarray(got, np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN"
    err = np.abs(got - ref)
    bad = err > MARGIN * bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements over {MARGIN} x bound; worst at {i}: got {got[i]:.6g} "
                             f"ref {ref[i]:.6g} bound {bound[i]:.3e}; normwise {err.max() / max(np.abs(ref).max(), 1e-300):.3e}")


def ws_bytes(B, H, N, causal, window, stored):
    """Workspace for the stored-dS way (which must apply) or the minimum (dQ recomputes S and dP)."""
    need = osfa.bwd_workspace_bytes(B, H, N)
    if stored:
        st = osfa.bwd_stored_ds_workspace_bytes(B, H, N, causal, window)
        assert st > need
        need = st
    return need


def run_fwd_bwd(inp, do_bits, stored=True):
    q, k, v = upload_bf16(inp.q_bits), upload_bf16(inp.k_bits), upload_bf16(inp.v_bits)
    dout = upload_bf16(do_bits)
    B, H, N, d = inp.q.shape
    kvl = None if inp.kv_len is None else torch.from_numpy(inp.kv_len).to("cuda:0")
    o, lse = osfa.attn_fwd(q, k, v, scale=inp.scale, causal=inp.causal, window=inp.window, kv_len=kvl)
    grads = [Guarded((B, H, N, d), torch.bfloat16) for _ in range(3)]
    ws = Guarded(((ws_bytes(B, H, N, inp.causal, inp.window, stored) + 3) // 4,), torch.float32)
    osfa.attn_bwd(q, k, v, o, dout, lse, scale=inp.scale, causal=inp.causal, window=inp.window, kv_len=kvl,
                  dq=grads[0].t, dk=grads[1].t, dv=grads[2].t, workspace=ws.t)
    torch.cuda.synchronize()
    for g in grads:
        g.check()
    ws.check()
    return [g.t.float().cpu().numpy() for g in grads]


def check(inp, do, got, heads=None):
    B, H, N, d = inp.q.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        kvl = None if inp.kv_len is None else inp.kv_len[b:b + 1]
        args = (inp.q[sl], inp.k[sl], inp.v[sl], do[sl], inp.scale)
        kw = dict(causal=inp.causal, window=inp.window, kv_len=kvl)
        ref = attention_bwd_ref(*args, **kw)
        bnd = attention_bwd_error_bound(*args, **kw)
        vis = visible_mask(np.arange(N), np.arange(N), N, N if kvl is None else int(kvl[0]), inp.causal,
                           inp.window)
        for name, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bnd):
            assert_grad(g[b, h], r[0, 0], bd[0, 0], f"b={b} h={h} {name}")
        assert np.all(got[0][b, h][~vis.any(axis=1)] == 0), f"b={b} h={h}: dQ of a query that sees no key"
        unseen = ~vis.any(axis=0)
        assert np.all(got[1][b, h][unseen] == 0) and np.all(got[2][b, h][unseen] == 0), \
            f"b={b} h={h}: dK/dV of a key that no query sees"


CASES = [
    # (B, H, N, causal, window, kv_len, n_big)
    (1, 1, 1, False, 0, None, 0),
    (1, 2, 1, True, 0, None, 0),
    (1, 2, 65, False, 0, None, 0),
    (2, 1, 129, True, 0, None, 0),
    (1, 2, 1000, True, 0, None, 0),
    (1, 1, 1000, False, 0, None, 0),
    (2, 2, 300, True, 7, None, 0),
    (1, 2, 700, True, 100, [650], 3),
    (2, 1, 500, False, 60, [430, 500], 0),
    (2, 1, 333, True, 0, [0, 200], 0),         # batch 0: every row fully masked
    (1, 1, 256, True, 64, [100], 0),           # window + padding: rows 163.. see nothing
    (1, 3, 513, False, 0, [257], 4),
    (3, 2, 127, False, 1000, None, 0),
    (1, 1, 384, True, 128, None, 0),           # window = one query tile
    (1, 1, 200, False, 2**31 - 1, None, 0),    # window beyond N: no mask
    (2, 1, 150, True, 2**31 - 1, [150, 77], 0),
]


@pytest.mark.parametrize("stored", [True, False], ids=["stored_ds", "recompute"])
@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_bwd_parity(case, stored):
    B, H, N, causal, window, kv_len, nbig = case
    print(f"attn_bwd bf16 B={B} H={H} N={N} d=128 causal={causal} window={window} kv_len={kv_len} stored={stored}",
          flush=True)
    inp = attn_inputs(B, H, N, 128, dtype="bf16", seed=N + B + 7, causal=causal, window=window, kv_len=kv_len,
                      n_big_keys=nbig)
    do_bits, do = grad_inputs(B, H, N, 128, seed=N + 3)
    got = run_fwd_bwd(inp, do_bits, stored)
    check(inp, do, got)


def _sweep_cases(n=10, seed=20261203):
    """Seeded random backward configurations (d = 128): 1 to ~700 queries (log-uniform), causal or not, a
    window on half of them, per-batch padding (possibly 0) on some, planted large keys on some."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        N = int(np.clip(np.exp(rng.uniform(0, np.log(700))), 1, 700))
        causal = bool(rng.integers(0, 2))
        window = int(rng.integers(1, N + 40)) if rng.uniform() < 0.5 else 0
        kv_len = [int(x) for x in rng.integers(0, N + 1, size=B)] if rng.uniform() < 0.4 else None
        out.append((B, H, N, causal, window, kv_len, int(rng.integers(0, min(N, 4) + 1))))
    return out


@pytest.mark.parametrize("stored", [True, False], ids=["stored_ds", "recompute"])
@pytest.mark.parametrize("case", _sweep_cases(), ids=[f"s{i}" for i in range(10)])
def test_bwd_random_sweep(case, stored):
    """Every head of every drawn configuration against the oracle's gradients, within the bound."""
    B, H, N, causal, window, kv_len, nbig = case
    print(f"attn_bwd sweep B={B} H={H} N={N} causal={causal} window={window} kv_len={kv_len} big={nbig} "
          f"stored={stored}", flush=True)
    inp = attn_inputs(B, H, N, 128, dtype="bf16", seed=N * 5 + B, causal=causal, window=window, kv_len=kv_len,
                      n_big_keys=nbig)
    do_bits, do = grad_inputs(B, H, N, 128, seed=N + 11)
    got = run_fwd_bwd(inp, do_bits, stored)
    check(inp, do, got)


@pytest.mark.parametrize("case", [CASES[7], CASES[8], CASES[12]], ids=["window_pad", "noncausal_window", "wide"])
def test_bwd_paths_agree(case):
    """dK and dV come from the same kernel either way (identical); dQ from the stored dS or from recomputed S and
    dP, which form dS the same way."""
    B, H, N, causal, window, kv_len, nbig = case
    inp = attn_inputs(B, H, N, 128, dtype="bf16", seed=N + 11, causal=causal, window=window, kv_len=kv_len,
                      n_big_keys=nbig)
    do_bits, do = grad_inputs(B, H, N, 128, seed=N + 5)
    a = run_fwd_bwd(inp, do_bits, True)
    r = run_fwd_bwd(inp, do_bits, False)
    assert np.array_equal(a[1], r[1]) and np.array_equal(a[2], r[2])
    print(f"dQ identical across the two ways: {np.array_equal(a[0], r[0])}; max diff {np.abs(a[0] - r[0]).max():.3e}",
          flush=True)
    check(inp, do, a)


def test_bwd_default_workspace_choice(monkeypatch):
    """Without a workspace the binding picks the way by size: the stored-dS way by default, the recomputing
    way with stored_ds=False or when the stored workspace exceeds its cap; the three give the same gradients
    (bit for bit: both ways form dS alike and accumulate in the same order)."""
    from online_softmax_fa2_amd import _binding
    inp = attn_inputs(1, 2, 300, 128, dtype="bf16", seed=91, causal=True, window=70)
    do_bits, do = grad_inputs(1, 2, 300, 128, seed=92)
    q, k, v = upload_bf16(inp.q_bits), upload_bf16(inp.k_bits), upload_bf16(inp.v_bits)
    dout = upload_bf16(do_bits)
    o, lse = osfa.attn_fwd(q, k, v, scale=inp.scale, causal=True, window=70)
    print("attn_bwd default workspace: B=1 H=2 N=300 causal window=70", flush=True)
    outs = [osfa.attn_bwd(q, k, v, o, dout, lse, scale=inp.scale, causal=True, window=70)]
    outs.append(osfa.attn_bwd(q, k, v, o, dout, lse, scale=inp.scale, causal=True, window=70, stored_ds=False))
    monkeypatch.setattr(_binding, "STORED_DS_MAX_BYTES", 0)
    outs.append(osfa.attn_bwd(q, k, v, o, dout, lse, scale=inp.scale, causal=True, window=70))
    torch.cuda.synchronize()
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)
    check(inp, do, [g.float().cpu().numpy() for g in outs[0]])


def test_bwd_self_only():
    """Causal window 1: P = 1 on the diagonal, so dV = dO exactly and dS = 0 (dQ, dK vanish up to rounding)."""
    inp = attn_inputs(1, 2, 300, 128, dtype="bf16", seed=93, causal=True, window=1)
    do_bits, do = grad_inputs(1, 2, 300, 128, seed=94)
    dq, dk, dv = run_fwd_bwd(inp, do_bits)
    assert np.array_equal(dv, do)
    assert np.abs(dq).max() <= 1e-3 and np.abs(dk).max() <= 1e-3


def _full(name, heads, stored=True):
    w = WORKLOADS[name]
    print(f"attn_bwd full workload {name} stored={stored}", flush=True)
    inp = workload_attn_inputs(name)
    do_bits, do = grad_inputs(w["B"], w["H"], w["N"], w["d"], seed=w["seed"])
    got = run_fwd_bwd(inp, do_bits, stored)
    for g in got:
        assert np.isfinite(g).all()
    check(inp, do, got, heads=heads)


def test_bwd_full_bf16_causal_2048():
    _full("attn_bf16_causal_b4h32_n2048_d128", heads=[(0, 0), (2, 13), (3, 31)])


@pytest.mark.parametrize("stored", [True, False], ids=["stored_ds", "recompute"])
def test_bwd_full_bf16_window_pad_8192(stored):
    _full("attn_bf16_causal_w1024_pad512_b1h64_n8192_d128", heads=[(0, 0), (0, 63)], stored=stored)


def test_bwd_largest_offsets():
    """Three heads of 2^22 + 37 queries (d = 128, causal, window 100, padding): the last head starts past
    byte 2^31 of every tensor.

    Q, K, V, dO are random on the sampled blocks' dependency ranges (the W - 1
    rows before a block and after it) and zero elsewhere: a zero query with a
    zero dO adds nothing to dK, dV, so the oracle's sub-problem on that range
    gives the exact gradients of the block's rows, and a read from a wrong
    offset changes them.
    """
    B, H, N, d, W, M = 1, 3, (1 << 22) + 37, 128, 100, 48
    kvl = N - 50
    blocks = [(h, s) for h in (0, 2) for s in (0, N // 2 + 5, N - M - 60)]  # the last keys are padding
    regions = [(0, h, max(0, s - W + 1), min(N, s + M + W - 1)) for h, s in blocks]
    qb, kb, vb, dob = attn_bits_large(B, H, N, d, regions, seed=78, count=4)
    q, k, v, dout = upload_bf16(qb), upload_bf16(kb), upload_bf16(vb), upload_bf16(dob)
    assert 2 * N * d * 2 > 2**31
    scale = float(np.float32(1.0 / np.sqrt(d)))
    kv = torch.tensor([kvl], dtype=torch.int32, device="cuda:0")
    o, lse = osfa.attn_fwd(q, k, v, scale=scale, causal=True, window=W, kv_len=kv)
    grads = [Guarded((B, H, N, d), torch.bfloat16) for _ in range(3)]
    ws = Guarded(((ws_bytes(B, H, N, True, W, True) + 3) // 4,), torch.float32)  # the stored-dS way
    osfa.attn_bwd(q, k, v, o, dout, lse, scale=scale, causal=True, window=W, kv_len=kv, dq=grads[0].t,
                  dk=grads[1].t, dv=grads[2].t, workspace=ws.t)
    torch.cuda.synchronize()
    for g in grads:
        g.check()
    ws.check()
    for (h, s), (_, _, lo, hi) in zip(blocks, regions):
        sl = (slice(0, 1), slice(h, h + 1), slice(lo, hi))
        args = tuple(bf16_bits_to_f32(a[sl]) for a in (qb, kb, vb, dob)) + (scale,)
        kw = dict(causal=True, window=W, kv_len=[max(0, min(kvl, hi) - lo)])
        ref = attention_bwd_ref(*args, **kw)
        bnd = attention_bwd_error_bound(*args, **kw)
        r = slice(s - lo, s - lo + M)
        for name, g, rf, bd in zip(("dQ", "dK", "dV"), grads, ref, bnd):
            got = g.t[0, h, s:s + M].float().cpu().numpy()
            assert_grad(got, rf[0, 0, r], bd[0, 0, r], f"h={h} rows {s}..{s + M - 1} {name}")
