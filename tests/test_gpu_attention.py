"""GPU parity: attn_fwd (float32 and bfloat16) against the FP64 oracle.

Small cases span several 128-query tiles and 64-key blocks with ragged
tails and exact multiples of the block sizes, every mask combination, fully
masked rows and late maxima; the full workloads are checked element by
element on every head, in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import online_softmax_fa2_amd as osfa
from online_softmax_fa2_amd.inputs import WORKLOADS, attn_bits_large, attn_inputs, bf16_bits_to_f32, workload_attn_inputs
from oracle import attention_ref
from tests.gpu_util import (Guarded, assert_bf16_out, assert_f32_rel, assert_lse_abs, assert_normwise, oracle_map,
                            upload_bf16, upload_f32)

pytestmark = pytest.mark.gpu


def run_fwd(inp, poly_every=0):
    """attn_fwd, or attn_fwd_exp2_offload when poly_every > 0 (bf16 only)."""
    if inp.dtype == "bf16":
        q, k, v = upload_bf16(inp.q_bits), upload_bf16(inp.k_bits), upload_bf16(inp.v_bits)
        odt = torch.bfloat16
    else:
        q, k, v = upload_f32(inp.q), upload_f32(inp.k), upload_f32(inp.v)
        odt = torch.float32
    B, H, N, d = inp.q.shape
    o = Guarded((B, H, N, d), odt)
    lse = Guarded((B, H, N), torch.float32)
    kvl = None if inp.kv_len is None else torch.from_numpy(inp.kv_len).to("cuda:0")
    if poly_every:
        osfa.attn_fwd_exp2_offload(q, k, v, poly_every, scale=inp.scale, causal=inp.causal, window=inp.window,
                                   kv_len=kvl, out=o.t, lse=lse.t)
    else:
        osfa.attn_fwd(q, k, v, scale=inp.scale, causal=inp.causal, window=inp.window, kv_len=kvl, out=o.t,
                      lse=lse.t)
    torch.cuda.synchronize()
    o.check()
    lse.check()
    return o.t.float().cpu().numpy(), lse.t.cpu().numpy()


def check(inp, O, L, rows=None, heads=None):
    """Compare (selected heads / rows of) the GPU result with the oracle, element by element."""
    B, H, N, d = inp.q.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads

    def ref(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(h, h + 1))
        return attention_ref(inp.q[sl], inp.k[sl], inp.v[sl], inp.scale, causal=inp.causal, window=inp.window,
                             kv_len=None if inp.kv_len is None else inp.kv_len[b:b + 1], rows=rows)

    refs = oracle_map(ref, heads) if len(heads) > 1 else [ref(heads[0])]
    for (b, h), (Or, Lr) in zip(heads, refs):
        og = O[b, h] if rows is None else O[b, h, rows]
        lg = L[b, h] if rows is None else L[b, h, rows]
        what = f"b={b} h={h}"
        if inp.dtype == "f32":
            assert_normwise(og, Or[0, 0], 1e-5, what=what + " O")
            assert_f32_rel(lg, Lr[0, 0], 1e-5, what=what + " LSE", floor=1.0)
        else:
            assert_bf16_out(og, Or[0, 0], what=what + " O")
            assert_lse_abs(lg, Lr[0, 0], 1e-3, what=what + " LSE")


CASES = [
    # (B, H, N, d, causal, window, kv_len, n_big)
    (1, 1, 1, 64, False, 0, None, 0),
    (1, 2, 1, 128, True, 0, None, 0),
    (1, 2, 65, 64, False, 0, None, 0),
    (2, 1, 129, 128, True, 0, None, 0),
    (1, 2, 1000, 64, False, 0, None, 0),
    (1, 2, 1000, 128, True, 0, None, 0),
    (2, 2, 300, 64, True, 7, None, 0),
    (1, 2, 700, 128, True, 100, [650], 3),
    (2, 1, 500, 128, False, 60, [430, 500], 0),
    (2, 1, 333, 64, True, 0, [0, 200], 0),        # batch 0: every row fully masked
    (2, 1, 333, 128, True, 0, [0, 200], 0),
    (1, 1, 400, 128, True, 1, None, 0),           # each row sees only itself
    (1, 1, 256, 64, True, 64, [100], 0),          # window + padding: rows 163.. see nothing
    (1, 1, 256, 128, True, 64, [100], 0),
    (1, 3, 513, 128, False, 0, [257], 4),
    (3, 2, 127, 128, False, 1000, None, 0),
    (1, 1, 200, 64, False, 2**31 - 1, None, 0),   # window beyond N: no mask
    (2, 1, 150, 128, True, 2**31 - 1, [150, 77], 0),
    # exact multiples of the tile (128) and block (64) sizes, and one short of them
    (1, 2, 2, 128, True, 0, None, 0),
    (1, 2, 63, 128, False, 0, None, 0),
    (1, 2, 64, 64, True, 0, None, 0),
    (1, 2, 128, 128, True, 0, None, 0),
    (2, 1, 256, 64, False, 0, [256, 192], 0),
    (1, 1, 512, 128, True, 0, [448], 2),
    # the benchmark's window of 1024 at a size the oracle finishes quickly
    (1, 2, 1600, 128, True, 1024, [1400], 3),
    (1, 1, 2048, 64, True, 1024, None, 0),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_fwd_parity(dtype, case):
    B, H, N, d, causal, window, kv_len, nbig = case
    print(f"attn_fwd {dtype} B={B} H={H} N={N} d={d} causal={causal} window={window} kv_len={kv_len}", flush=True)
    inp = attn_inputs(B, H, N, d, dtype=dtype, seed=N + d + B, causal=causal, window=window, kv_len=kv_len,
                      n_big_keys=nbig)
    O, L = run_fwd(inp)
    check(inp, O, L)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_late_maxima_and_far_apart_rows(dtype):
    """Large scores planted in the last keys; rows whose scores sit +-1000 apart in one tile."""
    inp = attn_inputs(1, 1, 1000, 64, dtype=dtype, seed=90)
    inp.k[:, :, -5:, :] *= 8.0
    if dtype == "bf16":
        from online_softmax_fa2_amd.inputs import bf16_round
        inp.k_bits, inp.k = bf16_round(inp.k)
    O, L = run_fwd(inp)
    check(inp, O, L)
    inp2 = attn_inputs(1, 1, 256, 64, dtype=dtype, seed=91)
    inp2.q[0, 0, ::2] *= 0.0
    inp2.q[0, 0, ::2, 0] = 400.0
    inp2.q[0, 0, 1::2, 0] = -400.0
    inp2.k[0, 0, :, 0] = np.abs(inp2.k[0, 0, :, 0]) + 0.5
    if dtype == "bf16":
        from online_softmax_fa2_amd.inputs import bf16_round
        inp2.q_bits, inp2.q = bf16_round(inp2.q)
        inp2.k_bits, inp2.k = bf16_round(inp2.k)
    O, L = run_fwd(inp2)
    check(inp2, O, L)


def test_fwd_closed_forms_bf16():
    """Causal window 1: O_i = v_i exactly; V = 1: O = 1 exactly."""
    inp = attn_inputs(1, 2, 300, 128, dtype="bf16", seed=92, causal=True, window=1)
    O, L = run_fwd(inp)
    assert np.array_equal(O, inp.v)
    inp.v[:] = 1.0
    inp.v_bits[:] = 0x3F80
    inp.window = 0
    O, _ = run_fwd(inp)
    assert np.all(O == 1.0)


def _full(name, heads=None, nrows=64, poly_every=0):
    """The full workload; heads=None compares every head whole, otherwise the listed heads whole plus sampled
    rows of every fifth head."""
    w = WORKLOADS[name]
    print(f"attn_fwd full workload {name} poly_every={poly_every}", flush=True)
    inp = workload_attn_inputs(name)
    O, L = run_fwd(inp, poly_every)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    check(inp, O, L, heads=heads)
    if heads is not None:
        rng = np.random.default_rng(123)
        rows = np.sort(rng.choice(w["N"], nrows, replace=False))
        rows = np.unique(np.concatenate([rows, [0, w["N"] - 1]]))
        all_heads = [(b, h) for b in range(w["B"]) for h in range(w["H"])]
        check(inp, O, L, rows=rows, heads=all_heads[::5])
    return inp, O, L


@pytest.mark.parametrize("poly_every", [2, 4, 8])
@pytest.mark.parametrize("case", [c for c in CASES if c[3] == 128], ids=[f"c{i}" for i, c in enumerate(CASES) if c[3] == 128])
def test_fwd_exp2_offload_parity(case, poly_every):
    """The variant with part of the exponentials on the FMA pipes meets the same bar as attn_fwd."""
    B, H, N, d, causal, window, kv_len, n_big = case
    print(f"attn_fwd_exp2_offload poly_every={poly_every} B={B} H={H} N={N} causal={causal} window={window}", flush=True)
    inp = attn_inputs(B, H, N, d, dtype="bf16", seed=200 + N, causal=causal, window=window, kv_len=kv_len,
                      n_big_keys=n_big)
    O, L = run_fwd(inp, poly_every)
    check(inp, O, L)


def test_fwd_exp2_offload_full_window_pad_8192():
    """The variant in the launch configuration the benchmark times (one pair in four on the FMA pipes)."""
    _full("attn_bf16_causal_w1024_pad512_b1h64_n8192_d128", heads=[(0, 0)], nrows=48, poly_every=4)


@pytest.mark.parametrize("B,H,N,d,causal,window,kv_len", [
    (2, 16, 1100, 64, True, 300, [1100, 1000]),
    (1, 32, 1030, 128, False, 0, None),
])
def test_fwd_f32_tile_path(B, H, N, d, causal, window, kv_len):
    """float32 launches with at least 256 tiles of 128 queries take the 128-query tile kernel; launches with
    fewer take a key-split kernel: 32-query workgroups (test_fwd_f32_split32_path), or 16-query ones when
    there are fewer than 256 tiles of 32 queries, which the other float32 cases here run (d = 64 and 128)."""
    assert B * H * ((N + 127) // 128) >= 256
    print(f"attn_fwd f32 tile path B={B} H={H} N={N} d={d}", flush=True)
    inp = attn_inputs(B, H, N, d, dtype="f32", seed=N + d, causal=causal, window=window, kv_len=kv_len)
    O, L = run_fwd(inp)
    check(inp, O, L, heads=[(0, 0), (B - 1, H - 1), (0, H // 2)])


@pytest.mark.parametrize("B,H,N,d,causal,window,kv_len", [
    (1, 16, 600, 64, True, 200, None),
    (1, 8, 1100, 128, False, 0, [900]),
    (2, 5, 833, 64, False, 100, [833, 17]),
])
def test_fwd_f32_split32_path(B, H, N, d, causal, window, kv_len):
    """float32 launches with fewer than 256 tiles of 128 queries but at least 256 of 32 take the key-split
    kernel with 32-query workgroups."""
    assert B * H * ((N + 127) // 128) < 256 <= B * H * ((N + 31) // 32)
    print(f"attn_fwd f32 split32 path B={B} H={H} N={N} d={d}", flush=True)
    inp = attn_inputs(B, H, N, d, dtype="f32", seed=N + 3 * d, causal=causal, window=window, kv_len=kv_len)
    O, L = run_fwd(inp)
    check(inp, O, L, heads=[(0, 0), (B - 1, H - 1), (0, H // 2)])


def test_fwd_full_f32_n1000():
    inp = workload_attn_inputs("attn_f32_b1h1_n1000_d64")
    O, L = run_fwd(inp)
    check(inp, O, L)


def test_fwd_full_bf16_causal_2048():
    """All 128 heads of the causal 4 x 32 x 2048 workload, element by element."""
    _full("attn_bf16_causal_b4h32_n2048_d128")


def test_fwd_full_bf16_window_pad_8192():
    """All 64 heads of the window + padding workload, element by element."""
    inp, O, L = _full("attn_bf16_causal_w1024_pad512_b1h64_n8192_d128")
    # every query sees at least itself or the keys before the padding: no -inf rows here
    assert np.all(np.isfinite(L))


def test_fwd_bf16_largest_offsets():
    """Three heads of 2^22 + 37 queries (d = 128): the last head starts past byte 2^31 of each tensor.

    Q, K, V are random on the rows of the sampled blocks and their visible
    keys (start, middle and end of the first and the last head) and zero
    elsewhere, so a read from a wrong offset changes a sampled result.  The
    oracle solves the sub-problem of each block's visible keys (causal and
    window masks only depend on i - j, so a shifted slice reproduces them).
    """
    B, H, N, d, W, M = 1, 3, (1 << 22) + 37, 128, 100, 48
    kvl = N - 50
    blocks = [(h, s) for h in (0, 2) for s in (0, N // 2 + 5, N - M)]
    regions = [(0, h, max(0, s - W + 1), s + M) for h, s in blocks]
    qb, kb, vb = attn_bits_large(B, H, N, d, regions, seed=77)
    q, k, v = upload_bf16(qb), upload_bf16(kb), upload_bf16(vb)
    assert 2 * N * d * 2 > 2**31  # byte offset of the last head
    scale = 1.0 / np.sqrt(d)
    o = Guarded((B, H, N, d), torch.bfloat16)
    lse = Guarded((B, H, N), torch.float32)
    osfa.attn_fwd(q, k, v, scale=scale, causal=True, window=W, kv_len=torch.tensor([kvl], dtype=torch.int32,
                  device="cuda:0"), out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    o.check()
    lse.check()
    for (h, s), (_, _, lo, hi) in zip(blocks, regions):
        sl = (slice(0, 1), slice(h, h + 1), slice(lo, hi))
        Or, Lr = attention_ref(bf16_bits_to_f32(qb[sl]), bf16_bits_to_f32(kb[sl]), bf16_bits_to_f32(vb[sl]),
                               scale, causal=True, window=W, kv_len=[max(0, min(kvl, hi) - lo)],
                               rows=np.arange(s - lo, s - lo + M))
        og = o.t[0, h, s:s + M].float().cpu().numpy()
        lg = lse.t[0, h, s:s + M].cpu().numpy()
        what = f"h={h} rows {s}..{s + M - 1}"
        assert_bf16_out(og, Or[0, 0], what=what + " O")
        assert_lse_abs(lg, Lr[0, 0], 1e-3, what=what + " LSE")


def _sweep_configs(n=16, seed=20261202):
    """Seeded random forward configurations: sizes from 1 to ~900 queries (log-uniform), both head
    dimensions, causal or not, a window on half of them, per-batch padding on some, planted large keys on
    some. Every launch path of attn_fwd's small sizes is drawn (FP32: the 16-query split kernel; bf16: the
    d = 64 and d = 128 tile kernels)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(np.clip(np.exp(rng.uniform(0, np.log(900))), 1, 900))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        window = int(rng.integers(1, N + 40)) if rng.uniform() < 0.5 else 0
        kv_len = [int(x) for x in rng.integers(0, N + 1, size=B)] if rng.uniform() < 0.4 else None
        big = int(rng.integers(0, min(N, 4) + 1))
        out.append((B, H, N, d, causal, window, kv_len, big))
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cfg", _sweep_configs(), ids=[f"s{i}" for i in range(16)])
def test_fwd_random_sweep(dtype, cfg):
    """Every head of every drawn configuration against the oracle, element by element, at the dtype's bar."""
    B, H, N, d, causal, window, kv_len, big = cfg
    print(f"attn_fwd sweep {dtype} B={B} H={H} N={N} d={d} causal={causal} window={window} kv_len={kv_len} "
          f"big={big}", flush=True)
    inp = attn_inputs(B, H, N, d, dtype=dtype, seed=N * 7 + d + B, causal=causal, window=window, kv_len=kv_len,
                      n_big_keys=big)
    O, L = run_fwd(inp)
    check(inp, O, L)
