"""GPU parity: attn_decode_splitkv against the FP64 oracle."""
import numpy as np
import pytest
import torch

import online_softmax_fa2_amd as osfa
from online_softmax_fa2_amd.inputs import WORKLOADS, decode_inputs, decode_slice
from oracle import decode_ref
from tests.gpu_util import Guarded, assert_normwise, upload_bf16, upload_f32

pytestmark = pytest.mark.gpu


def run_decode(inp, nsplit):
    if inp["dtype"] == "bf16":
        q, k, v = upload_bf16(inp["q_bits"]), upload_bf16(inp["k_bits"]), upload_bf16(inp["v_bits"])
    else:
        q, k, v = upload_f32(inp["q"]), upload_f32(inp["k"]), upload_f32(inp["v"])
    B, H, d = inp["q"].shape
    o = Guarded((B, H, d), torch.float32)
    osfa.attn_decode_splitkv(q, k, v, nsplit, out=o.t)
    torch.cuda.synchronize()
    o.check()
    return o.t.cpu().numpy()


def check(got, ref, what, dtype="bf16"):
    """float32 inputs: normwise relative error <= 1e-5 per head (the float32 bar; o is a weighted mean and
    crosses zero, so its elementwise relative error is unbounded).  bf16 inputs: <= 1e-2 absolute, and a
    normwise 1e-4 as a diagnostic of the float32 statistics."""
    assert not np.isnan(got).any()
    err = np.abs(got - ref)
    if dtype == "f32":
        B, H = got.shape[:2]
        for b in range(B):
            for h in range(H):
                assert_normwise(got[b, h], ref[b, h], 1e-5, what=f"{what} b={b} h={h}")
        return
    assert err.max() <= 1e-2, f"{what}: max abs err {err.max():.3e}"
    assert_normwise(got, ref, 1e-4, what=what)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,Nkv,d,nsplit", [
    (1, 1, 1, 64, 1), (1, 2, 300, 64, 1), (1, 2, 300, 64, 7), (1, 2, 300, 64, 300), (2, 3, 4097, 128, 64),
    (1, 1, 5, 128, 5), (1, 4, 2048, 128, 3), (1, 1, 100, 128, 33), (2, 1, 1000, 64, 9),
])
def test_decode_parity(dtype, B, H, Nkv, d, nsplit):
    print(f"decode {dtype} B={B} H={H} Nkv={Nkv} d={d} nsplit={nsplit}", flush=True)
    inp = decode_inputs(B, H, Nkv, d, seed=Nkv + nsplit, dtype=dtype)
    got = run_decode(inp, nsplit)
    check(got, decode_ref(inp["q"], inp["k"], inp["v"]), f"decode {dtype}", dtype)


def test_decode_split_invariance():
    inp = decode_inputs(1, 2, 5000, 128, seed=3)
    outs = [run_decode(inp, s) for s in (1, 2, 64, 4096)]  # 4096: 2500 splits of 2 keys, 1596 empty
    ref = decode_ref(inp["q"], inp["k"], inp["v"])
    for o in outs:
        check(o, ref, "split invariance")
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-5


def test_decode_equal_keys_mean():
    inp = decode_inputs(1, 1, 777, 64, seed=4, dtype="f32")
    inp["k"][:] = inp["k"][:, :, :1, :]
    got = run_decode(inp, 16)
    assert np.max(np.abs(got[0, 0] - inp["v"][0, 0].astype(np.float64).mean(axis=0))) < 1e-5


def test_decode_full_workload():
    w = WORKLOADS["decode_bf16_b1h32_nkv131072_d128_split64"]
    B, H, Nkv, d = w["B"], w["H"], w["Nkv"], w["d"]
    print("decode full workload", flush=True)
    kb = np.empty((B, H, Nkv, d), np.uint16)
    vb = np.empty((B, H, Nkv, d), np.uint16)
    qb = np.empty((B, H, d), np.uint16)
    ref = np.zeros((B, H, d))
    for h in range(H):
        q, k, v, qb[0, h], kb[0, h], vb[0, h] = decode_slice(w["seed"], 0, h, Nkv, d)
        ref[0, h] = decode_ref(q[None, None], k[None, None], v[None, None])[0, 0]
    q_t, k_t, v_t = upload_bf16(qb), upload_bf16(kb), upload_bf16(vb)
    del kb, vb
    o = Guarded((B, H, d), torch.float32)
    osfa.attn_decode_splitkv(q_t, k_t, v_t, w["nsplit"], out=o.t)
    torch.cuda.synchronize()
    o.check()
    check(o.t.cpu().numpy(), ref, "decode full")
