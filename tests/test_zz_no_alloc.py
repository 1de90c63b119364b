"""GPU test of attn_decode_splitkv_noalloc, the decode entry point that allocates nothing.

Called through the C ABI (ctypes, no torch allocation inside the call): two
calls in a row, the second on a smaller input, each compared with
attn_decode_splitkv on the same inputs (the same kernels, so the results
must be identical) and with the FP64 oracle at the decode bar; a request
larger than the scratch array is refused before any launch.
"""
import numpy as np
import pytest
import torch

import online_softmax_fa2_amd as osfa
from online_softmax_fa2_amd import _binding as bd
from online_softmax_fa2_amd.inputs import decode_inputs
from oracle import decode_ref
from tests.gpu_util import Guarded, assert_normwise, upload_bf16, upload_f32

pytestmark = pytest.mark.gpu


def _inputs(B, H, Nkv, d, dtype, seed):
    inp = decode_inputs(B, H, Nkv, d, seed=seed, dtype=dtype)
    up = (lambda n: upload_bf16(inp[n + "_bits"])) if dtype == "bf16" else (lambda n: upload_f32(inp[n]))
    return inp, up("q"), up("k"), up("v")


def _noalloc(lib, dtype, q, k, v, out, nsplit):
    B, H, Nkv, d = k.shape
    st = lib.attn_decode_splitkv_noalloc(bd.ATTN_BF16 if dtype == "bf16" else bd.ATTN_F32, q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), out.data_ptr(), B, H, Nkv, d, nsplit,
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.attn_last_error()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_matches_workspace_decode_twice(dtype):
    lib = osfa.load_library()
    cases = [(2, 16, 20000, 128, 64), (1, 3, 777, 64, 9)]  # the second call is smaller
    for i, (B, H, Nkv, d, nsplit) in enumerate(cases):
        print(f"decode noalloc {dtype} B={B} H={H} Nkv={Nkv} d={d} nsplit={nsplit}", flush=True)
        assert osfa.decode_workspace_bytes(B, H, d, nsplit) <= bd.DECODE_NOALLOC_SCRATCH_BYTES
        inp, q, k, v = _inputs(B, H, Nkv, d, dtype, seed=40 + i)
        got = Guarded((B, H, d), torch.float32)
        _noalloc(lib, dtype, q, k, v, got.t, nsplit)
        want = osfa.attn_decode_splitkv(q, k, v, nsplit)
        torch.cuda.synchronize()
        got.check()
        g, w = got.t.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g, w), f"differs from attn_decode_splitkv by {np.abs(g - w).max():.3e}"
        ref = decode_ref(inp["q"], inp["k"], inp["v"])
        if dtype == "f32":
            for b in range(B):
                for h in range(H):
                    assert_normwise(g[b, h], ref[b, h], 1e-5, what=f"noalloc f32 b={b} h={h}")
        else:
            assert np.abs(g - ref).max() <= 1e-2


def test_noalloc_decode_refuses_more_than_its_scratch():
    lib = osfa.load_library()
    B, H, d, nsplit = 1, 64, 128, 128  # 64 * 128 * 130 * 4 bytes > 4 MiB
    assert osfa.decode_workspace_bytes(B, H, d, nsplit) > bd.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((B, H, 256, d), dtype=torch.bfloat16, device="cuda:0")
    out = torch.zeros((B, H, d), dtype=torch.float32, device="cuda:0")
    st = lib.attn_decode_splitkv_noalloc(bd.ATTN_BF16, q.data_ptr(), k.data_ptr(), k.data_ptr(), out.data_ptr(), B, H,
                                         256, d, nsplit, torch.cuda.current_stream().cuda_stream)
    assert st == bd.ATTN_ERR_INVALID_ARG and b"scratch" in lib.attn_last_error()
