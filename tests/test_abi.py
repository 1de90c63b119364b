"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
and rejects invalid arguments on the host before any launch.

Calls with invalid arguments fail validation before any launch (the fake
pointers are never dereferenced).  The only valid calls are in
``test_valid_call_without_a_device_reports_hip_error``, which runs only where
no GPU is visible: there the launch itself is refused by the runtime.
"""
import ctypes
import os
import re

import pytest

from online_softmax_fa2_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osfa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from online_softmax_fa2_amd.build import build_library
        build_library()
    return bd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("attn_fwd", "attn_fwd_fp8", "attn_bwd", "attn_bwd_workspace_bytes",
                 "attn_bwd_stored_ds_workspace_bytes", "attn_decode_splitkv",
                 "attn_decode_splitkv_workspace_bytes",
                 "online_softmax_rows", "online_softmax_topk_rows", "attn_last_error", "osfa_version"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in osfa.h but not exported"
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version(lib):
    assert b"gfx950" in lib.osfa_version()


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced


def _fwd(lib, **kw):
    a = dict(dtype=bd.ATTN_BF16, Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, B=1, H=1, N=16, d=128, scale=0.1,
             causal=0, window=0, kv_len=None, stream=None)
    a.update(kw)
    return lib.attn_fwd(a["dtype"], a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["N"], a["d"],
                        a["scale"], a["causal"], a["window"], a["kv_len"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Q=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(LSE=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(N=0), bd.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(B=-1), bd.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(d=96), bd.ATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(d=256), bd.ATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(scale=0.0), bd.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=-1.0), bd.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), bd.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("inf")), bd.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(causal=2), bd.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(window=-3), bd.ATTN_ERR_INVALID_ARG, "window"),
    (dict(dtype=7), bd.ATTN_ERR_INVALID_ARG, "dtype"),
    (dict(Q=FAKE + 2), bd.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(B=1 << 12, H=1 << 12, N=1 << 12, d=128), bd.ATTN_ERR_INVALID_ARG, "too large"),
    (dict(N=1 << 23, d=128), bd.ATTN_ERR_INVALID_ARG, "one head"),
    (dict(LSE=FAKE + 2), bd.ATTN_ERR_INVALID_ARG, "LSE and kv_len"),
    (dict(kv_len=FAKE + 1), bd.ATTN_ERR_INVALID_ARG, "LSE and kv_len"),
])
def test_attn_fwd_rejects(lib, kw, status, msg):
    assert _fwd(lib, **kw) == status
    assert msg in lib.attn_last_error().decode()


def _exp2_offload(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, B=1, H=1, N=16, d=128, scale=0.1, causal=0, window=0,
             kv_len=None, poly_every=4, stream=None)
    a.update(kw)
    return lib.attn_fwd_exp2_offload(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["N"], a["d"],
                                     a["scale"], a["causal"], a["window"], a["kv_len"], a["poly_every"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(poly_every=3), bd.ATTN_ERR_UNSUPPORTED, "poly_every"),
    (dict(poly_every=0), bd.ATTN_ERR_UNSUPPORTED, "poly_every"),
    (dict(poly_every=16), bd.ATTN_ERR_UNSUPPORTED, "poly_every"),
    (dict(d=64), bd.ATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(V=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(N=0), bd.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(scale=float("nan")), bd.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(causal=5), bd.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(window=-1), bd.ATTN_ERR_INVALID_ARG, "window"),
    (dict(O=FAKE + 8), bd.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(N=1 << 23), bd.ATTN_ERR_INVALID_ARG, "one head"),
    (dict(LSE=FAKE + 1), bd.ATTN_ERR_INVALID_ARG, "LSE and kv_len"),
    (dict(kv_len=FAKE + 2), bd.ATTN_ERR_INVALID_ARG, "LSE and kv_len"),
])
def test_exp2_offload_rejects(lib, kw, status, msg):
    assert _exp2_offload(lib, **kw) == status
    assert msg in lib.attn_last_error().decode()


def test_workspace_bytes(lib):
    assert lib.attn_decode_splitkv_workspace_bytes(1, 32, 128, 64) == 32 * 64 * 130 * 4
    assert lib.attn_decode_splitkv_workspace_bytes(2, 3, 64, 7) == 2 * 3 * 7 * 66 * 4
    assert lib.attn_decode_splitkv_workspace_bytes(0, 3, 64, 7) == 0
    assert lib.attn_decode_splitkv_workspace_bytes(1, 3, 64, 0) == 0


def _dec(lib, **kw):
    a = dict(dtype=bd.ATTN_BF16, q=FAKE, K=FAKE, V=FAKE, o=FAKE, B=1, H=2, Nkv=100, d=128, nsplit=4, ws=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.attn_decode_splitkv(a["dtype"], a["q"], a["K"], a["V"], a["o"], a["B"], a["H"], a["Nkv"], a["d"],
                                   a["nsplit"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(ws=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(Nkv=0), bd.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(d=80), bd.ATTN_ERR_UNSUPPORTED, "not built"),
    (dict(nsplit=0), bd.ATTN_ERR_INVALID_ARG, "nsplit"),
    (dict(nsplit=101), bd.ATTN_ERR_INVALID_ARG, "nsplit"),
    (dict(Nkv=100000, nsplit=5000), bd.ATTN_ERR_INVALID_ARG, "nsplit"),
    (dict(ws_bytes=2 * 4 * 130 * 4 - 1), bd.ATTN_ERR_INVALID_ARG, "workspace"),
    (dict(K=FAKE + 4), bd.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(dtype=3), bd.ATTN_ERR_INVALID_ARG, "dtype"),
])
def test_decode_rejects(lib, kw, status, msg):
    assert _dec(lib, **kw) == status
    assert msg in lib.attn_last_error().decode()


def _fp8(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, B=1, H=2, N=16, d=128, scale=0.1, qd=0.01, kd=0.02, vd=0.03,
             causal=0, window=0, kv_len=None, stream=None)
    a.update(kw)
    return lib.attn_fwd_fp8(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                            a["qd"], a["kd"], a["vd"], a["causal"], a["window"], a["kv_len"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(V=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(B=0), bd.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(d=64), bd.ATTN_ERR_UNSUPPORTED, "not built"),
    (dict(qd=0.0), bd.ATTN_ERR_INVALID_ARG, "descale"),
    (dict(vd=float("nan")), bd.ATTN_ERR_INVALID_ARG, "descale"),
    (dict(scale=-1.0), bd.ATTN_ERR_INVALID_ARG, "descale"),
    (dict(qd=1e30, kd=1e30), bd.ATTN_ERR_INVALID_ARG, "range"),
    (dict(causal=3), bd.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(window=-1), bd.ATTN_ERR_INVALID_ARG, "window"),
    (dict(O=FAKE + 4), bd.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(N=1 << 23), bd.ATTN_ERR_INVALID_ARG, "one head"),
    (dict(LSE=FAKE + 2), bd.ATTN_ERR_INVALID_ARG, "LSE and kv_len"),
    (dict(kv_len=FAKE + 3), bd.ATTN_ERR_INVALID_ARG, "LSE and kv_len"),
])
def test_fp8_rejects(lib, kw, status, msg):
    assert _fp8(lib, **kw) == status
    assert msg in lib.attn_last_error().decode()


def _bwd(lib, **kw):
    a = dict(dtype=bd.ATTN_BF16, Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE, B=1, H=2,
             N=16, d=128, scale=0.1, causal=0, window=0, kv_len=None, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.attn_bwd(a["dtype"], a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
                        a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["window"], a["kv_len"], a["ws"],
                        a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dO=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(ws=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(N=0), bd.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(d=64), bd.ATTN_ERR_UNSUPPORTED, "not built"),
    (dict(dtype=bd.ATTN_F32), bd.ATTN_ERR_UNSUPPORTED, "bf16"),
    (dict(dtype=5), bd.ATTN_ERR_INVALID_ARG, "dtype"),
    (dict(scale=0.0), bd.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(causal=2), bd.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(window=-3), bd.ATTN_ERR_INVALID_ARG, "window"),
    (dict(ws_bytes=2 * 2 * 16 * 4 - 1), bd.ATTN_ERR_INVALID_ARG, "workspace"),
    (dict(dK=FAKE + 8), bd.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(LSE=FAKE + 2), bd.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(kv_len=FAKE + 2), bd.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(N=1 << 23), bd.ATTN_ERR_INVALID_ARG, "one head"),
])
def test_bwd_rejects(lib, kw, status, msg):
    assert _bwd(lib, **kw) == status
    assert msg in lib.attn_last_error().decode()


def test_bwd_workspace_bytes(lib):
    assert lib.attn_bwd_workspace_bytes(2, 3, 5) == 2 * 2 * 3 * 5 * 4
    assert lib.attn_bwd_workspace_bytes(0, 3, 5) == 0


def test_bwd_stored_ds_workspace_bytes(lib):
    """The D / LSE part rounded up to 256 bytes, then one 2 KB tile per (32-query block, visible 32-key block slot)."""
    f = lib.attn_bwd_stored_ds_workspace_bytes
    f.argtypes = [ctypes.c_int] * 5
    f.restype = ctypes.c_size_t
    # N = 8192: 256 query blocks; causal window 1024 -> 33 key-block slots, non-causal -> 66, none -> 256.
    assert f(1, 64, 8192, 1, 1024) == 64 * 8192 * 8 + 64 * 256 * 33 * 2048
    assert f(1, 1, 8192, 0, 1024) == 65536 + 256 * 66 * 2048
    assert f(1, 1, 8192, 1, 0) == 65536 + 256 * 256 * 2048
    assert f(2, 1, 100, 1, 5000) == 1792 + 2 * 4 * 4 * 2048  # window clamped to N; 1600 B rounded up to 1792
    assert f(1, 1, 1 << 20, 0, 0) == 0  # one head's tiles would pass 2^31 bytes
    assert f(0, 1, 8, 0, 0) == 0 and f(1, 1, 8, 2, 0) == 0 and f(1, 1, 8, 0, -1) == 0


@pytest.mark.parametrize("args,msg", [
    ((None, FAKE, 4, 4), "null"),
    ((FAKE, FAKE, 0, 4), "rows"),
    ((FAKE, FAKE, 4, 0), "rows"),
    ((FAKE, FAKE + 4 * 3, 4, 4), "overlap"),
    ((FAKE + 1, FAKE + 1, 4, 4), "aligned"),
])
def test_softmax_rejects(lib, args, msg):
    x, y, rows, cols = args
    assert lib.online_softmax_rows(x, y, rows, cols, None) == bd.ATTN_ERR_INVALID_ARG
    assert msg in lib.attn_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(k=0), bd.ATTN_ERR_INVALID_ARG, "k=0"),
    (dict(k=11, cols=10), bd.ATTN_ERR_INVALID_ARG, "k=11"),
    (dict(k=17), bd.ATTN_ERR_UNSUPPORTED, "k=17"),
    (dict(x=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(topi=None), bd.ATTN_ERR_INVALID_ARG, "null"),
    (dict(y=FAKE), bd.ATTN_ERR_INVALID_ARG, "alias"),
    (dict(rows=0), bd.ATTN_ERR_INVALID_ARG, "rows"),
])
def test_topk_rejects(lib, kw, status, msg):
    a = dict(x=FAKE, y=None, topv=FAKE * 2, topi=FAKE * 3, rows=4, cols=100, k=5)
    a.update(kw)
    assert lib.online_softmax_topk_rows(a["x"], a["y"], a["topv"], a["topi"], a["rows"], a["cols"], a["k"],
                                        None) == status
    assert msg in lib.attn_last_error().decode()


def test_error_text_is_per_thread(lib):
    import threading
    assert _fwd(lib, d=96) == bd.ATTN_ERR_UNSUPPORTED
    seen = {}

    def other():
        seen["text"] = lib.attn_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["text"] == ""
    assert "head dim" in lib.attn_last_error().decode()


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        bd.online_softmax_rows(x)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every entry point raises instead of computing anything."""
    import torch
    import online_softmax_fa2_amd as osfa
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "libosfa.so"))
    monkeypatch.setattr(bd, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        bd.load_library()
    x = torch.zeros(4, 8)
    with pytest.raises((RuntimeError, ValueError)):
        osfa.online_softmax_rows(x)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="valid calls with fake pointers must never reach a real device")
def test_valid_call_without_a_device_reports_hip_error(lib):
    """Valid arguments and no device: every entry point returns ATTN_ERR_HIP (the runtime refuses the launch),
    never crashes and never reports success."""
    calls = {
        "attn_fwd": lambda: _fwd(lib),
        "attn_fwd_exp2_offload": lambda: _exp2_offload(lib),
        "attn_fwd_fp8": lambda: _fp8(lib),
        "attn_bwd": lambda: _bwd(lib),
        "attn_decode_splitkv": lambda: _dec(lib),
        "attn_decode_splitkv_noalloc": lambda: lib.attn_decode_splitkv_noalloc(bd.ATTN_BF16, FAKE, FAKE, FAKE, FAKE, 1,
                                                                               2, 100, 128, 4, None),
        "online_softmax_rows": lambda: lib.online_softmax_rows(FAKE, FAKE, 4, 100, None),
        "online_softmax_topk_rows": lambda: lib.online_softmax_topk_rows(FAKE, None, FAKE * 2, FAKE * 3, 4, 100, 5,
                                                                         None),
    }
    for name, call in calls.items():
        assert call() == bd.ATTN_ERR_HIP, name
        text = lib.attn_last_error().decode()
        assert name in text and "launch failed" in text, text


def _cpu(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("which", ["out_dtype", "out_shape", "lse_shape", "lse_dtype"])
def test_binding_checks_supplied_outputs_before_any_launch(which):
    """A caller-supplied output of the wrong dtype or shape raises ValueError before the library is called
    (the ABI cannot see buffer sizes: a short buffer would be written past its end)."""
    import torch
    q = _cpu((1, 2, 16, 128), torch.bfloat16)
    out, lse = _cpu((1, 2, 16, 128), torch.bfloat16), _cpu((1, 2, 16), torch.float32)
    if which == "out_dtype":
        out = _cpu((1, 2, 16, 128), torch.float32)
    elif which == "out_shape":
        out = _cpu((1, 2, 15, 128), torch.bfloat16)
    elif which == "lse_shape":
        lse = _cpu((1, 2, 8), torch.float32)
    else:
        lse = _cpu((1, 2, 16), torch.bfloat16)
    name = "out" if which.startswith("out") else "lse"
    for fn in (lambda: bd.attn_fwd(q, q, q, out=out, lse=lse),
               lambda: bd.attn_fwd_exp2_offload(q, q, q, 4, out=out, lse=lse)):
        with pytest.raises(ValueError, match=f"^{name} must be"):
            fn()


def test_binding_checks_other_supplied_outputs():
    import torch
    q = _cpu((1, 2, 16, 128), torch.bfloat16)
    lse = _cpu((1, 2, 16), torch.float32)
    with pytest.raises(ValueError, match="^dk must be"):
        bd.attn_bwd(q, q, q, q, q, lse, dk=_cpu((1, 2, 16, 128), torch.float32))
    u8 = _cpu((1, 2, 16, 128), torch.uint8)
    with pytest.raises(ValueError, match="^out must be"):
        bd.attn_fwd_fp8(u8, u8, u8, 1.0, 1.0, 1.0, out=_cpu((1, 2, 16, 128), torch.float32))
    with pytest.raises(ValueError, match="^out must be"):
        bd.attn_decode_splitkv(_cpu((1, 2, 128), torch.bfloat16), q, q, 4, out=_cpu((1, 2, 128), torch.bfloat16))
    x = _cpu((4, 100), torch.float32)
    with pytest.raises(ValueError, match="^out must be"):
        bd.online_softmax_rows(x, out=_cpu((4, 99), torch.float32))
