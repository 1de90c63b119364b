"""ctypes binding over libosfa.so: argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI
(``include/osfa.h``).  PyTorch supplies device memory and the current stream.
If the library is not built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libosfa.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_BF16 = 0, 1
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_HIP"}

_lib = None


class OsfaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libosfa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m online_softmax_fa2_amd.build` "
                           "(or __graft_entry__.build()) first; there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    p, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [i, p, p, p, p, p, i, i, i, i, f, i, i, p, p]
    lib.attn_fwd.restype = i
    lib.attn_fwd_exp2_offload.argtypes = [p, p, p, p, p, i, i, i, i, f, i, i, p, i, p]
    lib.attn_fwd_exp2_offload.restype = i
    lib.attn_fwd_fp8.argtypes = [p, p, p, p, p, i, i, i, i, f, f, f, f, i, i, p, p]
    lib.attn_fwd_fp8.restype = i
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd_stored_ds_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_stored_ds_workspace_bytes.restype = sz
    lib.attn_bwd.argtypes = [i, p, p, p, p, p, p, p, p, p, i, i, i, i, f, i, i, p, p, sz, p]
    lib.attn_bwd.restype = i
    lib.attn_decode_splitkv_workspace_bytes.argtypes = [i, i, i, i]
    lib.attn_decode_splitkv_workspace_bytes.restype = sz
    lib.attn_decode_splitkv.argtypes = [i, p, p, p, p, i, i, i, i, i, p, sz, p]
    lib.attn_decode_splitkv.restype = i
    lib.attn_decode_splitkv_noalloc.argtypes = [i, p, p, p, p, i, i, i, i, i, p]
    lib.attn_decode_splitkv_noalloc.restype = i
    lib.online_softmax_rows.argtypes = [p, p, i, i, p]
    lib.online_softmax_rows.restype = i
    lib.online_softmax_topk_rows.argtypes = [p, p, p, p, i, i, i, p]
    lib.online_softmax_topk_rows.restype = i
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.osfa_version.argtypes = []
    lib.osfa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise OsfaError(status, load_library().attn_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need_device(*ts) -> None:
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _need_out(t, shape, dtype, like, name: str) -> None:
    """A caller-supplied output must match exactly: the C ABI cannot see sizes, so a short or mistyped buffer
    would be written past its end."""
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != like.device:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {like.device} "
                         f"(got {t.dtype} {tuple(t.shape)} on {t.device})")


_DT = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = False, window: int = 0,
             kv_len=None, out=None, lse=None, stream=None):
    """O, LSE = attention(q, k, v) for [B, H, N, d] tensors (f32 or bf16)."""
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need_out(out, q.shape, q.dtype, q, "out")
    _need_out(lse, (B, H, N), torch.float32, q, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if kv_len is not None and (kv_len.dtype != torch.int32 or kv_len.numel() != B or kv_len.device != q.device):
        raise ValueError("kv_len must be int32 [B] on the device of q")
    _need_device(q, k, v, kv_len, out, lse)
    _check(load_library().attn_fwd(_DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                   float(scale), int(bool(causal)), int(window), _ptr(kv_len), _stream(stream)))
    return out, lse


def attn_fwd_exp2_offload(q, k, v, poly_every: int, scale: float | None = None, causal: bool = False,
                          window: int = 0, kv_len=None, out=None, lse=None, stream=None):
    """attn_fwd for bf16 [B, H, N, 128] with one exponential in poly_every (2, 4, 8) on the FMA pipes."""
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need_out(out, q.shape, q.dtype, q, "out")
    _need_out(lse, (B, H, N), torch.float32, q, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if kv_len is not None and (kv_len.dtype != torch.int32 or kv_len.numel() != B or kv_len.device != q.device):
        raise ValueError("kv_len must be int32 [B] on the device of q")
    _need_device(q, k, v, kv_len, out, lse)
    _check(load_library().attn_fwd_exp2_offload(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                                float(scale), int(bool(causal)), int(window), _ptr(kv_len),
                                                int(poly_every), _stream(stream)))
    return out, lse


def attn_fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float, scale: float | None = None,
                 causal: bool = False, window: int = 0, kv_len=None, out=None, lse=None, stream=None):
    """O (bf16), LSE = attention of e4m3 codes q, k, v ([B, H, N, d], uint8 or float8_e4m3fn) x their descales."""
    ok = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    if q.dtype not in ok or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype uint8 or float8_e4m3fn (e4m3 codes)")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need_out(out, q.shape, torch.bfloat16, q, "out")
    _need_out(lse, (B, H, N), torch.float32, q, "lse")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if kv_len is not None and (kv_len.dtype != torch.int32 or kv_len.numel() != B or kv_len.device != q.device):
        raise ValueError("kv_len must be int32 [B] on the device of q")
    _need_device(q, k, v, kv_len, out, lse)
    _check(load_library().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                                       float(q_descale), float(k_descale), float(v_descale), int(bool(causal)),
                                       int(window), _ptr(kv_len), _stream(stream)))
    return out, lse


def bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, H, N))


def bwd_stored_ds_workspace_bytes(B: int, H: int, N: int, causal: bool = False, window: int = 0) -> int:
    """Workspace bytes with which attn_bwd stores dS and forms dQ from it (0: that way does not apply)."""
    return int(load_library().attn_bwd_stored_ds_workspace_bytes(B, H, N, int(bool(causal)), int(window)))


# Largest workspace attn_bwd allocates by itself to store dS; beyond it (or beyond a quarter of the free
# device memory) it takes the minimum workspace and recomputes.  dS takes 2 bytes per visible pair, which
# without a window grows as N^2.
STORED_DS_MAX_BYTES = 8 << 30


def attn_bwd(q, k, v, o, dout, lse, scale: float | None = None, causal: bool = False, window: int = 0,
             kv_len=None, dq=None, dk=None, dv=None, workspace=None, stream=None, stored_ds: bool = True):
    """(dQ, dK, dV) of attention for [B, H, N, d] bf16 tensors, given O and LSE from attn_fwd.

    Without a `workspace`, one is allocated: large enough to store dS (the faster way) when `stored_ds`,
    that way applies and it needs at most STORED_DS_MAX_BYTES and a quarter of the free device memory;
    else the minimum (dQ recomputes S and dP).  A given workspace decides by its size.
    """
    if q.dtype not in _DT or any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must share one dtype")
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must all be [B, H, N, d]")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or lse.shape != (B, H, N):
        raise ValueError("lse must be float32 [B, H, N]")
    if kv_len is not None and (kv_len.dtype != torch.int32 or kv_len.numel() != B or kv_len.device != q.device):
        raise ValueError("kv_len must be int32 [B] on the device of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need_out(t, q.shape, q.dtype, q, name)
    if workspace is not None and (workspace.device != q.device or
                                  workspace.numel() * workspace.element_size() < bwd_workspace_bytes(B, H, N)):
        raise ValueError("workspace must be on the device of q and hold bwd_workspace_bytes(B, H, N) bytes")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    need = bwd_workspace_bytes(B, H, N)
    if stored_ds and workspace is None:
        st = bwd_stored_ds_workspace_bytes(B, H, N, causal, window)
        if 0 < st <= STORED_DS_MAX_BYTES and st <= torch.cuda.mem_get_info(q.device)[0] // 4:
            need = max(need, st)
    if workspace is None:
        workspace = torch.empty((max(need, 4) + 3) // 4, dtype=torch.float32, device=q.device)
    _need_device(q, k, v, o, dout, lse, kv_len, dq, dk, dv, workspace)
    _check(load_library().attn_bwd(_DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                                   int(window), _ptr(kv_len), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def decode_workspace_bytes(B: int, H: int, d: int, nsplit: int) -> int:
    return int(load_library().attn_decode_splitkv_workspace_bytes(B, H, d, nsplit))


def attn_decode_splitkv(q, k, v, nsplit: int, out=None, workspace=None, stream=None):
    """o [B, H, d] float32 from q [B, H, d] and K, V [B, H, Nkv, d]."""
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, Nkv, d = k.shape
    if q.shape != (B, H, d) or v.shape != k.shape:
        raise ValueError("q must be [B, H, d] and K, V [B, H, Nkv, d]")
    _need_out(out, (B, H, d), torch.float32, q, "out")
    if workspace is not None and workspace.device != q.device:
        raise ValueError("workspace must be on the device of q")
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H, d, nsplit)
    if workspace is None:
        workspace = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=q.device)
    _need_device(q, k, v, out, workspace)
    _check(load_library().attn_decode_splitkv(_DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Nkv, d,
                                              int(nsplit), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream(stream)))
    return out


# Bytes of the partials attn_decode_splitkv_noalloc can hold (its scratch array).
DECODE_NOALLOC_SCRATCH_BYTES = 4 << 20


def attn_decode_splitkv_noalloc(q, k, v, nsplit: int, out, stream=None):
    """attn_decode_splitkv with the partials in the library's scratch (no workspace); ``out`` must be supplied
    ([B, H, d] float32), since the point of this entry is that nothing is allocated."""
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, Nkv, d = k.shape
    if q.shape != (B, H, d) or v.shape != k.shape:
        raise ValueError("q must be [B, H, d] and K, V [B, H, Nkv, d]")
    if out is None:
        raise ValueError("out must be supplied")
    _need_out(out, (B, H, d), torch.float32, q, "out")
    _need_device(q, k, v, out)
    _check(load_library().attn_decode_splitkv_noalloc(_DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Nkv,
                                                      d, int(nsplit), _stream(stream)))
    return out


def online_softmax_rows(x, out=None, stream=None):
    """y = softmax(x, dim=-1) for a 2-D float32 tensor."""
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be a 2-D float32 tensor")
    _need_out(out, x.shape, torch.float32, x, "out")
    if out is None:
        out = torch.empty_like(x)
    rows, cols = x.shape
    _need_device(x, out)
    _check(load_library().online_softmax_rows(_ptr(x), _ptr(out), rows, cols, _stream(stream)))
    return out


def online_softmax_topk_rows(x, k: int, with_probs: bool = False, stream=None):
    """(topv [rows, k] float32, topi [rows, k] int32[, y]) of softmax(x) per row."""
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be a 2-D float32 tensor")
    rows, cols = x.shape
    topv = torch.empty((rows, k), dtype=torch.float32, device=x.device)
    topi = torch.empty((rows, k), dtype=torch.int32, device=x.device)
    y = torch.empty_like(x) if with_probs else None
    _need_device(x)
    _check(load_library().online_softmax_topk_rows(_ptr(x), _ptr(y), _ptr(topv), _ptr(topi), rows, cols, int(k),
                                                   _stream(stream)))
    return (topv, topi, y) if with_probs else (topv, topi)
