"""online_softmax_fa2_amd -- exact softmax attention by the online-softmax
recurrence, hand-written in HIP for AMD MI355X (gfx950).

The compute path is the C-ABI library ``_lib/libosfa.so`` (sources in
``csrc/``, declarations in ``include/osfa.h``); the functions exported here
only marshal PyTorch tensors and streams into it.  Importing this package
does not load the library; the first call does, and raises if it is not
built.
"""
from ._binding import (OsfaError, attn_bwd, attn_decode_splitkv, attn_decode_splitkv_noalloc, attn_fwd, attn_fwd_exp2_offload, attn_fwd_fp8,  # noqa: F401
                       bwd_stored_ds_workspace_bytes, bwd_workspace_bytes, decode_workspace_bytes, load_library,
                       online_softmax_rows, online_softmax_topk_rows)

__all__ = ["attn_fwd", "attn_fwd_exp2_offload", "attn_fwd_fp8", "attn_bwd", "bwd_workspace_bytes",
           "bwd_stored_ds_workspace_bytes", "attn_decode_splitkv", "attn_decode_splitkv_noalloc", "decode_workspace_bytes",
           "online_softmax_rows", "online_softmax_topk_rows", "load_library", "OsfaError"]
