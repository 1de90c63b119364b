// Host side of the C ABI declared in include/osfa.h: argument validation
// (before any launch), dispatch to the kernel launchers, error reporting.
#include "osfa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

// OSFA_SYNC_CHECK=1 in the environment (read at every call): after a
// successful launch, wait for the stream and report a fault of the kernel
// as ATTN_ERR_HIP from the call that launched it.  A debugging aid; without
// it the library never synchronizes.
bool sync_check() {
  const char* v = std::getenv("OSFA_SYNC_CHECK");
  return v && v[0] == '1' && v[1] == '\0';
}

attn_status_t hip_status(hipError_t e, const char* what, hipStream_t stream) {
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (sync_check()) {
    const hipError_t s = hipStreamSynchronize(stream);
    if (s != hipSuccess) return fail(ATTN_ERR_HIP, "%s: kernel failed (OSFA_SYNC_CHECK): %s", what, hipGetErrorString(s));
  }
  return ATTN_OK;
}

// LSE is float32 and kv_len int32: both must be 4-byte aligned (kv_len may be NULL).
bool misaligned4(const void* a, const void* b) { return (((uintptr_t)a | (uintptr_t)b) & 3) != 0; }

constexpr long long kMaxElems = 1LL << 40;

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_last_error; }

const char* osfa_version(void) { return "osfa 0.1.0 (gfx950)"; }

attn_status_t attn_fwd(attn_dtype_t dtype, const void* Q, const void* K, const void* V, void* O, float* LSE,
                       int B, int H, int N, int d, float scale, int causal, int window, const int32_t* kv_len,
                       hipStream_t stream) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: unknown dtype %d", (int)dtype);
  if (!Q || !K || !V || !O || !LSE) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: null tensor pointer");
  if (B < 1 || H < 1 || N < 1 || d < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: sizes must be >= 1 (B=%d H=%d N=%d d=%d)", B, H, N, d);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: head dim d=%d not built (64 or 128)", d);
  if ((long long)B * H * N * d >= kMaxElems) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: B*H*N*d too large");
  if ((long long)B * H >= (1LL << 24)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: B*H too large");
  if ((long long)N * d >= (1LL << 30)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: N*d must be < 2^30 (one head)");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: scale must be finite and > 0 (got %g)", (double)scale);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: causal must be 0 or 1");
  if (window < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: window must be >= 0 (0 = no window)");
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15)
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: Q, K, V, O must be 16-byte aligned");
  if (misaligned4(LSE, kv_len)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd: LSE and kv_len must be 4-byte aligned");
  osfa::FwdArgs a{Q, K, V, O, LSE, kv_len, B, H, N, d, scale, causal, window};
  const hipError_t e = dtype == ATTN_BF16 ? osfa::launch_attn_fwd_bf16(a, stream) : osfa::launch_attn_fwd_f32(a, stream);
  return hip_status(e, "attn_fwd", stream);
}

attn_status_t attn_fwd_exp2_offload(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                    int N, int d, float scale, int causal, int window, const int32_t* kv_len,
                                    int poly_every, hipStream_t stream) {
  if (poly_every != 2 && poly_every != 4 && poly_every != 8)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_exp2_offload: poly_every=%d not built (2, 4 or 8)", poly_every);
  if (!Q || !K || !V || !O || !LSE) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: null tensor pointer");
  if (B < 1 || H < 1 || N < 1 || d < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: sizes must be >= 1 (B=%d H=%d N=%d d=%d)", B, H, N, d);
  if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_exp2_offload: head dim d=%d not built (128)", d);
  if ((long long)B * H * N * d >= kMaxElems) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: B*H*N*d too large");
  if ((long long)B * H >= (1LL << 24)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: B*H too large");
  if ((long long)N * d >= (1LL << 30))
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: N*d must be < 2^30 (one head)");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: scale must be finite and > 0 (got %g)", (double)scale);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: causal must be 0 or 1");
  if (window < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: window must be >= 0 (0 = no window)");
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15)
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: Q, K, V, O must be 16-byte aligned");
  if (misaligned4(LSE, kv_len)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_exp2_offload: LSE and kv_len must be 4-byte aligned");
  osfa::FwdArgs a{Q, K, V, O, LSE, kv_len, B, H, N, d, scale, causal, window};
  return hip_status(osfa::launch_attn_fwd_bf16_exp2_offload(a, poly_every, stream), "attn_fwd_exp2_offload", stream);
}

attn_status_t attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N,
                           int d, float scale, float q_descale, float k_descale, float v_descale, int causal,
                           int window, const int32_t* kv_len, hipStream_t stream) {
  if (!Q || !K || !V || !O || !LSE) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: null tensor pointer");
  if (B < 1 || H < 1 || N < 1 || d < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: sizes must be >= 1 (B=%d H=%d N=%d d=%d)", B, H, N, d);
  if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: head dim d=%d not built (128)", d);
  if ((long long)B * H * N * d >= kMaxElems) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: B*H*N*d too large");
  if ((long long)B * H >= (1LL << 24)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: B*H too large");
  if ((long long)N * d >= (1LL << 30)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: N*d must be < 2^30 (one head)");
  const float sc[4] = {scale, q_descale, k_descale, v_descale};
  for (float x : sc)
    if (!std::isfinite(x) || !(x > 0.0f))
      return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: scale and descales must be finite and > 0 (got %g)", (double)x);
  const float qk = q_descale * k_descale;
  if (!std::isfinite(qk) || !(qk > 0.0f) || !std::isfinite(scale * qk) || !(scale * qk > 0.0f))
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: scale * q_descale * k_descale out of float32 range");
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: causal must be 0 or 1");
  if (window < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: window must be >= 0 (0 = no window)");
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15)
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: Q, K, V, O must be 16-byte aligned");
  if (misaligned4(LSE, kv_len)) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_fp8: LSE and kv_len must be 4-byte aligned");
  osfa::FwdArgs a{Q, K, V, O, LSE, kv_len, B, H, N, d, scale, causal, window};
  return hip_status(osfa::launch_attn_fwd_fp8(a, qk, v_descale, stream), "attn_fwd_fp8", stream);
}

size_t attn_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return 2 * (size_t)B * H * N * sizeof(float);
}

// The dS tiles start at the D / LSE part rounded up to 256 bytes.
static size_t bwd_ds_offset(int B, int H, int N) { return (attn_bwd_workspace_bytes(B, H, N) + 255) / 256 * 256; }

size_t attn_bwd_stored_ds_workspace_bytes(int B, int H, int N, int causal, int window) {
  if (B < 1 || H < 1 || N < 1 || window < 0 || (causal != 0 && causal != 1)) return 0;
  const int w = window > N ? N : window;  // as the launcher clamps it
  const long long head = osfa::ds_head_bytes(N, causal, w);
  if (head >= (1LL << 31)) return 0;
  const double total = (double)B * H * (double)head;
  if (total > 9.0e18) return 0;
  return bwd_ds_offset(B, H, N) + (size_t)B * H * (size_t)head;
}

attn_status_t attn_bwd(attn_dtype_t dtype, const void* Q, const void* K, const void* V, const void* O, const void* dO,
                       const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int N, int d, float scale,
                       int causal, int window, const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: unknown dtype %d", (int)dtype);
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || !workspace)
    return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: null pointer");
  if (B < 1 || H < 1 || N < 1 || d < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: sizes must be >= 1 (B=%d H=%d N=%d d=%d)", B, H, N, d);
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: only bf16 is built");
  if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: head dim d=%d not built (128)", d);
  if ((long long)B * H * N * d >= kMaxElems) return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: B*H*N*d too large");
  if ((long long)B * H >= (1LL << 24)) return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: B*H too large");
  if ((long long)N * d >= (1LL << 30)) return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: N*d must be < 2^30 (one head)");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: scale must be finite and > 0 (got %g)", (double)scale);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: causal must be 0 or 1");
  if (window < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: window must be >= 0 (0 = no window)");
  const size_t need = attn_bwd_workspace_bytes(B, H, N);
  if (workspace_bytes < need)
    return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)dO | (uintptr_t)dQ | (uintptr_t)dK |
       (uintptr_t)dV) & 15)
    return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: Q, K, V, O, dO, dQ, dK, dV must be 16-byte aligned");
  if (((uintptr_t)LSE | (uintptr_t)workspace | (uintptr_t)kv_len) & 3)
    return fail(ATTN_ERR_INVALID_ARG, "attn_bwd: LSE, workspace and kv_len must be 4-byte aligned");
  // Room for the dS tiles: store dS once and form dQ from it.
  const size_t stored = attn_bwd_stored_ds_workspace_bytes(B, H, N, causal, window);
  void* ds = (stored != 0 && workspace_bytes >= stored) ? static_cast<char*>(workspace) + bwd_ds_offset(B, H, N) : nullptr;
  osfa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, kv_len, static_cast<float*>(workspace), ds, B, H, N, d, scale, causal,
                  window};
  return hip_status(osfa::launch_attn_bwd_bf16(a, stream), "attn_bwd", stream);
}

size_t attn_decode_splitkv_workspace_bytes(int B, int H, int d, int nsplit) {
  if (B < 1 || H < 1 || d < 1 || nsplit < 1) return 0;
  return (size_t)B * H * nsplit * (size_t)(d + 2) * sizeof(float);
}

attn_status_t attn_decode_splitkv(attn_dtype_t dtype, const void* q, const void* K, const void* V, float* o, int B,
                                  int H, int Nkv, int d, int nsplit, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: unknown dtype %d", (int)dtype);
  if (!q || !K || !V || !o || !workspace) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: null pointer");
  if (B < 1 || H < 1 || Nkv < 1 || d < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: sizes must be >= 1 (B=%d H=%d Nkv=%d d=%d)", B, H, Nkv, d);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_splitkv: d=%d not built (64 or 128)", d);
  if (nsplit < 1 || nsplit > Nkv || nsplit > 4096)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: nsplit=%d must be in [1, min(Nkv, 4096)]", nsplit);
  if ((long long)B * H * Nkv * d >= kMaxElems) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: too large");
  if ((long long)B * H * nsplit >= (1LL << 31)) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: grid too large");
  const size_t need = attn_decode_splitkv_workspace_bytes(B, H, d, nsplit);
  if (workspace_bytes < need)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (((uintptr_t)q | (uintptr_t)K | (uintptr_t)V) & 15)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: q, K, V must be 16-byte aligned");
  if (((uintptr_t)o | (uintptr_t)workspace) & 3)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv: o and workspace must be 4-byte aligned");
  osfa::DecodeArgs a{q, K, V, o, static_cast<float*>(workspace), B, H, Nkv, d, nsplit};
  const hipError_t e = dtype == ATTN_BF16 ? osfa::launch_decode_bf16(a, stream) : osfa::launch_decode_f32(a, stream);
  return hip_status(e, "attn_decode_splitkv", stream);
}

attn_status_t attn_decode_splitkv_noalloc(attn_dtype_t dtype, const void* q, const void* K, const void* V, float* o,
                                          int B, int H, int Nkv, int d, int nsplit, hipStream_t stream) {
  static_assert(osfa::kDecodeScratchBytes == OSFA_DECODE_NOALLOC_SCRATCH_BYTES, "header and library agree");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: unknown dtype %d", (int)dtype);
  if (!q || !K || !V || !o) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: null pointer");
  if (B < 1 || H < 1 || Nkv < 1 || d < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: sizes must be >= 1 (B=%d H=%d Nkv=%d d=%d)", B, H,
                Nkv, d);
  if (d != 64 && d != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_splitkv_noalloc: d=%d not built (64 or 128)", d);
  if (nsplit < 1 || nsplit > Nkv || nsplit > 4096)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: nsplit=%d must be in [1, min(Nkv, 4096)]", nsplit);
  if ((long long)B * H * Nkv * d >= kMaxElems) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: too large");
  if ((long long)B * H * nsplit >= (1LL << 31))
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: grid too large");
  const size_t need = attn_decode_splitkv_workspace_bytes(B, H, d, nsplit);
  if (need > osfa::kDecodeScratchBytes)
    return fail(ATTN_ERR_INVALID_ARG,
                "attn_decode_splitkv_noalloc: partials need %zu bytes, more than the %zu-byte scratch (B*H*nsplit*(d+2)*4)",
                need, osfa::kDecodeScratchBytes);
  if (((uintptr_t)q | (uintptr_t)K | (uintptr_t)V) & 15)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: q, K, V must be 16-byte aligned");
  if ((uintptr_t)o & 3) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_splitkv_noalloc: o must be 4-byte aligned");
  osfa::DecodeArgs a{q, K, V, o, nullptr, B, H, Nkv, d, nsplit};
  return hip_status(osfa::launch_decode_noalloc(a, dtype == ATTN_BF16, stream), "attn_decode_splitkv_noalloc", stream);
}

attn_status_t online_softmax_rows(const float* x, float* y, int rows, int cols, hipStream_t stream) {
  if (!x || !y) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_rows: null pointer");
  if (rows < 1 || cols < 1) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_rows: rows=%d cols=%d must be >= 1", rows, cols);
  if (cols > (1 << 28)) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_rows: cols=%d > 2^28", cols);
  if (((uintptr_t)x | (uintptr_t)y) & 3) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_rows: x, y must be 4-byte aligned");
  if (x != y) {
    const char* xb = reinterpret_cast<const char*>(x);
    const char* yb = reinterpret_cast<const char*>(y);
    const size_t bytes = (size_t)rows * cols * sizeof(float);
    if (xb < yb + bytes && yb < xb + bytes)
      return fail(ATTN_ERR_INVALID_ARG, "online_softmax_rows: x and y overlap partially");
  }
  return hip_status(osfa::launch_softmax_rows(x, y, rows, cols, stream), "online_softmax_rows", stream);
}

attn_status_t online_softmax_topk_rows(const float* x, float* y, float* topv, int32_t* topi, int rows, int cols, int k,
                                       hipStream_t stream) {
  if (!x || !topv || !topi) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_topk_rows: null pointer");
  if (rows < 1 || cols < 1) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_topk_rows: rows=%d cols=%d must be >= 1", rows, cols);
  if (cols > (1 << 28)) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_topk_rows: cols=%d > 2^28", cols);
  if (k < 1 || k > cols) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_topk_rows: k=%d must be in [1, cols]", k);
  if (k > 16) return fail(ATTN_ERR_UNSUPPORTED, "online_softmax_topk_rows: k=%d > 16 not built", k);
  if (((uintptr_t)x | (uintptr_t)topv | (uintptr_t)topi | (uintptr_t)y) & 3)
    return fail(ATTN_ERR_INVALID_ARG, "online_softmax_topk_rows: pointers must be 4-byte aligned");
  if (y == x) return fail(ATTN_ERR_INVALID_ARG, "online_softmax_topk_rows: y must not alias x");
  return hip_status(osfa::launch_softmax_topk(x, y, topv, topi, rows, cols, k, stream), "online_softmax_topk_rows", stream);
}

}  // extern "C"
