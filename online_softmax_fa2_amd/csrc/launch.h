// Internal interface between the C-ABI layer (api.cpp) and the kernel
// translation units.  Arguments reaching a launcher have been validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace osfa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_len;  // device [B] or nullptr
  int B, H, N, d;
  float scale;
  int causal, window;
};

// Each returns the hipError_t of its launch(es).
hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream);
// bf16, d = 128: one exponential pair in every poly_every (2, 4 or 8) on the FMA pipes.
hipError_t launch_attn_fwd_bf16_exp2_offload(const FwdArgs& a, int poly_every, hipStream_t stream);
// e4m3 Q, K, V (d = 128), bf16 O: scores take scale * qk_descale, O takes v_descale.
hipError_t launch_attn_fwd_fp8(const FwdArgs& a, float qk_descale, float v_descale, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* kv_len;  // device [B] or nullptr
  float* ws;              // [2, B, H, N]: D and LSE in log2 units
  void* ds;               // stored-dS tiles (bf16), or nullptr: dQ recomputes S and dP
  int B, H, N, d;
  float scale;
  int causal, window;
};
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream);

// Stored dS of the backward: bf16 tiles of 32 keys x 32 queries (key-major,
// 2 KB), per head ceil(N / 32) query blocks of ds_span() tile slots; the tile
// of query block qb and key block kb sits in slot kb - ds_first(qb).  Every
// key block some query of block qb can see lies in that range.  `window` is
// the window after clamping to N (0 = none).
constexpr int kDsTile = 32;
constexpr long long ds_span(int N, int causal, int window) {
  const long long nb = (N + kDsTile - 1) / kDsTile;
  if (window <= 0) return nb;
  // causal: key blocks from that of 32 qb - W + 1 to qb; otherwise also up
  // to that of 32 qb + 31 + W - 1.
  const long long span = causal ? 1 + (window - 1 + kDsTile - 1) / kDsTile : (2LL * window + 29) / kDsTile + 2;
  return span < nb ? span : nb;
}
constexpr int ds_first(int qb, int window) {
  const int lo = kDsTile * qb - window + 1;
  return (window > 0 && lo > 0) ? lo / kDsTile : 0;
}
// Bytes of one head's tiles (the kernels address them with 32-bit offsets).
constexpr long long ds_head_bytes(int N, int causal, int window) {
  return (long long)((N + kDsTile - 1) / kDsTile) * ds_span(N, causal, window) * kDsTile * kDsTile * 2;
}

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* ws;  // [B, H, nsplit, d + 2]
  int B, H, Nkv, d, nsplit;
};
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);
// The same kernels with the partials in the library's per-device scratch
// array (a.ws is ignored); the caller has checked that they fit in
// kDecodeScratchBytes.
constexpr size_t kDecodeScratchBytes = size_t(4) << 20;
hipError_t launch_decode_noalloc(const DecodeArgs& a, bool bf16, hipStream_t stream);

hipError_t launch_softmax_rows(const float* x, float* y, int rows, int cols, hipStream_t stream);
hipError_t launch_softmax_topk(const float* x, float* y, float* topv, int32_t* topi, int rows,
                               int cols, int k, hipStream_t stream);

}  // namespace osfa
