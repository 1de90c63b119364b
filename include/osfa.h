/*
 * osfa.h -- C ABI of the online-softmax exact-attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * Every entry point is extern "C", thread-safe (no shared mutable state
 * apart from the per-thread error text), never allocates device memory,
 * never synchronizes, and enqueues its kernels asynchronously on `stream`
 * (0 means the null stream).  All tensor pointers are device pointers owned
 * by the caller; the library keeps none of them after returning.
 *
 * Errors: the return code is the only channel.  All argument checks run on
 * the host BEFORE anything is launched, so on ATTN_ERR_INVALID_ARG or
 * ATTN_ERR_UNSUPPORTED nothing is enqueued and no output is written.
 * ATTN_ERR_HIP reports a failed launch (hipGetLastError after the launch);
 * faults raised while a kernel runs surface at the caller's next
 * synchronization.  attn_last_error() returns a description of the last
 * non-OK status on the calling thread.
 *
 * Debugging: with OSFA_SYNC_CHECK=1 in the environment (read at every
 * call), each entry point waits for `stream` after a successful launch and
 * reports a fault of its own kernels as ATTN_ERR_HIP.  Without it nothing
 * synchronizes.
 *
 * Alignment: LSE and kv_len (where present) must be 4-byte aligned; tensor
 * arguments as stated per entry point.
 *
 * Inputs are assumed finite; NaN or Inf inputs propagate.  Outputs must not
 * alias inputs, except x == y in online_softmax_rows.
 *
 * Pages cited (by title): "Derive online softmax, prove it is exact"; "Online
 * softmax for a whole query tile, matrix form"; "Online softmax" (the article
 * on Milakov and Gimelshein's online normalizer).
 */
#ifndef OSFA_H
#define OSFA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* a null pointer, a size < 1, a bad mask or scale */
  ATTN_ERR_UNSUPPORTED = 2, /* valid in principle but not built: d not in {64, 128}, k > 16 */
  ATTN_ERR_HIP = 3          /* the HIP runtime refused a launch (no device, bad stream, ...) */
} attn_status_t;

typedef enum {
  ATTN_F32 = 0,  /* IEEE float32 elements */
  ATTN_BF16 = 1  /* bfloat16 elements (the upper 16 bits of a float32) */
} attn_dtype_t;

/*
 * attn_fwd -- fused attention forward pass with per-row log-sum-exp.
 *
 * Computes, for every batch b, head h and query i,
 *   O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) V[b,h,j,:]
 * over the keys j visible to i, by the query-tile online-softmax
 * recurrence: each tile of queries keeps a running row maximum m, a running
 * normalizer l and an unnormalized accumulator A, rescales all three by
 * alpha = exp(m_old - m_new) as each key block arrives, and divides A by l
 * once after the last block (page "Online softmax for a whole query tile,
 * matrix form", "A strong answer" and its TL;DR; page "Derive online
 * softmax, prove it is exact", "A strong answer").  The N x N score matrix
 * is never written to memory.
 *
 * Layout: Q, K, V, O are [B, H, N, d] contiguous, d fastest, elements of
 * `dtype` (O has the same dtype as the inputs; bf16 O is rounded to nearest
 * even).  LSE is [B, H, N] float32: LSE = ln sum_j exp(scale * q_i . k_j)
 * over visible j, in natural-log units of the scaled score (page "Derive
 * online softmax, prove it is exact", "What interviewers probe next").
 *
 * Visibility of key j to query i (page "Online softmax for a whole query
 * tile, matrix form", causal / window / padding masks):
 *   j < kv_len[b]  and  (causal == 0 or j <= i)  and  (window <= 0 or |i - j| < window)
 * kv_len: NULL (every key visible up to N) or a DEVICE pointer to B int32
 * values; values are clamped to [0, N] on the device.  A query with no
 * visible key gets O = 0 and LSE = -inf, never NaN (the fully-masked-row
 * guard of the same page).
 *
 * scale must be finite and > 0 (typically 1/sqrt(d)).  Supported: d in
 * {64, 128} for both dtypes; B, H, N >= 1; B * H * N * d < 2^40; N * d < 2^30.
 */
attn_status_t attn_fwd(attn_dtype_t dtype, const void* Q, const void* K, const void* V,
                       void* O, float* LSE, int B, int H, int N, int d, float scale,
                       int causal, int window, const int32_t* kv_len, hipStream_t stream);

/*
 * attn_fwd_exp2_offload -- attn_fwd for bf16, d = 128, with part of the
 * exponentials computed on the FMA pipes: FlashAttention-4's answer to
 * exponential units that lag the matrix cores (page "Derive online softmax,
 * prove it is exact", "What interviewers probe next").  Of every poly_every
 * consecutive pairs of exponentials a lane forms for a key block, the last
 * pair is 2^n * p(f) (x = n + f, |f| <= 1/2, p a cubic with relative error
 * <= 7.5e-5, 2^n by v_ldexp_f32) instead of v_exp_f32; the rest is attn_fwd
 * exactly.  Results agree with attn_fwd to within that error, far below the
 * bf16 rounding of P and O.  On gfx950 the polynomial costs eight VALU
 * instructions against one transcendental, so this variant is slower than
 * attn_fwd there; it exists to measure the trade.
 *
 * Arguments, layout, masks and errors: as attn_fwd with dtype = bf16.
 * poly_every: 2, 4 or 8 (one exponential in 2, 4 or 8 on the FMA pipes;
 * others -> ATTN_ERR_UNSUPPORTED).  Supported: d = 128 (others ->
 * ATTN_ERR_UNSUPPORTED); Q, K, V, O 16-byte aligned.
 */
attn_status_t attn_fwd_exp2_offload(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                    int N, int d, float scale, int causal, int window, const int32_t* kv_len,
                                    int poly_every, hipStream_t stream);

/*
 * attn_fwd_fp8 -- attn_fwd with FP8 inputs: Q, K, V are OCP e4m3 (e4m3fn)
 * codes, one byte per element, and each tensor has one float32 descale, so
 * that the value of an element is code x descale.  Computes the same O and
 * LSE as attn_fwd for the dequantized Q, K, V (same masks, guard, deferred
 * division and LSE; pages as cited there), with both products on the FP8
 * matrix core and float32 statistics: the FP8 step the pages name for FA3
 * (page "Derive online softmax, prove it is exact", "What interviewers probe
 * next"; article "Online softmax", "Trade-offs and edge cases").
 *
 * P is rounded to e4m3 before P V, in a per-(query, 64-key block) power-of-
 * two frame that maps the block's largest P into (128, 256]; O divides by
 * the sum of those rounded P, LSE uses the float32 sum.  The result differs
 * from the exact attention of the dequantized inputs by the rounding of P
 * (relative 2^-4 per element) and the matrix core's accumulation (about
 * 2^-15 of the sum of |terms| per instruction).
 *
 * Layout: Q, K, V [B, H, N, d] bytes, d fastest; O [B, H, N, d] bf16 (round
 * to nearest even); LSE [B, H, N] float32, natural log, as attn_fwd.  Codes
 * 0x7F and 0xFF (NaN) are out of contract.  q_descale, k_descale,
 * v_descale: finite and > 0.  Supported: d = 128 (others ->
 * ATTN_ERR_UNSUPPORTED); B, H, N >= 1; B * H * N * d < 2^40; N * d < 2^30;
 * Q, K, V, O 16-byte aligned.
 */
attn_status_t attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N,
                           int d, float scale, float q_descale, float k_descale, float v_descale, int causal,
                           int window, const int32_t* kv_len, hipStream_t stream);

/*
 * attn_bwd_workspace_bytes -- bytes of device workspace that attn_bwd needs:
 * 2 * B * H * N * 4 (per query, D = rowsum(dO * O) and LSE in log2 units,
 * float32).  Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/*
 * attn_bwd_stored_ds_workspace_bytes -- bytes of workspace with which
 * attn_bwd also stores dS (bf16, in tiles of 32 keys x 32 queries over the
 * key blocks the mask lets each query block see) and forms dQ = scale dS K
 * from the stored tiles instead of recomputing S and dP: attn_bwd_workspace_
 * bytes(B, H, N) rounded up to 256, plus B * H * ceil(N / 32) * S * 2048,
 * where S is the number of 32-key blocks one 32-query block can see (all of
 * them without a window; about window / 32 + 1 causal, window / 16 + 2
 * otherwise; `window` as attn_bwd takes it).  Returns 0 for invalid sizes
 * and where one head's tiles would exceed 2^31 bytes (attn_bwd then always
 * recomputes).
 */
size_t attn_bwd_stored_ds_workspace_bytes(int B, int H, int N, int causal, int window);

/*
 * attn_bwd -- backward pass of attn_fwd: the gradients dQ, dK, dV of the
 * forward output O for an incoming gradient dO.
 *
 * The forward's per-row log-sum-exp is all that is kept: P is recomputed
 * block by block from Q, K and LSE as the normalized P = exp(scale Q K^T -
 * LSE), with no running maximum (page "Derive online softmax, prove it is
 * exact", "What interviewers probe next"; page "Online softmax for a whole
 * query tile, matrix form", "What interviewers probe next").  With
 * D_i = sum_d dO_id O_id,
 *   dV = P^T dO,   dS = P * (dO V^T - D),   dQ = scale dS K,   dK = scale dS^T Q,
 * over the same visible pairs as attn_fwd (same causal / window / kv_len
 * arguments and the same reading of them).  A query that sees no key (LSE =
 * -inf) contributes nothing.
 *
 * Layout: Q, K, V, O, dO, dQ, dK, dV are [B, H, N, d] bf16, d fastest; LSE
 * is [B, H, N] float32 as written by attn_fwd for the same Q, K, V.  dQ, dK,
 * dV are fully overwritten (rounded to nearest even).  workspace:
 * caller-owned device memory of at least attn_bwd_workspace_bytes(B, H, N)
 * bytes, 4-byte aligned; its contents on return are unspecified.  With at
 * least attn_bwd_stored_ds_workspace_bytes(B, H, N, causal, window) bytes
 * (and that function non-zero), dS is stored in the workspace once and dQ
 * is a product with it; with less, dQ recomputes S and dP.  The two ways
 * compute dS identically.
 * Supported: dtype ATTN_BF16 and d = 128 (others -> ATTN_ERR_UNSUPPORTED);
 * B, H, N >= 1; B * H * N * d < 2^40; N * d < 2^30.
 */
attn_status_t attn_bwd(attn_dtype_t dtype, const void* Q, const void* K, const void* V, const void* O,
                       const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int N,
                       int d, float scale, int causal, int window, const int32_t* kv_len, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_splitkv_workspace_bytes -- bytes of device workspace that
 * attn_decode_splitkv needs: B * H * nsplit * (d + 2) * 4 (one partial
 * (m, l, a[d]) triple per split, float32).  Returns 0 for invalid sizes.
 */
size_t attn_decode_splitkv_workspace_bytes(int B, int H, int d, int nsplit);

/*
 * attn_decode_splitkv -- single-query attention per (b, h) with the keys
 * split across workgroups (split-KV / Flash-Decoding).
 *
 * Split c covers keys [c*L, min((c+1)*L, Nkv)) with L = ceil(Nkv / nsplit);
 * each split runs the online-softmax recurrence over its keys and leaves a
 * partial (m_c, l_c, a_c); a second kernel merges the partials with the
 * associative rescale rule M = max m_c, o = sum_c e^{m_c-M} a_c / sum_c
 * e^{m_c-M} l_c, an empty split contributing nothing (page "Derive online
 * softmax, prove it is exact", the batch-1 decoding follow-up; article
 * "Online softmax", Step 4 and the Flash-Decoding note).  Non-causal,
 * unmasked, scale = 1/sqrt(d) rounded to float32.
 *
 * Layout: q [B, H, d], K and V [B, H, Nkv, d] of `dtype`, d fastest; o
 * [B, H, d] float32.  workspace: caller-owned device memory of at least
 * attn_decode_splitkv_workspace_bytes(B, H, d, nsplit) bytes; its contents
 * on return are unspecified.  Supported: d in {64, 128}; 1 <= nsplit <=
 * Nkv; nsplit <= 4096.
 */
attn_status_t attn_decode_splitkv(attn_dtype_t dtype, const void* q, const void* K, const void* V,
                                  float* o, int B, int H, int Nkv, int d, int nsplit,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_splitkv_noalloc -- attn_decode_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and the same
 * result, with the split partials kept in a scratch array inside the
 * library instead of a caller-supplied workspace.
 *
 * The scratch array is a device global of OSFA_DECODE_NOALLOC_SCRATCH_BYTES
 * (4 MiB): each GPU the library runs on holds its own copy until the
 * process ends.  The partials take B * H * nsplit * (d + 2) * 4 bytes
 * (attn_decode_splitkv_workspace_bytes); larger requests return
 * ATTN_ERR_INVALID_ARG.  The call allocates nothing (no hipMalloc, no
 * hipFree); its first call on a device looks up that device's copy.
 * Every call on one GPU shares that copy: calls whose kernels overlap on
 * the same GPU (different streams, or another thread) race and give
 * undefined results; calls ordered on one stream are safe.  The partials
 * are fully rewritten by each call before they are read.
 *
 * Arguments, layout, scale and errors otherwise as attn_decode_splitkv.
 */
#define OSFA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
attn_status_t attn_decode_splitkv_noalloc(attn_dtype_t dtype, const void* q, const void* K, const void* V,
                                          float* o, int B, int H, int Nkv, int d, int nsplit, hipStream_t stream);

/*
 * online_softmax_rows -- y[r, :] = softmax(x[r, :]) for every row, float32.
 *
 * Pass 1 runs the online normalizer: a running pair (m, d), the sum d
 * rescaled by exp(m_old - m_new) whenever the maximum grows, partial pairs
 * of lanes and waves combined by the associative merge; pass 2 writes
 * exp(x - m) / d (article "Online softmax", Steps 2-4).  Rows of up to
 * 8192 columns stay in registers between the passes (one read and one
 * write of each element); longer rows re-read x in pass 2.
 *
 * Layout: x and y [rows, cols] row-major float32; x == y is allowed.
 * Supported: rows >= 1, 1 <= cols <= 2^28.
 */
attn_status_t online_softmax_rows(const float* x, float* y, int rows, int cols, hipStream_t stream);

/*
 * online_softmax_topk_rows -- softmax fused with a top-k selection, one
 * read of x.
 *
 * In a single pass over each row, keeps the online normalizer (m, d) and
 * the k largest elements seen so far, then writes the k probabilities
 * exp(x - m) / d and their column indices (article "Online softmax", Step
 * 3, the fused top-k variant).  Order: descending probability, ties
 * broken by the lower column index.
 *
 * Layout: x [rows, cols] float32 row-major; topv [rows, k] float32; topi
 * [rows, k] int32; y: NULL, or [rows, cols] float32 receiving the full
 * softmax (this costs a second read of x).  Supported: 1 <= k <= 16, k <=
 * cols, rows >= 1, cols <= 2^28.
 */
attn_status_t online_softmax_topk_rows(const float* x, float* y, float* topv, int32_t* topi,
                                       int rows, int cols, int k, hipStream_t stream);

/* Description of the last non-OK status on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Library version string. */
const char* osfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSFA_H */
