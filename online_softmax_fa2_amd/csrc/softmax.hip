// Row-wise online softmax and softmax fused with top-k, float32, gfx950.
//
// Method (article "Online softmax"): pass 1 computes the pair (m, d), the
// row maximum and the sum of exp(x - m), keeping a running maximum and
// rescaling the running sum by exp(m_old - m_new) when it grows (Step 2);
// partial pairs of lanes and waves are combined by the associative merge
// (Step 4); pass 2 writes exp(x - m) / d (Step 3).  The fused variant keeps
// a top-k list next to (m, d) during the single pass and outputs only the k
// probabilities and their column indices (Step 3, fusion with top-k).
//
// gfx950 mapping: one 256-thread workgroup per row, or, when at least 4096
// rows of at most 4096 aligned floats fill the chip, one wave per row (per
// two rows above 2048 floats).  Each lane folds its elements into its own
// (m, d) a chunk at a time (chunk maximum, one rescale of d, one exp2 per
// element with log2(e) folded into an FMA), then the 64 lanes of a wave
// merge by butterfly exchanges and the waves of a workgroup through LDS.
// Rows of up to 8192 columns are held in registers between the passes, so
// HBM sees one read and one write per element; longer rows re-read x.
// Accesses are float4 (16 B per lane, fully coalesced) when the row length
// is a multiple of 4 and the pointers are 16-byte aligned, else scalar.
#include "device_common.h"
#include "launch.h"

namespace osfa {
namespace {

constexpr int kSmThreads = 256;
constexpr int kSmWaves = kSmThreads / 64;
// Rows of at most 4096 aligned floats, at least 16 per CU: one wave per row,
// or per two rows of more than 2048 floats (else a workgroup per row).
constexpr bool kSoftmaxWavePerRow = true;

// Element access, 4-wide when the row allows it.  ld/st go through the
// caches; ld_nt/st_nt mark data touched exactly once (non-temporal) so it does
// not displace data that is reused.
template <int W>
__device__ __forceinline__ void ld(const float* p, float* v) {
  if constexpr (W == 4) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p);
    v[0] = t[0];
    v[1] = t[1];
    v[2] = t[2];
    v[3] = t[3];
  } else {
    v[0] = *p;
  }
}
template <int W>
__device__ __forceinline__ void ld_nt(const float* p, float* v) {
  if constexpr (W == 4) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    v[0] = t[0];
    v[1] = t[1];
    v[2] = t[2];
    v[3] = t[3];
  } else {
    v[0] = __builtin_nontemporal_load(p);
  }
}
template <int W>
__device__ __forceinline__ void st_nt(float* p, const float* v) {
  if constexpr (W == 4) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
  } else {
    __builtin_nontemporal_store(v[0], p);
  }
}

// Fold a chunk of n values (maximum mx, raw units) into the running pair.
__device__ __forceinline__ void fold_chunk(MD& r, float mx, const float* vals, int n) {
  const float m_new = fmaxf(r.m, mx * kLog2e);
  const float m_ref = (m_new == kNegInf) ? 0.0f : m_new;
  float s = r.d * fast_exp2(r.m - m_ref);
  for (int i = 0; i < n; ++i) s += fast_exp2(fmaf(vals[i], kLog2e, -m_ref));
  r.m = m_new;
  r.d = s;
}

// Merge the pairs of all lanes of the workgroup; every thread gets the result.
__device__ __forceinline__ MD block_md(MD v) {
  __shared__ MD sh[kSmWaves];
  v = wave_md_merge(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  MD r = sh[0];
#pragma unroll
  for (int i = 1; i < kSmWaves; ++i) r = md_merge(r, sh[i]);
  return r;
}

// Register-resident rows: thread t owns accesses t + 256 i, i < VPT.
template <int W, int VPT>
__global__ __launch_bounds__(kSmThreads) void softmax_rows_reg_kernel(const float* x, float* y, int cols) {
  const int row = blockIdx.x;
  const float* xr = x + (size_t)row * cols;
  float* yr = y + (size_t)row * cols;
  const int nacc = cols / W;
  const int t = threadIdx.x;
  float v[VPT][W];
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int a = t + kSmThreads * i;
    if (a < nacc) {
      ld_nt<W>(xr + (size_t)a * W, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < W; ++e) v[i][e] = kNegInf;
    }
#pragma unroll
    for (int e = 0; e < W; ++e) mx = fmaxf(mx, v[i][e]);
  }
  MD r{kNegInf, 0.0f};
  fold_chunk(r, mx, &v[0][0], VPT * W);  // -inf slots contribute exp2(-inf) = 0
  r = block_md(r);
  const float inv = 1.0f / r.d;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int a = t + kSmThreads * i;
    if (a < nacc) {
      float o[W];
#pragma unroll
      for (int e = 0; e < W; ++e) o[e] = fast_exp2(fmaf(v[i][e], kLog2e, -r.m)) * inv;
      st_nt<W>(yr + (size_t)a * W, o);
    }
  }
}

// Rows of up to 64 x VPT 4-float accesses, one wave per row (or per R rows):
// lane l owns accesses l + 64 i, the pair is merged across the wave only (no
// LDS, no barrier), and a launch over a few thousand rows has every row's
// loads in flight at once instead of a workgroup per row in two rounds.
// With R = 2 a wave takes rows g and g + ceil(rows / 2) and issues the loads
// of both before it reduces the first, so the first row's stores overlap the
// second row's loads.
template <int VPT, int R>
__global__ __launch_bounds__(kSmThreads) void softmax_rows_wave_kernel(const float* x, float* y, int rows, int cols) {
  const int g = blockIdx.x * kSmWaves + (threadIdx.x >> 6);
  const int per = (rows + R - 1) / R;  // rows per slot s: row g + per s
  if (g >= per) return;
  const int lane = threadIdx.x & 63;
  const int nacc = cols / 4;
  float v[R][VPT][4];
#pragma unroll
  for (int s = 0; s < R; ++s) {
    // A slot past the last row loads row g again and is not used.
    const int row = g + per * s < rows ? g + per * s : g;
    const float* xr = x + (size_t)row * cols;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int a = lane + 64 * i;
      ld_nt<4>(xr + (size_t)(a < nacc ? a : 0) * 4, v[s][i]);
    }
  }
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const int row = g + per * s;
    if (row >= rows) break;  // wave-uniform
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const bool ok = lane + 64 * i < nacc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[s][i][e] = ok ? v[s][i][e] : kNegInf;
        mx = fmaxf(mx, v[s][i][e]);
      }
    }
    MD r{kNegInf, 0.0f};
    fold_chunk(r, mx, &v[s][0][0], VPT * 4);  // -inf slots contribute exp2(-inf) = 0
    r = wave_md_merge(r);
    const float inv = 1.0f / r.d;
    float* yr = y + (size_t)row * cols;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int a = lane + 64 * i;
      if (a < nacc) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fast_exp2(fmaf(v[s][i][e], kLog2e, -r.m)) * inv;
        st_nt<4>(yr + (size_t)a * 4, o);
      }
    }
  }
}

// Any row length: pass 1 streams x into the pair, pass 2 re-reads x.
template <int W>
__device__ __forceinline__ MD stream_md(const float* xr, int nacc) {
  constexpr int U = 4;
  MD r{kNegInf, 0.0f};
  for (int base = 0; base < nacc; base += kSmThreads * U) {
    float v[U][W];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int a = base + threadIdx.x + kSmThreads * u;
      if (a < nacc) {
        ld<W>(xr + (size_t)a * W, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < W; ++e) v[u][e] = kNegInf;
      }
#pragma unroll
      for (int e = 0; e < W; ++e) mx = fmaxf(mx, v[u][e]);
    }
    fold_chunk(r, mx, &v[0][0], U * W);
  }
  return r;
}

template <int W>
__device__ __forceinline__ void stream_write(const float* xr, float* yr, int nacc, MD r) {
  const float inv = 1.0f / r.d;
  for (int a = threadIdx.x; a < nacc; a += kSmThreads) {
    float v[W];
    ld_nt<W>(xr + (size_t)a * W, v);
#pragma unroll
    for (int e = 0; e < W; ++e) v[e] = fast_exp2(fmaf(v[e], kLog2e, -r.m)) * inv;
    st_nt<W>(yr + (size_t)a * W, v);
  }
}

template <int W>
__global__ __launch_bounds__(kSmThreads) void softmax_rows_stream_kernel(const float* x, float* y, int cols) {
  const int row = blockIdx.x;
  const float* xr = x + (size_t)row * cols;
  float* yr = y + (size_t)row * cols;
  const int nacc = cols / W;
  MD r = block_md(stream_md<W>(xr, nacc));
  stream_write<W>(xr, yr, nacc, r);
}

// ---------------------------------------------------------------------------
// Softmax fused with top-k.
//
// Each wave keeps its current top-k candidates in lanes 0..k-1 (lane i holds
// the i-th best; order: larger x first, lower column index on equal x) and a
// wave-uniform threshold (Tx, Ti): an element can only enter the list if it
// beats the threshold.  The threshold starts as the k-th largest of the 256
// lanes' maxima over the workgroup's first chunk (a lower bound of the row's
// k-th value: those k lane maxima are k distinct elements), so even the
// first chunk offers only a handful of candidates; later it is the largest
// of the wave's k-th entry and the other waves' published ones (a wave's own
// bound alone measured slower: more candidates).  Candidates are inserted
// one at a time (readlane to broadcast, a one-lane DPP shift of the list).
// At the end the 4 waves'
// lists are ranked in LDS and the k best are written with their
// probabilities exp(x - m) / d.
// ---------------------------------------------------------------------------

// (Bitwise operators: no short-circuit branches in per-lane uses.)
__device__ __forceinline__ bool better(float xa, int ia, float xb, int ib) {
  return (xa > xb) | ((xa == xb) & (ia < ib));
}
// Float order as signed-int order (for LDS integer max), and back.
__device__ __forceinline__ int ord_f(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float unord_f(int b) { return __builtin_bit_cast(float, b >= 0 ? b : b ^ 0x7fffffff); }

// WITH_Y: the full output y is written too (a second pass re-reads x, so the
// first pass keeps x in the caches); without it x is read once, non-temporal.
// (Two instantiations: with a run-time test the compiler merges the two
// loads into one and drops the non-temporal hint.)
// A chunk is U = 2 accesses per thread (8 KB for the workgroup in float4):
// two chunks in flight per workgroup measured faster than 16 KB chunks (less
// work between a chunk's arrival and the next load) and than three chunks
// in flight.
template <int W, bool WITH_Y>
__global__ __launch_bounds__(kSmThreads) void softmax_topk_kernel(const float* x, float* y, float* topv,
                                                                   int32_t* topi, int cols, int k) {
  constexpr int U = 2;
  constexpr int STEP = kSmThreads * U;
  const int row = blockIdx.x;
  const float* xr = x + (size_t)row * cols;
  const int nacc = cols / W;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;

  float lx = kNegInf;  // this lane's list entry (lanes < k)
  int li = 0x7fffffff;
  float Tx = kNegInf;  // wave-uniform threshold
  int Ti = 0x7fffffff;
  MD r{kNegInf, 0.0f};
  // The largest of the 4 waves' thresholds, as an order-preserving int (any
  // wave's k-th entry bounds the row's k-th value from below, so elements
  // under it are skipped by every wave).  Read and raised without a barrier:
  // a stale value is still a valid bound.
  __shared__ int t_shared;
  if (threadIdx.x == 0) t_shared = ord_f(kNegInf);
  __syncthreads();

  // Two register buffers used alternately (the loop is unrolled by two so no
  // buffer is copied): the loads of the next chunk are in flight while the
  // current one is folded and scanned.  Loads are unconditional (slots past
  // the row read its first element) and invalid slots become -inf when the
  // chunk is used, so the load counter can be waited on precisely.
  float va[U][W], vb[U][W];
  auto load_chunk = [&](int base, float (&dst)[U][W]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int a = base + threadIdx.x + kSmThreads * u;
      const float* src = xr + (size_t)(a < nacc ? a : 0) * W;
      if constexpr (WITH_Y)
        ld<W>(src, dst[u]);
      else
        ld_nt<W>(src, dst[u]);
    }
  };

  // Per-wave candidate queue, room for every slot of a chunk (it cannot
  // overflow); a wave only touches its own row of it, so the LDS writes of
  // the lanes and the reads of the drain need no barrier, only the wave's
  // own ordering of LDS operations.
  constexpr int kQueue = 64 * U * W;
  __shared__ float lm_s[kSmThreads];  // lane maxima of the first chunk
  __shared__ float qv_s[kSmWaves][kQueue];
  __shared__ int qi_s[kSmWaves][kQueue];
  // The candidate and the threshold are wave-uniform: they are taken through
  // readfirstlane so that the compiler keeps them in scalar registers and
  // branches on them without exec-mask bookkeeping, and the next
  // candidate's LDS read is issued before the current one is inserted.
  auto uni = [](float f) { return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, f))); };
  auto drain = [&](int n) {
    float nx = n > 0 ? qv_s[w][0] : 0.0f;
    int ni = n > 0 ? qi_s[w][0] : 0;
    for (int q = 0; q < n; ++q) {
      const float cx = uni(nx);
      const int ci = __builtin_amdgcn_readfirstlane(ni);
      if (q + 1 < n) {
        nx = qv_s[w][q + 1];
        ni = qi_s[w][q + 1];
      }
      if (!better(cx, ci, Tx, Ti) && !(cx == Tx && Ti == 0x7fffffff)) continue;  // wave-uniform
      // Insert: lanes whose entry is worse than the candidate take the
      // previous lane's entry, or the candidate if the previous is better.
      const bool mine = better(cx, ci, lx, li);
      const float px = dpp_f<0x111>(kNegInf, lx);  // lane i - 1 (row 0 holds the list)
      const int pi = dpp_i<0x111>(0x7fffffff, li);
      const bool prev_better = (lane > 0) & better(px, pi, cx, ci);
      const bool take = mine & (lane < 16);
      const bool use_c = lane == 0 || prev_better;
      const float ex = use_c ? cx : px;
      const int ei = use_c ? ci : pi;
      lx = take ? ex : lx;
      li = take ? ei : li;
      const float kx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lx), k - 1));
      const int ki = __builtin_amdgcn_readlane(li, k - 1);
      if (better(kx, ki, Tx, Ti) || (kx == Tx && Ti == 0x7fffffff && ki != 0x7fffffff)) {
        Tx = uni(kx);
        Ti = __builtin_amdgcn_readfirstlane(ki);
      }
    }
  };

  auto process = [&](int base, float (&v)[U][W]) {
    if (base + STEP > nacc) {  // the row's last chunk (wave-uniform)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = base + threadIdx.x + kSmThreads * u < nacc;
#pragma unroll
        for (int e = 0; e < W; ++e) v[u][e] = ok ? v[u][e] : kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < W; ++e) mx = fmaxf(mx, v[u][e]);
    fold_chunk(r, mx, &v[0][0], U * W);

    if (base == 0) {
      // Threshold from the first chunk: the k-th largest of the 256 lane
      // maxima of the workgroup (k elements reach it, so nothing below it is
      // in the row's top k; groups of equal maxima are counted together).
      // One barrier; every wave starts from the same bound.
      lm_s[threadIdx.x] = mx;
      __syncthreads();
      float a4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a4[t] = lm_s[lane + 64 * t];
      int cnt = 0;
      while (true) {
        const float M = wave_max_bcast(fmaxf(fmaxf(a4[0], a4[1]), fmaxf(a4[2], a4[3])));
        if (M == kNegInf) break;  // fewer than k elements in this chunk
        int c = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          c += a4[t] == M ? 1 : 0;
          a4[t] = a4[t] == M ? kNegInf : a4[t];
        }
        // sum of c over the wave (c in [0, 4]) by four ballots
#pragma unroll
        for (int t = 0; t < 4; ++t) cnt += __builtin_popcountll(__ballot(c > t));
        if (cnt >= k) {
          Tx = M;
          break;
        }
      }
    }

    // Publish this wave's threshold, take the workgroup's.
    if (lane == 0 && Tx != kNegInf) atomicMax(&t_shared, ord_f(Tx));
    const float Tf = fmaxf(Tx, unord_f(__builtin_amdgcn_readfirstlane(t_shared)));
    // Nothing in the chunk reaches the threshold: no slot needs a look.
    if (__ballot((mx >= Tf) & (mx != kNegInf)) == 0) return;
    // Candidates (values reaching the threshold) go to this wave's queue in
    // LDS: one compare per register slot, a ballot, and a write by the lanes
    // that have one; the insertion is then one copy of code run once per
    // candidate.  (Inlining the insertion in every slot made this kernel
    // larger than the instruction cache.)  Slots past the row hold -inf and
    // never qualify.
    const float T = fmaxf(Tx, Tf);
    int n = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int a0 = base + w * 64 + kSmThreads * u;  // access index of lane 0
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const bool c = (v[u][e] >= T) & (v[u][e] != kNegInf);
        const uint64_t mask = __ballot(c);
        if (mask == 0) continue;  // wave-uniform
        if (c) {
          const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          qv_s[w][pos] = v[u][e];
          qi_s[w][pos] = (a0 + lane) * W + e;
        }
        n += __builtin_popcountll(mask);
      }
    }
    drain(n);
  };

  // Chunks are taken in pairs; a pair's second chunk may lie wholly past the
  // row, in which case all its slots are -inf and it changes nothing.  (An
  // early exit there would join paths with loads in flight, and the compiler
  // then waits for all loads at the top of the loop.)
  load_chunk(0, va);
  for (int base = 0; base < nacc; base += 2 * STEP) {
    load_chunk(base + STEP, vb);
    process(base, va);
    load_chunk(base + 2 * STEP, va);
    process(base + STEP, vb);
  }

  r = block_md(r);  // contains a __syncthreads

  __shared__ float cx_s[kSmWaves * 16];
  __shared__ int ci_s[kSmWaves * 16];
  if (lane < k) {
    cx_s[w * k + lane] = lx;
    ci_s[w * k + lane] = li;
  }
  __syncthreads();
  if (w == 0) {
    // Lane l holds candidate l; its rank counts the better candidates, each
    // broadcast from its lane (no LDS round trip per comparison).
    const int nk = kSmWaves * k;
    const float mx = lane < nk ? cx_s[lane] : kNegInf;
    const int mi = lane < nk ? ci_s[lane] : 0x7fffffff;
    int rank = 0;
    for (int j = 0; j < nk; ++j) {
      const float bx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), j));
      const int bi = __builtin_amdgcn_readlane(mi, j);
      rank += better(bx, bi, mx, mi) ? 1 : 0;
    }
    if (lane < nk && rank < k) {
      topv[(size_t)row * k + rank] = fast_exp2(fmaf(mx, kLog2e, -r.m)) / r.d;
      topi[(size_t)row * k + rank] = mi;
    }
  }
  if constexpr (WITH_Y) stream_write<W>(xr, y + (size_t)row * cols, nacc, r);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_softmax_rows(const float* x, float* y, int rows, int cols, hipStream_t stream) {
  const bool vec = (cols % 4 == 0) && aligned16(x) && aligned16(y);
  const dim3 grid(rows), block(kSmThreads);
  if (vec && kSoftmaxWavePerRow && cols / 4 <= 64 * 16 && rows >= 16 * 256) {
    const int nacc = cols / 4;
    const dim3 wgrid((rows + kSmWaves - 1) / kSmWaves);
    const dim3 wgrid2(((rows + 1) / 2 + kSmWaves - 1) / kSmWaves);
    if (nacc <= 64 * 4)
      hipLaunchKernelGGL((softmax_rows_wave_kernel<4, 1>), wgrid, block, 0, stream, x, y, rows, cols);
    else if (nacc <= 64 * 8)
      hipLaunchKernelGGL((softmax_rows_wave_kernel<8, 1>), wgrid, block, 0, stream, x, y, rows, cols);
    else
      hipLaunchKernelGGL((softmax_rows_wave_kernel<16, 2>), wgrid2, block, 0, stream, x, y, rows, cols);
  } else if (vec) {
    const int nacc = cols / 4;
    if (nacc <= 256)
      hipLaunchKernelGGL((softmax_rows_reg_kernel<4, 1>), grid, block, 0, stream, x, y, cols);
    else if (nacc <= 512)
      hipLaunchKernelGGL((softmax_rows_reg_kernel<4, 2>), grid, block, 0, stream, x, y, cols);
    else if (nacc <= 1024)
      hipLaunchKernelGGL((softmax_rows_reg_kernel<4, 4>), grid, block, 0, stream, x, y, cols);
    else if (nacc <= 2048)
      hipLaunchKernelGGL((softmax_rows_reg_kernel<4, 8>), grid, block, 0, stream, x, y, cols);
    else
      hipLaunchKernelGGL((softmax_rows_stream_kernel<4>), grid, block, 0, stream, x, y, cols);
  } else {
    if (cols <= 1024)
      hipLaunchKernelGGL((softmax_rows_reg_kernel<1, 4>), grid, block, 0, stream, x, y, cols);
    else if (cols <= 4096)
      hipLaunchKernelGGL((softmax_rows_reg_kernel<1, 16>), grid, block, 0, stream, x, y, cols);
    else
      hipLaunchKernelGGL((softmax_rows_stream_kernel<1>), grid, block, 0, stream, x, y, cols);
  }
  return hipGetLastError();
}

hipError_t launch_softmax_topk(const float* x, float* y, float* topv, int32_t* topi, int rows, int cols, int k,
                               hipStream_t stream) {
  const bool vec = (cols % 4 == 0) && aligned16(x) && (y == nullptr || aligned16(y));
  const dim3 grid(rows), block(kSmThreads);
  if (vec && y)
    hipLaunchKernelGGL((softmax_topk_kernel<4, true>), grid, block, 0, stream, x, y, topv, topi, cols, k);
  else if (vec)
    hipLaunchKernelGGL((softmax_topk_kernel<4, false>), grid, block, 0, stream, x, y, topv, topi, cols, k);
  else if (y)
    hipLaunchKernelGGL((softmax_topk_kernel<1, true>), grid, block, 0, stream, x, y, topv, topi, cols, k);
  else
    hipLaunchKernelGGL((softmax_topk_kernel<1, false>), grid, block, 0, stream, x, y, topv, topi, cols, k);
  return hipGetLastError();
}

}  // namespace osfa
