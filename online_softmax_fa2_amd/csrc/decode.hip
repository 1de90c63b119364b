// Split-KV decode for gfx950: one query per (b, h), the keys split across
// workgroups, each split running the online-softmax recurrence and leaving
// a partial (m, l, a) triple, then a merge kernel combining the partials
// with the rescale rule (page "Derive online softmax, prove it is exact",
// the batch-1 decoding follow-up; article "Online softmax", Step 4 and the
// Flash-Decoding note under "Trade-offs and edge cases").
//
// This path streams K and V once and does a few FLOPs per byte, so it is
// HBM-bound: the design goal is full-width coalesced 16-byte loads with many
// bytes in flight, not matrix cores.  Layout of the work:
//   * grid = B * H * nsplit workgroups of 4 waves; split c of (b, h) covers
//     keys [c L, min((c + 1) L, Nkv)), L = ceil(Nkv / nsplit);
//   * a key row (d elements) is read by D/8 consecutive lanes, 8 elements
//     (16 B for bf16) each, so one wave-wide load covers 64 / (D/8)
//     consecutive key rows, contiguous in memory;
//   * each lane group (the D/8 lanes of one key slot) keeps its own
//     (m, l, a[8 d per lane]) over the keys it visits; the score of a key is
//     the group's dot-product partials summed with DPP row operations;
//   * at the end the 4 * 64/(D/8) group states are merged through LDS by the
//     same rule and written as the split's partial.
// Partials (workspace, float32): [B, H, nsplit, D + 2] = (m, l, a[0..D)),
// with m in log2 units of the scaled score (m = log2(e) * max score).
#include <atomic>

#include "device_common.h"
#include "launch.h"

namespace osfa {

// Partials of attn_decode_splitkv_noalloc, the entry point for callers that
// cannot allocate: a device global of kDecodeScratchBytes, one copy per GPU
// the library runs on, held until the process ends.  Host code never uses
// this name as an address; it uses the per-device pointer from
// decode_scratch() below.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {

constexpr int kDecThreads = 256;
constexpr int kUnroll = 8;  // key rows per lane per step (loads in flight)

template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  // 8 elements = 16 bytes
  typedef u32x4 Vec;
  __device__ static inline void unpack(const Vec& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v[i]);
      f[2 * i + 1] = bf16_hi(v[i]);
    }
  }
};
template <>
struct Elem<float> {
  struct Vec {
    f32x4 a, b;
  };
  __device__ static inline void unpack(const Vec& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = v.a[i];
      f[4 + i] = v.b[i];
    }
  }
};

__device__ __forceinline__ u32x4 nt_load(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ Elem<float>::Vec nt_load(const Elem<float>::Vec* p) {
  return Elem<float>::Vec{__builtin_nontemporal_load(&p->a), __builtin_nontemporal_load(&p->b)};
}

// Sum over each aligned group of G lanes (G = 8 or 16) with DPP row ops:
// xor-1 and xor-2 quad permutes, then mirror within 8, then within 16.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
  if constexpr (G == 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(const T* __restrict__ q,
                                                                     const T* __restrict__ K,
                                                                     const T* __restrict__ V,
                                                                     float* __restrict__ ws, int Nkv,
                                                                     int nsplit, int L, float c) {
  typedef typename Elem<T>::Vec Vec;
  constexpr int G = D / 8;             // lanes per key row
  constexpr int SLOTS = 64 / G;        // key rows per wave-wide load
  constexpr int WAVES = kDecThreads / 64;
  constexpr int STEP = WAVES * SLOTS * kUnroll;  // keys per workgroup step
  constexpr int NGROUPS = WAVES * SLOTS;

  const int wg = blockIdx.x;
  const int split = wg % nsplit;
  const int bh = wg / nsplit;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int slot = lane / G;
  const int dc = lane % G;  // d chunk: d = 8 dc + [0, 8)

  const size_t kv_off = (size_t)bh * (size_t)Nkv * D;
  const T* Kh = K + kv_off;
  const T* Vh = V + kv_off;
  float qf[8];
  Elem<T>::unpack(*reinterpret_cast<const Vec*>(q + (size_t)bh * D + 8 * dc), qf);

  const int lo = split * L;
  const int hi = min(lo + L, Nkv);

  float m = kNegInf, l = 0.0f;
  float a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = 0.0f;

  for (int base = lo; base < hi; base += STEP) {
    Vec kv[kUnroll], vv[kUnroll];
    int jj[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = base + (u * WAVES + w) * SLOTS + slot;
      jj[u] = j;
      const int js = j < hi ? j : hi - 1;
      kv[u] = nt_load(reinterpret_cast<const Vec*>(Kh + (size_t)js * D + 8 * dc));  // streamed once
      vv[u] = nt_load(reinterpret_cast<const Vec*>(Vh + (size_t)js * D + 8 * dc));
    }
    float s[kUnroll];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      Elem<T>::unpack(kv[u], kf);
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(qf[e], kf[e], part);
      part = group_sum<G>(part);
      s[u] = jj[u] < hi ? part : kNegInf;
      mx = fmaxf(mx, s[u]);
    }
    const float m_new = fmaxf(m, mx * c);
    const float m_ref = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m - m_ref);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float pexp = fast_exp2(fmaf(s[u], c, -m_ref));
      l += pexp;
      float vf[8];
      Elem<T>::unpack(vv[u], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = fmaf(pexp, vf[e], a[e]);
    }
    m = m_new;
  }

  // Merge the NGROUPS group states of the workgroup.
  __shared__ float sm[NGROUPS], sl[NGROUPS];
  __shared__ float sa[NGROUPS][D];
  const int g = w * SLOTS + slot;
  if (dc == 0) {
    sm[g] = m;
    sl[g] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sa[g][8 * dc + e] = a[e];
  __syncthreads();
  float* out = ws + ((size_t)bh * nsplit + split) * (D + 2);
  for (int d = tid; d < D; d += kDecThreads) {
    float M = kNegInf;
    for (int i = 0; i < NGROUPS; ++i) M = fmaxf(M, sm[i]);
    float lt = 0.0f, at = 0.0f;
    for (int i = 0; i < NGROUPS; ++i) {
      const float wgt = (sm[i] == kNegInf) ? 0.0f : fast_exp2(sm[i] - M);
      lt = fmaf(wgt, sl[i], lt);
      at = fmaf(wgt, sa[i][d], at);
    }
    out[2 + d] = at;
    if (d == 0) {
      out[0] = M;
      out[1] = lt;
    }
  }
}

// One workgroup per (b, h): o = sum_c w_c a_c / sum_c w_c l_c with
// w_c = 2^(m_c - M), M = max_c m_c, and w_c = 0 for an empty split.
// Only the weights depend on M, so every thread issues its loads at once --
// (m_c, l_c) of split c = tid and the first kMergeAhead values a_c[d] of its
// column -- and the three steps (M, the weighted l, the weighted a) then
// wait on one round of global latency instead of three.  Thread (d, g) sums
// the splits c = g mod G for column d in increasing c, and the G partial
// sums are combined through LDS; splits past the first pass (nsplit > 256,
// or past kMergeAhead G) are read in the same order afterwards.
constexpr int kMergeThreads = 256;
constexpr int kMergeAhead = 32;
template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float* __restrict__ ws,
                                                                     float* __restrict__ o, int nsplit) {
  constexpr int G = kMergeThreads / D;  // split groups
  __shared__ float s_w[4096];           // nsplit <= 4096
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ float s_acc[G][D];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const float* part = ws + (size_t)bh * nsplit * (D + 2);
  const int d = tid % D, g = tid / D;

  const bool own = tid < nsplit;
  const float m0 = own ? part[(size_t)tid * (D + 2)] : kNegInf;
  const float l0 = own ? part[(size_t)tid * (D + 2) + 1] : 0.0f;
  float av[kMergeAhead];
#pragma unroll
  for (int i = 0; i < kMergeAhead; ++i) {
    const int c = g + G * i;
    av[i] = c < nsplit ? part[(size_t)c * (D + 2) + 2 + d] : 0.0f;
  }

  float mloc = m0;
  for (int c = tid + kMergeThreads; c < nsplit; c += kMergeThreads) mloc = fmaxf(mloc, part[(size_t)c * (D + 2)]);
  mloc = wave_max(mloc);
  if (lane == 0) s_red[w] = mloc;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int i = 1; i < kMergeThreads / 64; ++i) M = fmaxf(M, s_red[i]);
  __syncthreads();  // s_red is reused below

  float lloc = 0.0f;
  if (own) {
    const float wgt = (m0 == kNegInf) ? 0.0f : fast_exp2(m0 - M);
    s_w[tid] = wgt;
    lloc = wgt * l0;
  }
  for (int c = tid + kMergeThreads; c < nsplit; c += kMergeThreads) {
    const float mc = part[(size_t)c * (D + 2)];
    const float wgt = (mc == kNegInf) ? 0.0f : fast_exp2(mc - M);
    s_w[c] = wgt;
    lloc = fmaf(wgt, part[(size_t)c * (D + 2) + 1], lloc);
  }
  lloc = wave_sum(lloc);
  if (lane == 0) s_red[w] = lloc;
  __syncthreads();
  float lt = 0.0f;
#pragma unroll
  for (int i = 0; i < kMergeThreads / 64; ++i) lt += s_red[i];

  float at = 0.0f;
#pragma unroll
  for (int i = 0; i < kMergeAhead; ++i) {
    const int c = g + G * i;
    if (c < nsplit) at = fmaf(s_w[c], av[i], at);
  }
  for (int c = g + G * kMergeAhead; c < nsplit; c += G) at = fmaf(s_w[c], part[(size_t)c * (D + 2) + 2 + d], at);
  s_acc[g][d] = at;
  __syncthreads();
  if (g == 0) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) a += s_acc[i][d];
    o[(size_t)bh * D + d] = lt > 0.0f ? a / lt : 0.0f;
  }
}

template <typename T>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int L = (a.Nkv + a.nsplit - 1) / a.nsplit;
  const float c = (float)(1.0 / __builtin_sqrt((double)a.d)) * kLog2e;
  const unsigned nwg = (unsigned)(a.B * a.H * a.nsplit);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  if (a.d == 128) {
    hipLaunchKernelGGL((decode_partial_kernel<T, 128>), dim3(nwg), dim3(kDecThreads), 0, stream, q, k, v, a.ws,
                       a.Nkv, a.nsplit, L, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(a.B * a.H), dim3(kMergeThreads), 0, stream, a.ws, a.o, a.nsplit);
  } else {
    hipLaunchKernelGGL((decode_partial_kernel<T, 64>), dim3(nwg), dim3(kDecThreads), 0, stream, q, k, v, a.ws,
                       a.Nkv, a.nsplit, L, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(a.B * a.H), dim3(kMergeThreads), 0, stream, a.ws, a.o, a.nsplit);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch_decode<__bf16>(a, stream); }
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) { return launch_decode<float>(a, stream); }

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];  // device address of `scratch` per device, set on first use
}  // namespace

// The address of `scratch` on the current device, looked up once per device
// with that device current (every GPU holds its own copy at its own address).
hipError_t decode_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* raw = nullptr;
    e = hipGetSymbolAddress(&raw, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (raw == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<float*>(raw);
    g_scratch[dev].store(p, std::memory_order_release);  // racing first calls store the same address
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_decode_noalloc(const DecodeArgs& a_in, bool bf16, hipStream_t stream) {
  DecodeArgs a = a_in;
  const hipError_t e = decode_scratch(&a.ws);
  if (e != hipSuccess) return e;
  return bf16 ? launch_decode<__bf16>(a, stream) : launch_decode<float>(a, stream);
}

}  // namespace osfa
