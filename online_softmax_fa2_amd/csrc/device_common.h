// Device helpers shared by the gfx950 kernels: vector types, exp2, bf16
// packing, wavefront reductions and the associative merge of (m, d) pairs.
//
// Conventions used by every kernel in this library:
//   * exponentials are computed as exp2 with log2(e) folded into the score
//     scale, so running maxima are kept in log2 units; LSE is converted back
//     to natural-log units once per row;
//   * a wavefront has 64 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 2^x on the FMA pipes instead of the transcendental unit (the exponential
// offload of FlashAttention-4, page "Derive online softmax, prove it is
// exact", "What interviewers probe next"): split x = n + f with n the
// nearest integer and |f| <= 1/2, take 2^f from a cubic whose coefficients
// minimize the maximum relative error on [-1/2, 1/2] (a linear program on a
// dense grid, exp2_poly.py; 7.5e-5 with float32 coefficients, below the
// 2^-9 rounding of a bf16 P), and apply 2^n with v_ldexp_f32.  Arguments
// below -200 (masked scores: -inf) give exactly 0.  Eight VALU instructions
// (max, rndne, sub, 3 fma, cvt, ldexp) against one v_exp_f32.
constexpr float kExp2C0 = 0.9999280571937561f;
constexpr float kExp2C1 = 0.6932608485221863f;
constexpr float kExp2C2 = 0.24261115491390228f;
constexpr float kExp2C3 = 0.05517221987247467f;
__device__ __forceinline__ float exp2_fma(float x) {
  x = fmaxf(x, -200.0f);
  const float n = __builtin_rintf(x);
  const float f = x - n;
  const float p = fmaf(fmaf(fmaf(kExp2C3, f, kExp2C2), f, kExp2C1), f, kExp2C0);
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

// Exchange across the two 32-lane halves with v_permlane32_swap.  With
// operands (a, b) both holding x, the instruction leaves lane l < 32 with
// (x[l], x[l + 32]) and lane l >= 32 with (x[l - 32], x[l]).  The compiler
// folds the two results together when both operands are the same value, so
// the second operand is an identity DPP copy it cannot see through.
struct HalfPair {
  float lo, hi;  // (a, b) after the swap
};
__device__ __forceinline__ HalfPair permlane32_pair(float x) {
  const uint32_t a = __builtin_bit_cast(uint32_t, x);
  const uint32_t b = (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xE4, 0xF, 0xF, true);  // quad_perm identity
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return HalfPair{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
// max / sum of x over lanes l and l xor 32 (order-independent, no lane test).
// Maxima of scores and running maxima (finite or -inf, never NaN).  The
// device code is built with -fno-honor-nans, so the compiler turns fmaxf
// chains into v_max3_f32 without NaN-quieting copies, and, unlike inline
// assembly, it sees the reads and inserts the wait states an MFMA result
// needs before a VALU instruction reads it.  (Translation units built
// without that flag get the quieting copies: correct, a little slower.)
__device__ __forceinline__ float vmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float vmax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float max_halves(float x) {
  const HalfPair p = permlane32_pair(x);
  return vmax(p.lo, p.hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  const HalfPair p = permlane32_pair(x);
  return p.lo + p.hi;
}

// DPP helpers (gfx9 encodings): row_shr:n = 0x110 + n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143.  Lanes whose source is outside the row keep `old`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, x),
                                                               CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xF, false);
}

// Maximum over the 64 lanes, returned to every lane (an inclusive DPP scan
// that leaves the total in lane 63, then a broadcast of lane 63).
__device__ __forceinline__ float wave_max_bcast(float x) {
  const float ninf = -__builtin_huge_valf();
  x = fmaxf(x, dpp_f<0x111>(ninf, x));
  x = fmaxf(x, dpp_f<0x112>(ninf, x));
  x = fmaxf(x, dpp_f<0x114>(ninf, x));
  x = fmaxf(x, dpp_f<0x118>(ninf, x));
  x = fmaxf(x, dpp_f<0x142, 0xA>(ninf, x));
  x = fmaxf(x, dpp_f<0x143, 0xC>(ninf, x));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Butterfly all-reductions over the full 64-lane wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x += __shfl_xor(x, s, 64);
  return x;
}

// Merge two online-normalizer pairs (m in log2 units): the larger maximum
// wins and each sum is rescaled to it before adding (article "Online
// softmax", Step 4).  (-inf, 0) is the identity.
struct MD {
  float m, d;
};
__device__ __forceinline__ MD md_merge(MD a, MD b) {
  const float M = fmaxf(a.m, b.m);
  if (M == kNegInf) return MD{kNegInf, 0.0f};
  const float wa = (a.m == kNegInf) ? 0.0f : fast_exp2(a.m - M);
  const float wb = (b.m == kNegInf) ? 0.0f : fast_exp2(b.m - M);
  return MD{M, a.d * wa + b.d * wb};
}

__device__ __forceinline__ MD wave_md_merge(MD v) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    MD o{__shfl_xor(v.m, s, 64), __shfl_xor(v.d, s, 64)};
    v = md_merge(v, o);
  }
  return v;
}

// Empty register constraint on a value: the code that computes it stays
// before this point (the compiler may not sink it towards its uses).  The
// constraint exists only for the device target; the host pass sees nothing.
#if defined(__HIP_DEVICE_COMPILE__)
#define OSFA_KEEP(x) asm volatile("" : "+v"(x))
#else
#define OSFA_KEEP(x) ((void)0)
#endif

// bf16 helpers.
// acc + lo + hi of a packed pair of bf16 values (v_dot2_f32_bf16 against
// (1, 1), float32 accumulate).
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

}  // namespace osfa
