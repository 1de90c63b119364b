// Masks applied to MFMA accumulators of scores, shared by the forward and
// backward kernels (P: any parameter block with `causal` and `window`).
// Visibility of key j to query i: j < jmax, causal j <= i, window |i - j| <
// W.  Each mask returns at once when every score of the block is visible
// (a uniform branch), so interior blocks pay nothing; the compare-and-select
// code runs on boundary blocks only.
#pragma once

#include "device_common.h"
#include "tile_layout.h"

namespace osfa {
namespace {

// Masks of one 64-key block of scores held as S^T accumulators (register r
// of group kt holds key j0 + 32 kt + 16 (r / 8) + 8 hf + r % 8 of query
// qi): nothing when every query of the wave's rows [qa, qb] sees every key;
// per 32-key half, all -inf when no row sees it, otherwise one or two
// compares per score against the query's bounds on the key offset.
// mask_qlane_cut is the part after that test (for a block some score of
// which is masked).
template <class P>
__device__ __forceinline__ void mask_qlane_cut(const P& p, int jmax, int qi, int qa, int qb, int hf, f32x16 (&s)[2],
                                               int j0) {
  int hi = jmax - 1 - j0;                                    // padding: j < jmax
  int hi_min = hi, hi_max = hi;                              // over the wave's rows
  if (p.causal) {
    hi = min(hi, qi - j0);                                   // j <= i
    hi_min = min(hi_min, qa - j0);
    hi_max = min(hi_max, qb - j0);
  }
  int lo = -1 - kBc, lo_min = -1 - kBc, lo_max = -1 - kBc;
  if (p.window > 0) {
    lo = qi - p.window - j0;                                 // i - j < window
    lo_min = qa - p.window - j0;
    lo_max = qb - p.window - j0;
    if (!p.causal) {
      hi = min(hi, qi + p.window - 1 - j0);                  // j - i < window
      hi_min = min(hi_min, qa + p.window - 1 - j0);
      hi_max = min(hi_max, qb + p.window - 1 - j0);
    }
  }
  lo -= 8 * hf;
  hi -= 8 * hf;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int t0 = 32 * kt, t1 = 32 * kt + 31;
    if (hi_max < t0 || lo_min >= t1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = kNegInf;
      continue;
    }
    const bool need_hi = hi_min < t1, need_lo = lo_max >= t0;
    if (need_hi && need_lo) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 16 * (r >> 3) + (r & 7);
        s[kt][r] = ((t > lo) & (t <= hi)) ? s[kt][r] : kNegInf;
      }
    } else if (need_hi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 16 * (r >> 3) + (r & 7);
        s[kt][r] = (t <= hi) ? s[kt][r] : kNegInf;
      }
    } else if (need_lo) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 16 * (r >> 3) + (r & 7);
        s[kt][r] = (t > lo) ? s[kt][r] : kNegInf;
      }
    }
  }
}


template <class P>
__device__ __forceinline__ void mask_qlane(const P& p, int jmax, int qi, int qa, int qb, int hf, f32x16 (&s)[2],
                                           int j0) {
  // Does every query of [qa, qb] see every key of [j0, j0 + 64)?
  bool all = j0 + kBc <= jmax;
  if (p.causal) all = all && j0 + kBc - 1 <= qa;
  if (p.window > 0) all = all && qb - j0 < p.window && (p.causal || (j0 + kBc - 1) - qa < p.window);
  if (all) return;
  mask_qlane_cut(p, jmax, qi, qa, qb, hf, s, j0);
}

// The transposed layout of the dK / dV kernels: key kj in the lane, register
// r holds query i0 + 16 (r / 8) + 8 hf + r % 8 (32 queries i0 .. i0 + 31 of
// a block, the wave's keys [ja, jb]).  Queries past N are masked too (their
// staged rows are clamps of row N - 1).
template <class P>
__device__ __forceinline__ void mask_klane(const P& p, int jmax, int N, int kj, int ja, int jb, int hf, f32x16& s,
                                           int i0) {
  const int ia = i0, ib = i0 + 31;
  bool all = ib < N && jb < jmax;
  if (p.causal) all = all && jb <= ia;
  if (p.window > 0) all = all && ib - ja < p.window && (p.causal || jb - ia < p.window);
  if (all) return;
  // Query offset t = i - i0 - 8 hf visible iff lo < t <= hi.
  const int base = i0 + 8 * hf;
  int hi = N - 1 - base;                                     // i < N
  int lo = -1;
  if (kj >= jmax) hi = -1;                                   // padding key: nothing
  if (p.causal) lo = max(lo, kj - 1 - base);                 // i >= j
  if (p.window > 0) {
    hi = min(hi, kj + p.window - 1 - base);                  // i - j < W
    if (!p.causal) lo = max(lo, kj - p.window - base);       // j - i < W
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = 16 * (r >> 3) + (r & 7);
    s[r] = ((t > lo) & (t <= hi)) ? s[r] : kNegInf;
  }
}

}  // namespace
}  // namespace osfa
