// Shared by the forward kernels (attn_fwd.hip, attn_fwd_fp8.hip): launch
// parameters, the XCD-aware tile order, the visible key range of a query
// tile and the mask predicates (causal j <= i, window |i - j| < W, padding
// j < kv_len[b]).  Everything lives in an anonymous namespace: each
// translation unit has its own copy.
#pragma once

#include "device_common.h"
#include "launch.h"
#include "masks.h"
#include "tile_layout.h"

namespace osfa {
namespace {

constexpr int kWaves = 4;         // waves per workgroup
constexpr int kBr = 32 * kWaves;  // queries per tile
constexpr int kThreads = 64 * kWaves;
// Lazy rescale: the reference m_ref of l and A moves only when a block's row
// maximum exceeds it by more than kTau (log2 units), so P = exp2(s - m_ref)
// stays <= 2^kTau.  Exact: O = A / l and LSE = m_ref + log2 l do not depend on
// which common reference was used (page "Online softmax for a whole query
// tile, matrix form", "What interviewers probe next").  The reference is
// always a visible score, so l >= 1 and nothing that matters underflows; P <=
// 2^32 bounds l by N 2^32 and |A| by N 2^32 max|v|, far inside float32 for
// N < 2^23 unless |v| > 2^72.  A large threshold makes the rescale of A (64
// multiplies per lane) rare.
constexpr float kTau = 32.0f;
// d = 128 bf16 kernel shape: waves per workgroup.
constexpr int kV2Waves = 4;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_len;
  int B, H, N;
  float c;  // scale * log2(e)
  int causal, window;
  float o_scale;  // multiplies O before the store (the V descale of the fp8 path; 1 otherwise)
  int br;       // query rows per tile
  int n_tiles;  // ceil(N / br)
  int total;    // B * H * n_tiles
};

// The 8 XCDs receive workgroups round-robin (hardware id % 8).  Give each XCD
// a contiguous range of logical ids so that the tiles of one (b, h), which
// share K and V, run on the same XCD and reuse its L2.  Tiles of a head run
// last-first: under causal masking they see the most keys.
struct Tile {
  int bh, q0;
  bool valid;
};
__device__ __forceinline__ Tile map_tile(const FwdParams& p) {
  const int per_xcd = gridDim.x / 8;  // grid is padded to a multiple of 8
  const int wg = blockIdx.x;
  const int logical = (wg % 8) * per_xcd + wg / 8;
  Tile t;
  t.valid = logical < p.total;
  const int bh = logical / p.n_tiles;
  const int tile = p.n_tiles - 1 - (logical - bh * p.n_tiles);
  t.bh = bh;
  t.q0 = tile * p.br;
  return t;
}

// Visible key range [kbeg, kend) of the tile's queries [q0, q0 + kBr) and the
// per-element bound on j (min(N, kv_len)).
struct KeyRange {
  int kbeg, kend, jmax;
};
__device__ __forceinline__ KeyRange key_range(const FwdParams& p, int b, int q0) {
  int klen = p.N;
  if (p.kv_len) {
    klen = p.kv_len[b];
    klen = klen < 0 ? 0 : (klen > p.N ? p.N : klen);
  }
  KeyRange r;
  r.jmax = klen;
  int kend = klen;
  if (p.causal) kend = min(kend, q0 + p.br);
  if (p.window > 0 && !p.causal) kend = min(kend, q0 + p.br - 1 + p.window);
  r.kend = kend;
  r.kbeg = (p.window > 0) ? max(0, q0 - p.window + 1) : 0;
  return r;
}

// True if every (i, j) with i in the tile and j in [j0, j0 + kBc) is visible.
__device__ __forceinline__ bool block_interior(const FwdParams& p, const KeyRange& r, int q0, int j0) {
  if (j0 + kBc > r.jmax) return false;
  if (p.causal && j0 + kBc - 1 > q0) return false;
  if (p.window > 0) {
    if ((q0 + p.br - 1) - j0 >= p.window) return false;
    if (!p.causal && (j0 + kBc - 1) - q0 >= p.window) return false;
  }
  return true;
}

__device__ __forceinline__ bool visible(const FwdParams& p, int jmax, int i, int j) {
  bool v = j < jmax;
  if (p.causal) v = v && (j <= i);
  if (p.window > 0) v = v && (i - j < p.window) && (j - i < p.window);
  return v;
}

// Does any query of rows [qa, qb] see a key of [j0, j0 + kBc)?  (A wave owns
// 32 rows; it skips the MFMAs and softmax of blocks it cannot see.)
__device__ __forceinline__ bool rows_see_block(const FwdParams& p, int jmax, int qa, int qb, int j0) {
  if (j0 >= jmax) return false;
  if (p.causal && j0 > qb) return false;
  if (p.window > 0) {
    if (qa - (j0 + kBc - 1) >= p.window) return false;
    if (!p.causal && j0 - qb >= p.window) return false;
  }
  return true;
}
// Does every query of rows [qa, qb] see every key of [j0, j0 + kBc)?
__device__ __forceinline__ bool rows_see_all(const FwdParams& p, int jmax, int qa, int qb, int j0) {
  if (j0 + kBc > jmax) return false;
  if (p.causal && j0 + kBc - 1 > qa) return false;
  if (p.window > 0) {
    if (qb - j0 >= p.window) return false;
    if (!p.causal && (j0 + kBc - 1) - qa >= p.window) return false;
  }
  return true;
}



// Masks of one 64-key block of scores held as S^T accumulators (register r
// of group kt holds key j0 + 32 kt + 16 (r / 8) + 8 hf + r % 8 of query qi).
__device__ __forceinline__ void mask_block(const FwdParams& p, const KeyRange& kr, int qi, int qa, int qb, int hf,
                                           f32x16 (&s)[2], int j0) {
  if (rows_see_all(p, kr.jmax, qa, qb, j0)) return;
  mask_qlane_cut(p, kr.jmax, qi, qa, qb, hf, s, j0);
}

FwdParams make_params(const FwdArgs& a, int br) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.kv_len = a.kv_len;
  p.B = a.B;
  p.H = a.H;
  p.N = a.N;
  p.c = a.scale * kLog2e;
  p.o_scale = 1.0f;
  p.causal = a.causal ? 1 : 0;
  // |i - j| <= N - 1 always, so a window beyond N masks nothing; clamping it
  // keeps every bound below int range.
  p.window = a.window > 0 ? (a.window > a.N ? a.N : a.window) : 0;
  p.br = br;
  p.n_tiles = (a.N + br - 1) / br;
  p.total = a.B * a.H * p.n_tiles;
  return p;
}

unsigned grid_for(const FwdParams& p) { return (unsigned)((p.total + 7) / 8 * 8); }

}  // namespace
}  // namespace osfa
