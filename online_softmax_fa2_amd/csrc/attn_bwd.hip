// Attention backward pass for gfx950 (bf16, d = 128): the gradients dQ, dK,
// dV of the forward output, with P recomputed block by block from Q, K and
// the per-row log-sum-exp the forward wrote, normalized directly as
// P = exp(S - LSE) with no running maximum (page "Derive online softmax,
// prove it is exact", "What interviewers probe next"; page "Online softmax
// for a whole query tile, matrix form", "What interviewers probe next").
//
//   D_i  = sum_d dO_id O_id                      (bwd_dq_kernel, for both)
//   dP   = dO V^T,  dS = P * (dP - D_i)          (the softmax Jacobian)
//   dQ   = scale dS K                             (bwd_dq_kernel: query tiles)
//   dV   = P^T dO                                  (bwd_dkdv_kernel: key tiles)
//   dK   = scale dS^T Q                            (bwd_dkdv_kernel)
//
// Each kernel recomputes the scores (and dP where it needs it) over the tiles
// it owns, so every gradient row is summed inside one workgroup (no atomics,
// deterministic).
//
// bwd_dq_kernel keeps the forward's layout: each wave owns 32 queries (the
// lane's column of every accumulator), Q and dO rows live in VGPRs as MFMA B
// operands, K and V blocks of 64 keys stream through LDS (buffer loads
// straight to LDS, double buffered), S^T = K Q^T and dP^T = V dO^T are MFMA
// contractions whose accumulators hold 8 consecutive keys per 8 registers,
// so the bf16 dS^T is directly the B operand of dQ^T += K^T dS^T (K read
// transposed from LDS).
//
// bwd_dkdv_kernel swaps the roles: each wave owns 32 keys (their K rows in
// VGPRs as the B operand of S, their V rows in LDS for dP), and blocks of 32
// queries (Q, dO, and their LSE and D) stream through LDS; P and dS are
// formed once for both gradients.  S = Q K^T and dP = dO V^T
// hold, per lane, 8 consecutive queries per 8 registers, which makes the
// bf16 P and dS the B operands of dV^T += dO^T P and dK^T += Q^T dS (dO and
// Q read transposed).
//
// Two waves per SIMD do not overlap one wave's VALU work with the other's
// MFMAs, and an MFMA whose LDS operand was read just before it waits out the
// read's latency; both kernels therefore keep a queue of operand fragments
// in flight a few MFMAs ahead of their use.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "masks.h"
#include "tile_layout.h"

namespace osfa {
namespace {

constexpr int D = 128;
constexpr int kW = 4;                 // waves per workgroup
constexpr int kT = 64 * kW;           // threads per workgroup
constexpr int kTile = 32 * kW;        // queries (dq) or keys (dkdv) per workgroup
constexpr int kQb = 32;               // queries per block in bwd_dkdv_kernel
constexpr int NKK = D / 16;
constexpr int NMD = D / 32;
// LDS operand fragments in flight ahead of their MFMA: bwd_dq_kernel's A
// operands, bwd_dkdv_kernel's A operands and its V rows.  Deeper queues do
// not fit in the 256 registers of two waves per SIMD (they spill).
constexpr int kDqAhead = 4, kKvAhead = 3, kVAhead = 2;

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* delta;  // workspace [B, H, N]: D_i
  float* lse2;   // workspace [B, H, N]: LSE_i log2(e), +inf for a row with no key
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  const int32_t* kv_len;
  int B, H, N;
  float c;      // scale * log2(e)
  float scale;
  int causal, window;
  int n_tiles;  // ceil(N / kTile)
  int total;    // B * H * n_tiles
  __bf16* ds;   // stored-dS tiles (launch.h: ds_span, ds_first), or nullptr
  int nqb;      // ceil(N / 32): query blocks per head
  int span;     // tile slots per query block
};

// Workgroups go to the 8 XCDs round-robin; each XCD takes a contiguous range
// of logical tiles (the tiles of one head share K, V, Q and dO in its L2).
struct Tile {
  int bh, t0;
  bool valid;
};
__device__ __forceinline__ Tile map_tile(const BwdParams& p, bool ascending, int tile_rows = kTile) {
  const int per_xcd = gridDim.x / 8;  // grid padded to a multiple of 8
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  Tile t;
  t.valid = logical < p.total;
  t.bh = logical / p.n_tiles;
  const int r = logical - t.bh * p.n_tiles;
  t.t0 = (ascending ? r : p.n_tiles - 1 - r) * tile_rows;
  return t;
}

__device__ __forceinline__ int key_limit(const BwdParams& p, int b) {
  int klen = p.N;
  if (p.kv_len) {
    klen = p.kv_len[b];
    klen = klen < 0 ? 0 : (klen > p.N ? p.N : klen);
  }
  return klen;
}

// Does some query of [qa, qb] see some key of [ja, jb]?  (j < jmax, causal
// j <= i, window |i - j| < W.)
__device__ __forceinline__ bool any_visible(const BwdParams& p, int jmax, int qa, int qb, int ja, int jb) {
  if (ja >= jmax) return false;
  if (p.causal) {
    if (ja > qb) return false;
    if (p.window > 0 && qa - jb >= p.window) return false;
  } else if (p.window > 0) {
    if (qa - jb >= p.window || ja - qb >= p.window) return false;
  }
  return true;
}
// any_visible without branches (a per-lane value for the stored-dS loads).
__device__ __forceinline__ bool any_visible_sel(const BwdParams& p, int jmax, int qa, int qb, int ja, int jb) {
  const bool w = p.window > 0;
  const bool c = ja <= qb && (!w | (qa - jb < p.window));
  const bool n = !w | ((qa - jb < p.window) & (ja - qb < p.window));
  return (ja < jmax) & (p.causal ? c : n);
}

// Buffer loads straight to LDS of rows [r0, r0 + 4 NLD) of a [N, 128] bf16
// matrix in the layout of tile_layout.h: load t of wave w fills 1 KB (rows
// 4 (w + kW t) .. + 3 of the block).  Rows past N read row N - 1.
template <int NLD>
__device__ __forceinline__ void stage_rows(__amdgpu_buffer_rsrc_t rs, char* dst, int r0, int N, int w, int lane) {
#pragma unroll
  for (int t = 0; t < NLD / kW; ++t) {
    const int row = 4 * (w + kW * t) + (lane >> 4);
    const int grow = min(r0 + row, N - 1);
    const int off = (grow * D + 8 * ((lane & 15) ^ swz(row))) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (w + kW * t) * 1024),
                                             16, (int)off, 0, 0, 0);
  }
}

// The 16-byte row fragment (chunk 2 kk + hf) of row `row` of a staged block.
__device__ __forceinline__ bf16x8 row_frag(const char* blk, int row, int kk, int hf) {
  return *reinterpret_cast<const bf16x8*>(blk + kv_off(row, 2 * kk + hf));
}

// Transposed reads: 8 consecutive rows (16 g + 8 hf .. + 7) of column
// 32 md + l32 of a staged block, as the A operand of a 32x32x16 MFMA.
struct TrOff {
  int off[2][NMD];
};
__device__ __forceinline__ TrOff tr_offsets(int lane) {
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int rowoff = 8 * (tr_g >> 1) + (tr_j >> 2);
  const int col = 16 * (tr_g & 1) + 4 * (tr_j & 3);
  const int byte = (tr_j & 1) * 8;
  TrOff t;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int md = 0; md < NMD; ++md) t.off[r][md] = kv_off(4 * r + rowoff, (32 * md + col) >> 3) + byte;
  return t;
}
__device__ __forceinline__ bf16x8 tr_frag(const char* blk, const TrOff& t, int md, int g) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x4 h[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(blk + t.off[r][md] + 4096 * g));
  const s16x8 hv = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8, hv);
}

// A wave's 32 output rows of 128 bf16 (lane: row l32, columns 32 md + 8 rq
// + 4 hf .. + 3 from a[md][4 rq .. 4 rq + 3], times f) stored as whole
// 256-byte rows r0 .. r0 + 31 of dst, rows >= nrows skipped.  Stored
// directly, each instruction would write 16-byte runs scattered over 32
// rows; the rows go through `reg`, 8 KB of LDS that only this wave uses
// (swizzled block layout), and back out 4 rows per instruction.
__device__ __forceinline__ void store_rows(char* reg, const f32x16 (&a)[NMD], float f, __bf16* dst, int r0, int nrows,
                                           int lane) {
  const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      u32x2 wv;
      wv[0] = pack_bf16x2(a[md][4 * rq + 0] * f, a[md][4 * rq + 1] * f);
      wv[1] = pack_bf16x2(a[md][4 * rq + 2] * f, a[md][4 * rq + 3] * f);
      *reinterpret_cast<u32x2*>(reg + kv_off(l32, 4 * md + rq) + 8 * hf) = wv;
    }
  u32x4 rows[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) rows[t] = *reinterpret_cast<const u32x4*>(reg + kv_off(4 * t + (lane >> 4), lane & 15));
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int r = r0 + 4 * t + (lane >> 4);
    if (r < nrows) *reinterpret_cast<u32x4*>(dst + (size_t)r * D + 8 * (lane & 15)) = rows[t];
  }
}

// ---------------------------------------------------------------------------
// dQ: query tiles of 128, key blocks of 64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT, 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int RQ = kDqAhead;
  constexpr int BLK = kBc * D * 2;  // 16 KB
  constexpr int LOADS = 16;         // load instructions per block (1 KB each)
  __shared__ __attribute__((aligned(1024))) char k0[BLK];
  __shared__ __attribute__((aligned(1024))) char k1[BLK];
  __shared__ __attribute__((aligned(1024))) char v0[BLK];
  __shared__ __attribute__((aligned(1024))) char v1[BLK];

  const Tile tile = map_tile(p, false);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.t0;
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)tile.bh * N;
  const int jmax = key_limit(p, b);

  // Key range of the tile (as the forward).
  int kend = jmax;
  if (p.causal) kend = min(kend, q0 + kTile);
  if (p.window > 0 && !p.causal) kend = min(kend, q0 + kTile - 1 + p.window);
  const int kbeg = p.window > 0 ? max(0, q0 - p.window + 1) : 0;
  const int kb_lo = kbeg / kBc;
  const int nblk = kend > kbeg ? (kend + kBc - 1) / kBc - kb_lo : 0;

  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + head * D), 0, N * D * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + head * D), 0, N * D * 2, kBufDword3);
  auto load_block = [&](int j, char* kd, char* vd) {
    stage_rows<LOADS>(krs, kd, (kb_lo + j) * kBc, N, w, lane);
    stage_rows<LOADS>(vrs, vd, (kb_lo + j) * kBc, N, w, lane);
  };
  if (nblk > 0) load_block(0, k0, v0);

  const int qi = q0 + 32 * w + l32;
  const bool qok = qi < N;
  bf16x8 qreg[NKK], doreg[NKK];
  {
    const size_t r = head + (size_t)(qok ? qi : 0);
    const u32x4* qs = reinterpret_cast<const u32x4*>(p.q + r * D + 8 * hf);
    const u32x4* gs = reinterpret_cast<const u32x4*>(p.dout + r * D + 8 * hf);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qreg[kk] = __builtin_bit_cast(bf16x8, qok ? qs[2 * kk] : u32x4{0, 0, 0, 0});
      doreg[kk] = __builtin_bit_cast(bf16x8, qok ? gs[2 * kk] : u32x4{0, 0, 0, 0});
    }
  }
  // D_i = sum_d dO_id O_id (this half's 64 columns, then the other half's)
  // and LSE in log2 units (+inf for a row with no key, so exp2(s - lse2) is
  // 0 there); written to the workspace for bwd_dkdv_kernel, which runs next.
  float dlt = 0.0f;
  {
    const u32x4* os = reinterpret_cast<const u32x4*>(p.o + (head + (qok ? qi : 0)) * D + 8 * hf);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 a = qok ? os[2 * kk] : u32x4{0, 0, 0, 0};
      const u32x4 g = __builtin_bit_cast(u32x4, doreg[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dlt = fmaf(bf16_lo(a[e]), bf16_lo(g[e]), dlt);
        dlt = fmaf(bf16_hi(a[e]), bf16_hi(g[e]), dlt);
      }
    }
  }
  dlt = sum_halves(dlt);
  const float lse_in = qok ? p.lse[head + qi] : kNegInf;
  const float lse2 = lse_in == kNegInf ? __builtin_huge_valf() : lse_in * kLog2e;
  if (qok && hf == 0) {
    p.delta[head + qi] = dlt;
    p.lse2[head + qi] = lse2;
  }
  const float c = p.c;
  const int qa = q0 + 32 * w, qb = qa + 31;
  const int krow = perm_key(l32);
  const TrOff tro = tr_offsets(lane);

  f32x16 acc[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[md][r] = 0.0f;

  auto block = [&](int j, const char* kl, const char* vl) {
    const int j0 = (kb_lo + j) * kBc;
    if (!any_visible(p, jmax, qa, qb, j0, j0 + kBc - 1)) return;
    // The block's 48 A operands in MFMA order: K rows (S^T), V rows (dP^T),
    // K transposed (dQ^T).  RQ of them are in flight ahead of their MFMA.
    auto frag = [&](int i) -> bf16x8 {
      if (i < 16) return row_frag(kl, 32 * (i >> 3) + krow, i & 7, hf);
      if (i < 32) return row_frag(vl, 32 * ((i - 16) >> 3) + krow, i & 7, hf);
      return tr_frag(kl, tro, (i - 32) >> 2, i & 3);
    };
    bf16x8 fq[RQ];
#pragma unroll
    for (int i = 0; i < RQ; ++i) fq[i] = frag(i);
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[i % RQ], qreg[i & 7], s[i >> 3], 0, 0, 0);
      fq[i % RQ] = frag(i + RQ);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Register r of group kt holds key j0 + 32 kt + 16 (r / 8) + 8 hf + r % 8
    // of query qi: masked scores take P = 0, and so dS = 0.  P replaces S in
    // place; dP^T is formed one 32-key group at a time (fewer live VGPRs).
    mask_qlane(p, jmax, qi, qa, qb, hf, s, j0);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = fast_exp2(fmaf(s[kt][r], c, -lse2));
    bf16x8 ds[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int i = 16 + 8 * kt + kk;
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[i % RQ], doreg[kk], dp, 0, 0, 0);
        fq[i % RQ] = frag(i + RQ);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = s[kt][8 * t + e] * (dp[8 * t + e] - dlt);
        ds[kt][t] = __builtin_convertvector(f, bf16x8);
      }
    }
    // dQ^T += K^T dS^T: K read transposed, 16 keys per MFMA.
#pragma unroll
    for (int i = 32; i < 48; ++i) {
      const int md = (i - 32) >> 2, g = i & 3;
      acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[i % RQ], ds[g >> 1][g & 1], acc[md], 0, 0, 0);
      if (i + RQ < 48) fq[i % RQ] = frag(i + RQ);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto iter = [&](int j, const char* kl, const char* vl, char* kn, char* vn) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (j + 1 < nblk) load_block(j + 1, kn, vn);
    block(j, kl, vl);
  };
  // Two blocks per trip, one call site per buffer: with an if/else on the
  // parity the accumulators came out of the join in different registers
  // and were copied every block.
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    iter(j, k0, v0, k1, v1);
    iter(j + 1, k1, v1, k0, v0);
  }
  if (j < nblk) iter(j, k0, v0, k1, v1);

  // dQ rows through the K buffers, once every wave is past its last read.
  static_assert(kW == 4, "two waves' rows per K buffer");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  store_rows((w < 2 ? k0 : k1) + (w & 1) * (32 * D * 2), acc, p.scale, p.dq + head * D, tile.t0 + 32 * w, N, lane);
}

// ---------------------------------------------------------------------------
// dK and dV: key tiles of 128, query blocks of 32.  Both 32 keys x 128
// columns accumulators of a wave (128 VGPRs) and its K rows (32) are held in
// registers; the V rows, needed only as the dP operand, are read from LDS
// (staged once).  Operand fragments are read a few MFMAs ahead, from offsets
// formed next to the read, which keeps the kernel at two waves per SIMD.
// ---------------------------------------------------------------------------
template <bool kStoreDs>
__global__ __launch_bounds__(kT, 2) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int RA = kKvAhead, RV = kVAhead;
  constexpr int QBLK = kQb * D * 2;  // 8 KB
  __shared__ __attribute__((aligned(1024))) char q0b[QBLK];
  __shared__ __attribute__((aligned(1024))) char q1b[QBLK];
  __shared__ __attribute__((aligned(1024))) char g0b[QBLK];
  __shared__ __attribute__((aligned(1024))) char g1b[QBLK];
  __shared__ __attribute__((aligned(256))) float st0[2 * 64];  // lse2, delta of a block (+ slack)
  __shared__ __attribute__((aligned(256))) float st1[2 * 64];
  __shared__ __attribute__((aligned(1024))) char vtile[kTile * D * 2];  // the tile's V rows, 32 KB

  const Tile tile = map_tile(p, true);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int k0 = tile.t0;
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)tile.bh * N;
  const int jmax = key_limit(p, b);

  // Queries that can see a key of [k0, k0 + kTile).
  int qbeg = 0, qend = N;
  if (p.causal) qbeg = k0;
  if (p.window > 0) {
    qbeg = max(qbeg, k0 - p.window + 1);
    qend = min(qend, k0 + kTile - 1 + p.window);
  }
  if (k0 >= jmax) qend = qbeg;  // every key of the tile is padding
  const int qb_lo = qbeg / kQb;
  const int nblk = qend > qbeg ? (qend + kQb - 1) / kQb - qb_lo : 0;

  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + head * D), 0, N * D * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.dout + head * D), 0, N * D * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.lse2 + head), 0, N * 4, kBufDword3);
  const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.delta + head), 0, N * 4, kBufDword3);
  // Stored dS of this head (< 2^31 bytes, checked by the host).
  const int ds_hbytes = kStoreDs ? p.nqb * p.span * (kDsTile * kDsTile * 2) : 0;
  const __amdgpu_buffer_rsrc_t dsrs = __builtin_amdgcn_make_buffer_rsrc(
      kStoreDs ? (void*)(p.ds + (size_t)tile.bh * p.nqb * p.span * (kDsTile * kDsTile)) : nullptr, 0, ds_hbytes,
      kBufDword3);
  auto store_ds = [&](int off, const bf16x8 (&v)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[t]), dsrs, off + (16 * t + 8 * hf) * 2, 0,
                                             kCpolNT);
  };
  auto load_block = [&](int j, char* qd, char* gd, float* sd) {
    const int r0 = (qb_lo + j) * kQb;
    stage_rows<8>(qrs, qd, r0, N, w, lane);
    stage_rows<8>(grs, gd, r0, N, w, lane);
    if (w == 0) {
      // 64 floats from row r0 (the block's 32 and the next 32, unused);
      // rows past N read as 0 (buffer range check).
      // (The row offset goes in the per-lane offset, which the buffer's
      // range check covers.)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)sd, 4, (r0 + lane) * 4, 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)(sd + 64), 4,
                                               (r0 + lane) * 4, 0, 0, 0);
    }
  };
  // K rows of this wave's 32 keys (B operand of S) stay in VGPRs for the
  // whole sweep (rows past N read as 0); the tile's V rows go to LDS.
  const int kj = k0 + 32 * w + l32;
  bf16x8 kreg[NKK];
  {
    const bool ok = kj < N;
    const u32x4* ks = reinterpret_cast<const u32x4*>(p.k + (head + (ok ? kj : 0)) * D + 8 * hf);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kreg[kk] = __builtin_bit_cast(bf16x8, ok ? ks[2 * kk] : u32x4{0, 0, 0, 0});
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + head * D), 0, N * D * 2, kBufDword3);
    stage_rows<32>(vrs, vtile, k0, N, w, lane);
  }
  if (nblk > 0) load_block(0, q0b, g0b, st0);
  bool pending = false;  // a block's dS waits in pend for its store
  int pend_off = 0;
  bf16x8 pend[2];
  const float c = p.c;
  const int ja = k0 + 32 * w, jb = ja + 31;
  const int qrow = perm_key(l32);
  const TrOff tro = tr_offsets(lane);

  f32x16 acck[NMD], accv[NMD];  // dK^T, dV^T
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acck[md][r] = 0.0f;
      accv[md][r] = 0.0f;
    }

  // Fragment offsets from four bases: under the XOR swizzle, chunk 2 kk + hf
  // of a row is at kv_off(row, hf) ^ 32 kk, and the transposed read of
  // column group md at its md = 0 offset ^ 64 md.
  const int rbase = kv_off(qrow, hf), vbase = kv_off(32 * w + l32, hf);
  const int tbase0 = tro.off[0][0], tbase1 = tro.off[1][0];
  auto block = [&](int j, const char* ql, const char* gl, const float* sl) {
    const int i0 = (qb_lo + j) * kQb;
    if (!any_visible(p, jmax, i0, i0 + kQb - 1, ja, jb)) return;
    // The block's 32 A operands in MFMA order -- S and dP alternate over the
    // 8 k-steps (Q rows, dO rows), then dO transposed (dV^T) and Q
    // transposed (dK^T) -- with RA in flight, and the V rows (B operand of
    // dP) with RV in flight.  The empty asm makes the bases new values each
    // block, so the XORs stay beside their reads instead of 24 offsets
    // living in registers across the loop.
    int rb = rbase, vb = vbase, tb0 = tbase0, tb1 = tbase1;
    asm volatile("" : "+v"(rb), "+v"(vb), "+v"(tb0), "+v"(tb1));
    auto trf = [&](const char* blk, int md, int g) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(blk + (tb0 ^ (md << 6)) + 4096 * g));
      const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(blk + (tb1 ^ (md << 6)) + 4096 * g));
      const s16x8 hv = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      return __builtin_bit_cast(bf16x8, hv);
    };
    auto afrag = [&](int i) -> bf16x8 {
      if (i < 16) return *reinterpret_cast<const bf16x8*>(((i & 1) ? gl : ql) + (rb ^ ((i >> 1) << 5)));
      if (i < 24) return trf(gl, (i - 16) >> 1, i & 1);
      return trf(ql, (i - 24) >> 1, i & 1);
    };
    auto vfrag = [&](int kk) -> bf16x8 { return *reinterpret_cast<const bf16x8*>(vtile + (vb ^ (kk << 5))); };
    bf16x8 fa[RA], fv[RV];
#pragma unroll
    for (int i = 0; i < RA; ++i) fa[i] = afrag(i);
#pragma unroll
    for (int i = 0; i < RV; ++i) fv[i] = vfrag(i);
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.0f;
      dp[r] = 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[(2 * kk) % RA], kreg[kk], s, 0, 0, 0);
      fa[(2 * kk) % RA] = afrag(2 * kk + RA);
      __builtin_amdgcn_sched_barrier(0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[(2 * kk + 1) % RA], fv[kk % RV], dp, 0, 0, 0);
      fa[(2 * kk + 1) % RA] = afrag(2 * kk + 1 + RA);
      if (kk + RV < NKK) fv[kk % RV] = vfrag(kk + RV);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Register r holds query i0 + 16 (r / 8) + 8 hf + r % 8 of key kj.
    mask_klane(p, jmax, N, kj, ja, jb, hf, s, i0);
    // B operands: P (for dV) and dS = P (dP - D) (for dK), bf16.
    bf16x8 pb[2], pv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(sl + 16 * t + 8 * hf);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(sl + 16 * t + 8 * hf + 4);
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(sl + 64 + 16 * t + 8 * hf);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(sl + 64 + 16 * t + 8 * hf + 4);
      f32x8 f, fp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * t + e;
        const float l2 = e < 4 ? l0[e] : l1[e - 4];
        const float pr = fast_exp2(fmaf(s[r], c, -l2));
        const float dl = e < 4 ? d0[e] : d1[e - 4];
        fp[e] = pr;
        f[e] = pr * (dp[r] - dl);
      }
      pb[t] = __builtin_convertvector(f, bf16x8);
      pv[t] = __builtin_convertvector(fp, bf16x8);
    }
    // Stored-dS path: this block's dS (32 keys x 32 queries, key-major) for
    // its tile slot; lane (key l32, half hf) holds queries 16 t + 8 hf .. + 7.
    if constexpr (kStoreDs) {
      const int qb = i0 / kDsTile;
      pend_off = ((qb * p.span + ja / kDsTile - ds_first(qb, p.window)) * (kDsTile * kDsTile) + l32 * kDsTile) * 2;
      pend[0] = pb[0];
      pend[1] = pb[1];
      pending = true;
    }
    // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per MFMA.
#pragma unroll
    for (int i = 16; i < 32; ++i) {
      const int md = (i & 7) >> 1;
      if (i < 24)
        accv[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i % RA], pv[i & 1], accv[md], 0, 0, 0);
      else
        acck[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i % RA], pb[i & 1], acck[md], 0, 0, 0);
      if (i + RA < 32) fa[i % RA] = afrag(i + RA);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // With stored dS a block's dS is stored at the start of the next
  // iteration, after its wait and barrier: the wait for a block's loads
  // (vmcnt counts stores too) then finds the stores a whole block old
  // instead of just issued.
  auto iter = [&](int j, const char* ql, const char* gl, const float* sl, char* qn, char* gn, float* sn) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if constexpr (kStoreDs) {
      if (pending) store_ds(pend_off, pend);
      pending = false;
    }
    if (j + 1 < nblk) load_block(j + 1, qn, gn, sn);
    block(j, ql, gl, sl);
  };
  // Two blocks per trip, one call site per buffer (see bwd_dq_kernel).
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    iter(j, q0b, g0b, st0, q1b, g1b, st1);
    iter(j + 1, q1b, g1b, st1, q0b, g0b, st0);
  }
  if (j < nblk) iter(j, q0b, g0b, st0, q1b, g1b, st1);
  if constexpr (kStoreDs) {
    if (pending) store_ds(pend_off, pend);
  }
  // No load into LDS may still be in flight when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // dK, then dV, rows through this wave's quarter of the V tile, once every
  // wave is past its last read of it.
  __syncthreads();
  char* reg = vtile + w * (32 * D * 2);
  store_rows(reg, acck, p.scale, p.dk + head * D, k0 + 32 * w, N, lane);
  store_rows(reg, accv, 1.0f, p.dv + head * D, k0 + 32 * w, N, lane);
}

// ---------------------------------------------------------------------------
// Stored-dS path.  bwd_dkdv_kernel also writes each visible block's dS (the
// tiles of launch.h), and dQ = scale dS K becomes a product over the stored
// tiles instead of a second pass computing S and dP: 4d FLOPs per visible
// pair fewer.  D and LSE log2(e), which bwd_dkdv_kernel needs first, come
// from bwd_prep_kernel.
// ---------------------------------------------------------------------------

// D_i = sum_d dO_id O_id and LSE_i log2(e) (+inf for a row with no key): the
// lanes, products and sums of bwd_dq_kernel's prologue, so both paths use the
// same values.  Each lane loads its own 16-byte pieces of O and dO (piece
// 2 kk + hf of its row, the piece bwd_dq_kernel reads from LDS for kk) and
// sums them in that order; no LDS, so many waves per CU keep loads in flight.
__global__ __launch_bounds__(kT) void bwd_prep_kernel(BwdParams p) {
  const Tile tile = map_tile(p, false);
  if (!tile.valid) return;
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)tile.bh * N;
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)(p.o + head * D), 0, N * D * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.dout + head * D), 0, N * D * 2, kBufDword3);
  const int qi = tile.t0 + 32 * w + l32;
  const bool qok = qi < N;
  const int row = qok ? qi : N - 1;  // rows past N read row N - 1 (not stored below)
  u32x4 a[NKK], g[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int off = (row * D + 8 * (2 * kk + hf)) * 2;
    a[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, off, 0, 0));
    g[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0));
  }
  const float lse_in = qok ? p.lse[head + qi] : kNegInf;
  float dlt = 0.0f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dlt = fmaf(bf16_lo(a[kk][e]), bf16_lo(g[kk][e]), dlt);
      dlt = fmaf(bf16_hi(a[kk][e]), bf16_hi(g[kk][e]), dlt);
    }
  }
  dlt = sum_halves(dlt);
  const float lse2 = lse_in == kNegInf ? __builtin_huge_valf() : lse_in * kLog2e;
  if (qok && hf == 0) {
    p.delta[head + qi] = dlt;
    p.lse2[head + qi] = lse2;
  }
}

// dQ^T += K^T dS^T over the stored tiles.  A workgroup of 4 waves owns
// kDqsTile queries, 32 kDqsQg per wave, and walks its key range in blocks of
// 64.  The operands come from LDS: K^T (transposed reads of the K block, the
// same for every wave) and dS^T (transposed reads of the wave's own
// queries).  With kDqsQg = 2 a wave reads each K^T fragment once for two
// MFMAs but the workgroup is alone on its CU (96 KB of LDS, one wave per
// SIMD); kDqsQg = 1 runs two workgroups per CU, whose prologues and
// epilogues overlap the other's loop, which measured faster.  The stored
// dS is streamed from HBM once, by non-temporal loads that leave K in L2.
// Each wave holds its 16-byte pieces of the next two blocks (K rows, then
// dS) in a ring of registers; while it multiplies block j it writes block
// j + 1 from the ring to the other LDS stage (the swizzled block layout: K,
// then dS for queries 0..127 (and 128..255)), one piece per MFMA pair, and
// reloads each piece's registers with block j + 3.  A tile no query of its
// block sees is loaded from past the end of the buffer and reads as zeros.
// Every accumulator takes its key groups in the order of bwd_dq_kernel.
constexpr int kDqsWaves = 4;
constexpr int kDqsQg = 1;                          // 32-query groups per wave
constexpr int kDqsTile = 32 * kDqsQg * kDqsWaves;  // queries per workgroup
constexpr int kDqsRing = 2;                        // ring slots (blocks) per wave
constexpr int kDqsHalves = kDqsTile / 128;         // LDS dS halves of 128 queries
__global__ __launch_bounds__(64 * kDqsWaves, 3 - kDqsHalves) void bwd_dqs_kernel(BwdParams p) {
  constexpr int BLK = kBc * D * 2;                      // 16 KB
  constexpr int KLOADS = 16 / kDqsWaves;                // 16-byte K pieces per lane per block
  constexpr int SLOADS = 16 * kDqsHalves / kDqsWaves;   // 16-byte dS pieces per lane per block
  constexpr int AHEAD = 4;                              // K^T fragments in flight
  static_assert(kDqsHalves == 1 || kDqsHalves == 2, "one or two LDS halves of 128 queries");
  // Two LDS stages of (K block, dS for queries 0..127 (, 128..255)).
  __shared__ __attribute__((aligned(1024))) char k0[BLK], k1[BLK];
  __shared__ __attribute__((aligned(1024))) char s0[kDqsHalves * BLK], s1[kDqsHalves * BLK];

  const Tile tile = map_tile(p, false, kDqsTile);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.t0;
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)tile.bh * N;
  const int jmax = key_limit(p, b);

  // Key range of the tile (as bwd_dq_kernel, for its kDqsTile queries).
  int kend = jmax;
  if (p.causal) kend = min(kend, q0 + kDqsTile);
  if (p.window > 0 && !p.causal) kend = min(kend, q0 + kDqsTile - 1 + p.window);
  const int kbeg = p.window > 0 ? max(0, q0 - p.window + 1) : 0;
  const int kb_lo = kbeg / kBc;
  const int nblk = kend > kbeg ? (kend + kBc - 1) / kBc - kb_lo : 0;

  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + head * D), 0, N * D * 2, kBufDword3);
  const int hbytes = p.nqb * p.span * (kDsTile * kDsTile * 2);  // < 2^31 (checked by the host)
  const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.ds + (size_t)tile.bh * p.nqb * p.span * (kDsTile * kDsTile)), 0, hbytes, kBufDword3);

  // Piece t of a block for this lane: K row 4 u + lane / 16 (u = w + 4 t),
  // or dS unit u = w + 4 t (half u / 16, key rows 4 (u % 16) + lane / 16);
  // LDS position lane % 16 of the row holds chunk (lane % 16) ^ swz(row).
  // Per dS piece the query block and the key rows are fixed; a key block
  // only moves the 32-key tile, so the offset is base + 2048 (tile index)
  // and visibility is a range of the tile's first key.
  int sbase[SLOADS], slo[SLOADS], shi[SLOADS];
#pragma unroll
  for (int t = 0; t < SLOADS; ++t) {
    const int u = w + kDqsWaves * t;
    const int row = 4 * (u & 15) + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    const int qb = q0 / kDsTile + 4 * (u >> 4) + (c >> 2);
    const int qa = kDsTile * qb, qz = qa + kDsTile - 1;
    // A 32-key tile starting at ja is seen by some query of [qa, qz] iff
    // ja < jmax, causal: ja <= qz, window: qa - (ja + 31) < W and
    // (non-causal) ja - qz < W.
    int hi = jmax - 1;
    if (p.causal) hi = min(hi, qz);
    else if (p.window > 0) hi = min(hi, qz + p.window - 1);
    if (qb >= p.nqb) hi = -1;
    shi[t] = hi;
    slo[t] = p.window > 0 ? qa - kDsTile + 2 - p.window : 0;
    sbase[t] = ((qb * p.span - ds_first(qb, p.window)) * (kDsTile * kDsTile) + (row % kDsTile) * kDsTile + 8 * (c & 3)) * 2 +
               (row / kDsTile) * (kDsTile * kDsTile * 2);
  }
  u32x4 kr[kDqsRing][KLOADS], sr[kDqsRing][SLOADS];
  // A block at or past nblk (the ring runs up to three ahead) loads from
  // past the end of the buffer: zeros, with no memory access to wait for.
  auto load_k = [&](int j, int t) {
    const int row = 4 * (w + kDqsWaves * t) + (lane >> 4);
    const int grow = min((kb_lo + j) * kBc + row, N - 1);
    const int off = j < nblk ? (grow * D + 8 * ((lane & 15) ^ swz(row))) * 2 : N * D * 2;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
  };
  auto load_s = [&](int j, int t) {
    const int j0 = (kb_lo + j) * kBc;
    const int ja = j0 + ((4 * ((w + kDqsWaves * t) & 15) + (lane >> 4)) & kDsTile);  // first key of the lane's tile
    const bool vis = (ja >= slo[t]) & (ja <= shi[t]);
    const unsigned off = vis ? (unsigned)sbase[t] + (unsigned)j0 * (kDsTile * 2) : (unsigned)hbytes;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(drs, (int)off, 0, kCpolNT));
  };
  auto fetch = [&](int j, u32x4 (&kd)[KLOADS], u32x4 (&sd)[SLOADS]) {
#pragma unroll
    for (int t = 0; t < KLOADS; ++t) kd[t] = load_k(j, t);
#pragma unroll
    for (int t = 0; t < SLOADS; ++t) sd[t] = load_s(j, t);
  };
  // Piece pc (K pieces first, then dS) of the block in ring slot `slot`:
  // written to LDS stage (kl, sl), then the slot's piece is reloaded with
  // block jn.
  auto move = [&](int pc, u32x4 (&kd)[KLOADS], u32x4 (&sd)[SLOADS], char* kl, char* sl, int jn) __attribute__((always_inline)) {
    if (pc < KLOADS) {
      *reinterpret_cast<u32x4*>(kl + (w + kDqsWaves * pc) * 1024 + lane * 16) = kd[pc];
      kd[pc] = load_k(jn, pc);
    } else {
      const int t = pc - KLOADS;
      *reinterpret_cast<u32x4*>(sl + (w + kDqsWaves * t) * 1024 + lane * 16) = sd[t];
      sd[t] = load_s(jn, t);
    }
  };

  const int qa = q0 + 32 * kDqsQg * w, qz = qa + 32 * kDqsQg - 1;
  const TrOff tro = tr_offsets(lane);
  // dS^T read offsets of query group qg of the wave: queries
  // o = 32 (kDqsQg w + qg) of the tile are column group (o / 32) % 4 of
  // half o / 128.
  int soff[kDqsQg][2];
  {
    const int tr_g = lane >> 4, tr_j = lane & 15;
    const int rowoff = 8 * (tr_g >> 1) + (tr_j >> 2);
    const int col = 16 * (tr_g & 1) + 4 * (tr_j & 3);
#pragma unroll
    for (int qg = 0; qg < kDqsQg; ++qg)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        soff[qg][r] = ((kDqsQg * w + qg) >> 2) * BLK + kv_off(4 * r + rowoff, (32 * ((kDqsQg * w + qg) & 3) + col) >> 3) +
                      (tr_j & 1) * 8;
  }
  auto sfrag = [&](const char* blk, int qg, int g) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x4 h[2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
      h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(blk + soff[qg][r] + 4096 * g));
    const s16x8 hv = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, hv);
  };
  f32x16 acc[kDqsQg][NMD];
#pragma unroll
  for (int qg = 0; qg < kDqsQg; ++qg)
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qg][md][r] = 0.0f;

  // The MFMAs of block j (stage kl, sl) with the 12 pieces of the next
  // block moved to the other stage between them, one per MFMA pair.  A wave
  // that sees none of block j skips the reads and MFMAs but moves the same
  // pieces in the same order: one path for the loads, so that the compiler
  // keeps the ring in the same registers.
  constexpr int NPC = KLOADS + SLOADS;
  static_assert(NPC <= 16, "one piece per MFMA pair");
  auto block = [&](int j, const char* kl, const char* sl, u32x4 (&kd)[KLOADS], u32x4 (&sd)[SLOADS], char* kn, char* sn,
                   int jn) __attribute__((always_inline)) {
    const int j0 = (kb_lo + j) * kBc;
    const bool vis = any_visible(p, jmax, qa, qz, j0, j0 + kBc - 1);
    bf16x8 bs[kDqsQg][4];
    bf16x8 fk[AHEAD];
    if (vis) {
#pragma unroll
      for (int qg = 0; qg < kDqsQg; ++qg) bs[qg][0] = sfrag(sl, qg, 0);
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) fk[i] = tr_frag(kl, tro, i & 3, i >> 2);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int g = i >> 2, md = i & 3;
      if (vis) {
        if (md == 0 && g < 3) {  // dS^T of the next key group, four steps ahead
#pragma unroll
          for (int qg = 0; qg < kDqsQg; ++qg) bs[qg][g + 1] = sfrag(sl, qg, g + 1);
        }
#pragma unroll
        for (int qg = 0; qg < kDqsQg; ++qg)
          acc[qg][md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[i % AHEAD], bs[qg][g], acc[qg][md], 0, 0, 0);
        if (i + AHEAD < 16) fk[i % AHEAD] = tr_frag(kl, tro, (i + AHEAD) & 3, (i + AHEAD) >> 2);
      }
      if (i < NPC) move(i, kd, sd, kn, sn, jn);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One workgroup barrier per block: before it, every wave's LDS writes of
  // the next block are done (lgkmcnt(0)) and its reads of the current one
  // were consumed by MFMAs.  It is a bare s_barrier between wavefront-scope
  // fences: __syncthreads' workgroup fence would also wait for every load in
  // flight in the register ring.
  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt left at their maxima
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Block b sits in ring slot b % 2.  Iteration j multiplies block j (stage
  // j % 2) and moves block j + 1 from slot (j + 1) % 2 to stage (j + 1) % 2,
  // refilling the slot with block j + 3.  The loop runs an even number of
  // iterations; one past nblk moves and reads blocks no query sees.
  static_assert(kDqsRing == 2, "block j + 1 sits in slot (j + 1) % 2");
  auto iter = [&](int j, auto step_c) {
    constexpr bool odd = decltype(step_c)::value;  // j % 2
    constexpr int SN = odd ? 0 : 1;                // slot of block j + 1
    block(j, odd ? k1 : k0, odd ? s1 : s0, kr[SN], sr[SN], odd ? k0 : k1, odd ? s0 : s1, j + kDqsRing + 1);
    barrier();
  };
  if (nblk > 0) {
#pragma unroll
    for (int i = 0; i < kDqsRing; ++i) fetch(i, kr[i], sr[i]);
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) move(pc, kr[0], sr[0], k0, s0, kDqsRing);
    barrier();
    for (int j = 0; j < nblk; j += 2) {
      iter(j, std::integral_constant<int, 0>());
      iter(j + 1, std::integral_constant<int, 1>());
    }
  }

  // dQ rows through LDS: a lane holds 8-byte pieces of one query row
  // (elements 32 md + 8 rq + 4 hf .. + 3), which stored directly would be
  // 16-byte runs scattered over 32 rows per instruction.  Each wave writes
  // its rows (32 per query group, swizzled block layout) to a region of its
  // own, past the loop's last barrier, and stores them back as whole
  // 256-byte rows.
  static_assert(kDqsWaves == 4 && 32 * kDqsQg * D * 2 * 2 == kDqsHalves * BLK, "two wave regions per LDS stage");
  char* reg = (w < 2 ? s0 : s1) + (w & 1) * (32 * kDqsQg * D * 2);
#pragma unroll
  for (int qg = 0; qg < kDqsQg; ++qg)
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 wv;
        wv[0] = pack_bf16x2(acc[qg][md][4 * rq + 0] * p.scale, acc[qg][md][4 * rq + 1] * p.scale);
        wv[1] = pack_bf16x2(acc[qg][md][4 * rq + 2] * p.scale, acc[qg][md][4 * rq + 3] * p.scale);
        *reinterpret_cast<u32x2*>(reg + kv_off(32 * qg + l32, 4 * md + rq) + 8 * hf) = wv;
      }
  constexpr int NT = 32 * kDqsQg / 4;  // 4 rows per instruction
  u32x4 rows[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) rows[t] = *reinterpret_cast<const u32x4*>(reg + kv_off(4 * t + (lane >> 4), lane & 15));
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int qi = qa + 4 * t + (lane >> 4);
    if (qi < N) *reinterpret_cast<u32x4*>(p.dq + (head + qi) * D + 8 * (lane & 15)) = rows[t];
  }
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const __bf16*>(a.q);
  p.k = static_cast<const __bf16*>(a.k);
  p.v = static_cast<const __bf16*>(a.v);
  p.o = static_cast<const __bf16*>(a.o);
  p.dout = static_cast<const __bf16*>(a.dout);
  p.lse = a.lse;
  const size_t rows = (size_t)a.B * a.H * a.N;
  p.delta = a.ws;
  p.lse2 = a.ws + rows;
  p.dq = static_cast<__bf16*>(a.dq);
  p.dk = static_cast<__bf16*>(a.dk);
  p.dv = static_cast<__bf16*>(a.dv);
  p.kv_len = a.kv_len;
  p.B = a.B;
  p.H = a.H;
  p.N = a.N;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  p.causal = a.causal;
  // |i - j| <= N - 1 always, so a window beyond N masks nothing; clamping it
  // keeps every bound below int range.
  p.window = a.window > a.N ? a.N : a.window;
  p.n_tiles = (a.N + kTile - 1) / kTile;
  p.total = a.B * a.H * p.n_tiles;
  p.ds = static_cast<__bf16*>(a.ds);
  p.nqb = (a.N + kDsTile - 1) / kDsTile;
  p.span = (int)ds_span(a.N, a.causal, p.window);
  const unsigned grid = (unsigned)((p.total + 7) / 8 * 8);
  if (p.ds) {
    // D and LSE log2(e); dK, dV and the dS tiles; dQ from the tiles.
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(grid), dim3(kT), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3(grid), dim3(kT), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    BwdParams pq = p;  // 256-query tiles
    pq.n_tiles = (a.N + kDqsTile - 1) / kDqsTile;
    pq.total = a.B * a.H * pq.n_tiles;
    hipLaunchKernelGGL(bwd_dqs_kernel, dim3((unsigned)((pq.total + 7) / 8 * 8)), dim3(64 * kDqsWaves), 0, stream, pq);
    return hipGetLastError();
  }
  // dQ first: it also writes D and LSE log2(e), which bwd_dkdv_kernel reads.
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(grid), dim3(kT), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3(grid), dim3(kT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace osfa
