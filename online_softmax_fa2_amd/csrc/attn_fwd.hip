// Fused attention forward pass for gfx950: the query-tile online-softmax
// recurrence with causal / sliding-window / padding masks, the
// fully-masked-row guard, FA2's single deferred division and per-row LSE.
//
// Method (page "Online softmax for a whole query tile, matrix form", "A
// strong answer"): a tile of queries keeps per-row m and l and an
// unnormalized accumulator A; for each key block
//     S = scale Q K^T,  m' = max(m, rowmax S),  P = exp(S - m'),
//     l' = alpha l + rowsum P,  A' = diag(alpha) A + P V,  alpha = exp(m - m'),
// with m' replaced by 0 in the exponents of rows that have seen no key yet
// (the guard), and O = diag(l)^-1 A once after the last block.  Blocks that
// no query of the tile can see are skipped before any load (page "Derive
// online softmax, prove it is exact", "Common mistakes": causal skipping).
//
// gfx950 mapping (one workgroup = one query tile of 32 * kWaves rows, each
// wave owns 32 query rows for the whole key sweep, queries outer):
//   * Q rows live in VGPRs for the whole sweep, in MFMA B-operand layout.
//   * K and V blocks of kBc keys are staged through LDS, double buffered;
//     V is stored transposed (d-major) so that each lane reads 8 keys of one
//     d column with a single 16-byte LDS read.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: the accumulator column is the query (lane
//     l holds query l % 32), so a query's row maximum and row sum are a
//     reduction over the lane's own registers plus one exchange between the
//     two 32-lane halves.  The K rows are fed to the MFMA in a permuted order
//     chosen so that each lane's 8 consecutive accumulator registers hold 8
//     consecutive keys: after exp2 and a bf16 conversion they are directly the
//     B operand of the P V MFMA (O^T = V^T P^T), with no LDS round trip.
//   * exp is exp2 with scale * log2(e) folded into one FMA per score; running
//     maxima are in log2 units.
//   * The accumulator O^T keeps the query in the lane too, so diag(alpha) A is
//     a lane-local multiply, skipped when alpha == 1 for the whole wave (the
//     max did not move: exact).
// The float32 path follows the same structure with v_mfma_f32_32x32x2f32 and
// float32 operands in LDS (no transposition needed: each MFMA step consumes
// one key per 32-lane half).
#include "device_common.h"
#include "launch.h"

namespace osfa {
namespace {

constexpr int kBc = 64;           // keys per block
constexpr int kWaves = 4;         // waves per workgroup
constexpr int kBr = 32 * kWaves;  // queries per tile
constexpr int kThreads = 64 * kWaves;
// s_waitcnt immediate for gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;
// Lazy rescale: the reference m_ref of l and A moves only when a block's row
// maximum exceeds it by more than kTau (log2 units), so P = exp2(s - m_ref)
// stays <= 2^kTau.  Exact: O = A / l and LSE = m_ref + log2 l do not depend on
// which common reference was used (page "Online softmax for a whole query
// tile, matrix form", "What interviewers probe next").
constexpr float kTau = 8.0f;
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

// Row m of the S^T MFMA takes key perm_key(m) of the 32-key group: bits 2 and
// 3 swapped.  With the 32x32 accumulator layout (lane l, register r holds row
// 8(r/4) + 4(l/32) + r%4) this puts keys 16(r/8) + 8(l/32) + r%8 in register r.
__device__ __forceinline__ int perm_key(int m) { return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1); }

// ---------------------------------------------------------------------------
// bf16 inputs, MFMA 32x32x16
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdParams p) {
  constexpr int KS = D + 8;           // K row stride in LDS (bf16), +16 B pad
  constexpr int VS = kBc + 8;         // V^T row stride in LDS (bf16), +16 B pad
  constexpr int KEL = kBc * KS;
  constexpr int VEL = D * VS;
  constexpr int BUF = KEL + VEL;
  constexpr int KPT = D / 32;         // key rows each thread stages per block
  constexpr int NKK = D / 16;         // MFMA k-steps over d
  constexpr int NMD = D / 32;         // 32-wide d tiles of the output
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];

  const Tile tile = map_tile(p);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.q0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // which 32-lane half
  const int N = p.N;
  const size_t head_off = (size_t)tile.bh * (size_t)N * D;
  const __bf16* Qg = static_cast<const __bf16*>(p.q) + head_off;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + head_off;
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + head_off;

  // Q rows of this lane: query qi, d = 16 kk + 8 hf + [0, 8).
  const int qi = q0 + 32 * w + l32;
  bf16x8 qreg[NKK];
  {
    const bool ok = qi < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(Qg + (size_t)(ok ? qi : 0) * D + 8 * hf);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = ok ? src[2 * kk] : u32x4{0, 0, 0, 0};
      qreg[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Retire the Q loads here, on every path: otherwise the wait for them is
  // merged into the loop and also blocks on the next block's prefetch.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  const KeyRange kr = key_range(p, b, q0);
  const int kb_lo = kr.kbeg / kBc;
  const int kb_hi = (kr.kend > kr.kbeg) ? (kr.kend + kBc - 1) / kBc : kb_lo;

  // Staging: thread stages KPT consecutive key rows x 8 d values of K and V.
  const int sc = tid % (D / 8);       // d chunk
  const int sk = (tid / (D / 8)) * KPT;  // first key row within the block
  u32x4 kst[KPT], vst[KPT];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      int j = kb * kBc + sk + r;
      j = j < N ? j : N - 1;  // rows past N are masked; read a valid row
      const size_t off = (size_t)j * D + 8 * sc;
      kst[r] = *reinterpret_cast<const u32x4*>(Kg + off);
      vst[r] = *reinterpret_cast<const u32x4*>(Vg + off);
    }
  };
  auto store_block = [&](int buf) {
    __bf16* kl = lds + buf * BUF;
    __bf16* vl = kl + KEL;
#pragma unroll
    for (int r = 0; r < KPT; ++r) *reinterpret_cast<u32x4*>(kl + (sk + r) * KS + 8 * sc) = kst[r];
    // Transpose V: for each of the 8 d values, the KPT keys go contiguous.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t wv[KPT / 2];
#pragma unroll
      for (int r2 = 0; r2 < KPT / 2; ++r2) {
        const uint32_t a = vst[2 * r2][e / 2], c = vst[2 * r2 + 1][e / 2];
        wv[r2] = (e & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      __bf16* dst = vl + (8 * sc + e) * VS + sk;
      if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{wv[0], wv[1]};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = wv[0];
      }
    }
  };

  f32x16 oacc[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
  float m_ref = kNegInf;  // reference of l_run and oacc, log2 units (>= true max - kTau)
  float l_run = 0.0f;     // this half's share of the running normalizer
  const float c = p.c;
  const int krow = perm_key(l32);
  const int qa = q0 + 32 * w, qb = qa + 31;  // this wave's query rows

  if (kb_lo < kb_hi) {
    load_block(kb_lo);
    store_block(0);
  }
  __syncthreads();

  for (int kb = kb_lo; kb < kb_hi; ++kb) {
    const int cur = (kb - kb_lo) & 1;
    const bool has_next = kb + 1 < kb_hi;
    if (has_next) load_block(kb + 1);

    const __bf16* kl = lds + cur * BUF;
    const __bf16* vl = kl + KEL;
    const int j0 = kb * kBc;

    if (rows_see_block(p, kr.jmax, qa, qb, j0)) {
      // S^T = K Q^T for two 32-key groups; the K fragments of a group are
      // read from LDS ahead of its MFMA chain.
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 kf[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          kf[kk] = *reinterpret_cast<const bf16x8*>(kl + (32 * kt + krow) * KS + 16 * kk + 8 * hf);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qreg[kk], s[kt], 0, 0, 0);
      }

      if (!rows_see_all(p, kr.jmax, qa, qb, j0)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + 32 * kt + 16 * (r >> 3) + 8 * hf + (r & 7);
            if (!visible(p, kr.jmax, qi, j)) s[kt][r] = kNegInf;
          }
      }

      // Row max of this block: the lane's 32 keys, then the other half's.
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
      const float mblk = max_halves(mx) * c;
      const bool move = mblk > m_ref + kTau;  // true for the first visible block (m_ref = -inf)
      if (__any(move)) {
        // Lanes that do not move keep alpha = 1 exactly: a lane that has seen
        // no key yet (m_ref = -inf) must not form exp2(-inf - (-inf)) = NaN.
        const float alpha = move ? fast_exp2(m_ref - mblk) : 1.0f;  // 0 when moving from -inf
        const float m_new = move ? mblk : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < NMD; ++md)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
        m_ref = m_new;
      }
      const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;  // guard: a row with no key yet
      float rs = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(s[kt][r], c, -mr));
          s[kt][r] = e;
          rs += e;
        }
      l_run += rs;

      // P^T as the B operand: registers 8t..8t+7 of group kt hold keys
      // 32 kt + 16 t + 8 hf + [0, 8).
      bf16x8 pb[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = s[kt][8 * t + e];
          pb[kt][t] = __builtin_convertvector(f, bf16x8);
        }

      // O^T += V^T P^T.
#pragma unroll
      for (int md = 0; md < NMD; ++md) {
        bf16x8 vf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vf[i] = *reinterpret_cast<const bf16x8*>(vl + (32 * md + l32) * VS + 16 * i + 8 * hf);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pb[i >> 1][i & 1], oacc[md], 0, 0, 0);
      }
    }

    if (has_next) store_block(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: one division per row (FA2), bf16 O, LSE in natural-log units.
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qi < N) {
    __bf16* Og = static_cast<__bf16*>(p.o) + head_off + (size_t)qi * D;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dcol = 32 * md + 8 * rq + 4 * hf;
        u32x2 wv;
        wv[0] = pack_bf16x2(oacc[md][4 * rq + 0] * inv, oacc[md][4 * rq + 1] * inv);
        wv[1] = pack_bf16x2(oacc[md][4 * rq + 2] * inv, oacc[md][4 * rq + 3] * inv);
        *reinterpret_cast<u32x2*>(Og + dcol) = wv;
      }
    if (hf == 0)
      p.lse[(size_t)tile.bh * N + qi] = l_tot > 0.0f ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs, d = 128: direct-to-LDS loads, swizzled LDS, transposed V reads
//
// K and V blocks (64 keys x 256 B each) are copied from global memory into
// LDS by global_load_lds_dwordx4 (16 B per lane, no VGPR staging), STAGES
// deep, one barrier per block.  Each load instruction fills 1 KB of LDS =
// 4 key rows in lane order; the lane fetches whichever 16-byte chunk belongs
// at its LDS slot under the layout
//     byte(row, chunk) = row * 256 + ((chunk ^ f(row)) * 16),
//     f(row) = ((row & 3) << 2) | ((row >> 2) & 3),
// an XOR swizzle under which the K-fragment reads (32 rows, one chunk) and
// the V^T transposed reads (8 rows x 64 B) both touch every LDS bank once.
// V stays row-major in LDS; ds_read_b64_tr_b16 returns, in each group of 16
// lanes, lane i's 4 values from the 4 chunks addressed by lanes 4e + i/4,
// element i % 4, so that a lane receives 4 consecutive keys of one d column:
// two such reads form the 8-key A operand of the P V MFMA.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int kv_off(int row, int chunk) { return row * 256 + ((chunk ^ swz(row)) << 4); }

template <int NW>
__global__ __launch_bounds__(64 * NW, (NW == 4 ? 2 : 1)) void fwd_bf16_d128_kernel(FwdParams p) {
  constexpr int D = 128;
  constexpr int BLK_BYTES = kBc * D * 2;         // one K or V block: 16 KB
  constexpr int STAGE_BYTES = 2 * BLK_BYTES;     // K then V
  constexpr int LOADS_PER_WAVE = 32 / NW;        // 16 K + 16 V instructions per block
  constexpr int NKK = D / 16;
  constexpr int NMD = D / 32;
  // Two stages as two distinct LDS objects: alias analysis can then tell the
  // in-flight LDS-DMA writes into one stage from the reads of the other, so
  // the reads do not wait for the prefetch.
  __shared__ __attribute__((aligned(1024))) char lds0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds1[STAGE_BYTES];

  const Tile tile = map_tile(p);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.q0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int N = p.N;
  const size_t head_off = (size_t)tile.bh * (size_t)N * D;
  const __bf16* Qg = static_cast<const __bf16*>(p.q) + head_off;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + head_off;
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + head_off;

  const KeyRange kr = key_range(p, b, q0);
  const int kb_lo = kr.kbeg / kBc;
  const int kb_hi = (kr.kend > kr.kbeg) ? (kr.kend + kBc - 1) / kBc : kb_lo;
  const int nblk = kb_hi - kb_lo;

  // This wave's share of the 32 load instructions of block kb, into `stage`.
  auto issue_block = [&](int kb, char* stage) {
#pragma unroll
    for (int t = 0; t < LOADS_PER_WAVE; ++t) {
      const int ii = w + NW * t;
      const bool isv = ii >= 16;
      const int i = ii & 15;
      const int row = 4 * i + (lane >> 4);
      const int chunk = (lane & 15) ^ swz(row);
      int j = kb * kBc + row;
      j = j < N ? j : N - 1;  // rows past N are masked; read a valid row
      const __bf16* src = (isv ? Vg : Kg) + (size_t)j * D + 8 * chunk;
      __builtin_amdgcn_global_load_lds(src, stage + (isv ? BLK_BYTES : 0) + i * 1024, 16, 0, 0);
    }
  };

  if (nblk > 0) issue_block(kb_lo, lds0);

  const int qi = q0 + 32 * w + l32;
  bf16x8 qreg[NKK];
  {
    const bool ok = qi < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(Qg + (size_t)(ok ? qi : 0) * D + 8 * hf);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = ok ? src[2 * kk] : u32x4{0, 0, 0, 0};
      qreg[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 oacc[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
  float m_ref = kNegInf;  // reference of l_run and oacc, log2 units
  float l_run = 0.0f;
  const float c = p.c;
  const int qa = q0 + 32 * w, qb = qa + 31;
  const int krow = perm_key(l32);
  // V^T transposed-read source address pieces for this lane.
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int tr_rowoff = 8 * (tr_g >> 1) + (tr_j >> 2);  // + 16 i + 4 r
  const int tr_col = 16 * (tr_g & 1) + 4 * (tr_j & 3);   // + 32 md
  const int tr_byte = (tr_j & 1) * 8;

  // One block: wait for its loads, barrier, prefetch the next block into the
  // other stage, compute from this stage.
  auto step = [&](int it, const char* cur, char* nxt) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (it + 1 < nblk) issue_block(kb_lo + it + 1, nxt);

    const char* kl = cur;
    const char* vl = cur + BLK_BYTES;
    const int j0 = (kb_lo + it) * kBc;
    if (!rows_see_block(p, kr.jmax, qa, qb, j0)) return;

    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8 kf[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8*>(kl + kv_off(32 * kt + krow, 2 * kk + hf));
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qreg[kk], s[kt], 0, 0, 0);
    }

    if (!rows_see_all(p, kr.jmax, qa, qb, j0)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kt + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (!visible(p, kr.jmax, qi, j)) s[kt][r] = kNegInf;
        }
    }

    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    const float mblk = max_halves(mx) * c;
    const bool move = mblk > m_ref + kTau;
    if (__any(move)) {
      // Lanes that do not move keep alpha = 1 exactly: a lane that has seen
      // no key yet (m_ref = -inf) must not form exp2(-inf - (-inf)) = NaN.
      const float alpha = move ? fast_exp2(m_ref - mblk) : 1.0f;  // 0 when moving from -inf
      const float m_new = move ? mblk : m_ref;
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
      m_ref = m_new;
    }
    const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;
    float rs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(s[kt][r], c, -mr));
        s[kt][r] = e;
        rs += e;
      }
    l_run += rs;

    bf16x8 pb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = s[kt][8 * t + e];
        pb[kt][t] = __builtin_convertvector(f, bf16x8);
      }

    // O^T += V^T P^T; V^T fragments by two transposed LDS reads each.
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int md = 0; md < NMD; ++md) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s16x4 h[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const char* a = vl + kv_off(16 * i + 4 * r + tr_rowoff, (32 * md + tr_col) >> 3) + tr_byte;
          h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
        }
        const s16x8 hv = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hv), pb[i >> 1][i & 1],
                                                          oacc[md], 0, 0, 0);
      }
    }
  };

  for (int it = 0; it < nblk; it += 2) {
    step(it, lds0, lds1);
    if (it + 1 < nblk) step(it + 1, lds1, lds0);
  }

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qi < N) {
    __bf16* Og = static_cast<__bf16*>(p.o) + head_off + (size_t)qi * D;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dcol = 32 * md + 8 * rq + 4 * hf;
        u32x2 wv;
        wv[0] = pack_bf16x2(oacc[md][4 * rq + 0] * inv, oacc[md][4 * rq + 1] * inv);
        wv[1] = pack_bf16x2(oacc[md][4 * rq + 2] * inv, oacc[md][4 * rq + 3] * inv);
        *reinterpret_cast<u32x2*>(Og + dcol) = wv;
      }
    if (hf == 0)
      p.lse[(size_t)tile.bh * N + qi] = l_tot > 0.0f ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// float32 inputs, MFMA 32x32x2 f32 (single-buffered; a correctness-first path)
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(FwdParams p) {
  constexpr int RS = D + 4;  // row stride in LDS (floats), +16 B pad
  constexpr int NKK = D / 2;
  constexpr int NMD = D / 32;
  __shared__ __attribute__((aligned(16))) float kl[kBc * RS];
  __shared__ __attribute__((aligned(16))) float vl[kBc * RS];

  const Tile tile = map_tile(p);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.q0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int N = p.N;
  const size_t head_off = (size_t)tile.bh * (size_t)N * D;
  const float* Qg = static_cast<const float*>(p.q) + head_off;
  const float* Kg = static_cast<const float*>(p.k) + head_off;
  const float* Vg = static_cast<const float*>(p.v) + head_off;

  // MFMA step kk pairs d = kk (lower half) with d = kk + D/2 (upper half).
  const int qi = q0 + 32 * w + l32;
  float qreg[NKK];
  {
    const bool ok = qi < N;
    const f32x4* src = reinterpret_cast<const f32x4*>(Qg + (size_t)(ok ? qi : 0) * D + (D / 2) * hf);
#pragma unroll
    for (int i = 0; i < NKK / 4; ++i) {
      f32x4 v = ok ? src[i] : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) qreg[4 * i + e] = v[e];
    }
  }

  const KeyRange kr = key_range(p, b, q0);
  const int kb_lo = kr.kbeg / kBc;
  const int kb_hi = (kr.kend > kr.kbeg) ? (kr.kend + kBc - 1) / kBc : kb_lo;

  f32x16 oacc[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  const float c = p.c;

  for (int kb = kb_lo; kb < kb_hi; ++kb) {
    const int j0 = kb * kBc;
    __syncthreads();  // previous block fully consumed
    for (int idx = tid; idx < kBc * D / 4; idx += kThreads) {
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      int j = j0 + row;
      j = j < N ? j : N - 1;
      *reinterpret_cast<f32x4*>(kl + row * RS + 4 * c4) = *reinterpret_cast<const f32x4*>(Kg + (size_t)j * D + 4 * c4);
      *reinterpret_cast<f32x4*>(vl + row * RS + 4 * c4) = *reinterpret_cast<const f32x4*>(Vg + (size_t)j * D + 4 * c4);
    }
    __syncthreads();

    // S^T for two 32-key groups: lane l, register r holds key
    // 32 kt + 8 (r/4) + 4 hf + r%4 of query qi.
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
      const float* krow = kl + (32 * kt + l32) * RS + (D / 2) * hf;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[kk], qreg[kk], s[kt], 0, 0, 0);
    }
    if (!block_interior(p, kr, q0, j0)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (!visible(p, kr.jmax, qi, j)) s[kt][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_ref = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    float rs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(s[kt][r], c, -m_ref));
        s[kt][r] = e;
        rs += e;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;

    // O^T += V^T P^T, one key per half per MFMA step.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
        for (int md = 0; md < NMD; ++md)
          oacc[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[key * RS + 32 * md + l32], s[kt][r], oacc[md], 0, 0, 0);
      }
  }

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qi < N) {
    float* Og = static_cast<float*>(p.o) + head_off + (size_t)qi * D;
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[md][4 * rq + e] * inv;
        *reinterpret_cast<f32x4*>(Og + 32 * md + 8 * rq + 4 * hf) = v;
      }
    if (hf == 0)
      p.lse[(size_t)tile.bh * N + qi] = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
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
  p.causal = a.causal ? 1 : 0;
  p.window = a.window > 0 ? a.window : 0;
  p.br = br;
  p.n_tiles = (a.N + br - 1) / br;
  p.total = a.B * a.H * p.n_tiles;
  return p;
}

unsigned grid_for(const FwdParams& p) { return (unsigned)((p.total + 7) / 8 * 8); }

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) {
    const FwdParams p = make_params(a, 32 * kV2Waves);
    hipLaunchKernelGGL((fwd_bf16_d128_kernel<kV2Waves>), dim3(grid_for(p)), dim3(64 * kV2Waves), 0, stream, p);
  } else {
    const FwdParams p = make_params(a, kBr);
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid_for(p)), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  const FwdParams p = make_params(a, kBr);
  const dim3 grid(grid_for(p)), block(kThreads);
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace osfa
