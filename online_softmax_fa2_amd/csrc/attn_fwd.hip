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
  int n_tiles;
  int total;  // B * H * n_tiles
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
  t.q0 = tile * kBr;
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
  if (p.causal) kend = min(kend, q0 + kBr);
  if (p.window > 0 && !p.causal) kend = min(kend, q0 + kBr - 1 + p.window);
  r.kend = kend;
  r.kbeg = (p.window > 0) ? max(0, q0 - p.window + 1) : 0;
  return r;
}

// True if every (i, j) with i in the tile and j in [j0, j0 + kBc) is visible.
__device__ __forceinline__ bool block_interior(const FwdParams& p, const KeyRange& r, int q0, int j0) {
  if (j0 + kBc > r.jmax) return false;
  if (p.causal && j0 + kBc - 1 > q0) return false;
  if (p.window > 0) {
    if ((q0 + kBr - 1) - j0 >= p.window) return false;
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
  float m_run = kNegInf;  // running max, log2 units
  float l_run = 0.0f;     // this half's share of the running normalizer
  const float c = p.c;
  const int krow = perm_key(l32);

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

    // S^T = K Q^T for two 32-key groups.
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + (32 * kt + krow) * KS + 16 * kk + 8 * hf);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[kt], 0, 0, 0);
      }
    }

    if (!block_interior(p, kr, q0, j0)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kt + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (!visible(p, kr.jmax, qi, j)) s[kt][r] = kNegInf;
        }
    }

    // Row max of this block (the lane's 32 keys, then the other half's).
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_ref = (m_new == kNegInf) ? 0.0f : m_new;  // guard
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
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
    }

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
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(vl + (32 * md + l32) * VS + 32 * kt + 16 * t + 8 * hf);
          oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][t], oacc[md], 0, 0, 0);
        }

    if (has_next) store_block(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: one division per row (FA2), bf16 O, LSE in natural-log units.
  const float l_tot = l_run + swap_halves(l_run);
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
      p.lse[(size_t)tile.bh * N + qi] = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
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
    mx = fmaxf(mx, swap_halves(mx));
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

  const float l_tot = l_run + swap_halves(l_run);
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

FwdParams make_params(const FwdArgs& a) {
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
  p.n_tiles = (a.N + kBr - 1) / kBr;
  p.total = a.B * a.H * p.n_tiles;
  return p;
}

unsigned grid_for(const FwdParams& p) { return (unsigned)((p.total + 7) / 8 * 8); }

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  const FwdParams p = make_params(a);
  const dim3 grid(grid_for(p)), block(kThreads);
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  const FwdParams p = make_params(a);
  const dim3 grid(grid_for(p)), block(kThreads);
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace osfa
