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
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "fwd_common.h"
#include "tile_layout.h"

namespace osfa {
namespace {

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
  float l_run = 0.0f;     // this half's share of the running normalizer (float32 P: LSE)
  float l_bf = 0.0f;      // the same over the bf16 P that enters P V (divides O)
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
        l_bf *= alpha;
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
      // 32 kt + 16 t + 8 hf + [0, 8).  l_bf sums the bf16 P that enters P V.
      bf16x8 pb[2][2];
      float rb = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = s[kt][8 * t + e];
          pb[kt][t] = __builtin_convertvector(f, bf16x8);
          const u32x4 w4 = __builtin_bit_cast(u32x4, pb[kt][t]);
#pragma unroll
          for (int e = 0; e < 4; ++e) rb = sum_bf16x2(w4[e], rb);
        }
      l_bf += rb;

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
  // O divides by the sum of the bf16 P it accumulated (their rounding
  // cancels in the ratio); LSE takes the float32 sum.
  const float l_tot = sum_halves(l_run);
  const float l_div = sum_halves(l_bf);
  const float inv = l_div > 0.0f ? 1.0f / l_div : 0.0f;
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
// bf16 inputs, d = 128: direct-to-LDS loads, swizzled LDS, transposed V
// reads, software pipelined across key blocks
//
// K and V blocks (64 keys x 256 B each) are copied into LDS by buffer loads
// straight to LDS in the swizzled layout of tile_layout.h, one barrier per
// block.  K fragments are row reads; V stays row-major in LDS and is read
// transposed (ds_read_b64_tr_b16), two reads forming the 8-key A operand of
// the P V MFMA.
//
// One wave's work on consecutive key blocks is overlapped so that the
// exponentials run while the matrix core is busy:
//   phase A of step j:  S_{j+1} = K_{j+1} Q^T (MFMA)   with exp of the second
//                       half of S_j's keys, their row sums and bf16 packing;
//   phase B of step j:  O += V_j P_j (MFMA)            with the mask and row
//                       maximum of S_{j+1}, the reference update and the exp
//                       of the first half of S_{j+1}'s keys.
// Each phase is written as 16 slots of one MFMA plus a few independent VALU
// instructions (sched_barrier keeps the slots in order), so the VALU work
// issues while the MFMA runs.  The factor that rescales the accumulator when
// the reference moves is applied just before the next P V product (the
// accumulator is still being written by P_j V_j when the factor is formed);
// l is rescaled at once.  K and V have separate double buffers: step j reads
// K_{j+1} and V_j and refills the buffers of K_j and V_{j-1} with K_{j+2} and
// V_{j+1}.
// ---------------------------------------------------------------------------


// LDS fragment reads are issued this many MFMA slots ahead of their use.
constexpr int KAHEAD = 4, VAHEAD = 4;
// float32 launches with fewer 128-query tiles than this use the key-split kernel.
constexpr long long kSplitTilesBelow = 256;

// POLY > 0: in every group of POLY consecutive pairs of exponentials of a
// half block, the last pair is computed by exp2_fma (the FMA-pipe
// exponential); POLY = 0: all on v_exp_f32.
template <int NW, int POLY>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_d128_kernel(FwdParams p) {
  constexpr int D = 128;
  constexpr int BLK = kBc * D * 2;  // one K or V block: 16 KB
  constexpr int LOADS = 16 / NW;    // load instructions per wave per block
  constexpr int NKK = D / 16;
  constexpr int NMD = D / 32;
  // Four distinct LDS objects so that alias analysis separates the in-flight
  // direct-to-LDS writes from the reads of the other buffers.
  __shared__ __attribute__((aligned(1024))) char k0[BLK];
  __shared__ __attribute__((aligned(1024))) char k1[BLK];
  __shared__ __attribute__((aligned(1024))) char v0[BLK];
  __shared__ __attribute__((aligned(1024))) char v1[BLK];

  const Tile tile = map_tile(p);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.q0;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  // This wave's share of the 16 load instructions of one K or V block: load
  // t fills LDS bytes [1024 i, 1024 i + 1024), i = w + NW t, i.e. key rows
  // 4 i .. 4 i + 3.  Buffer loads: the head's K (or V) is a buffer resource,
  // the block start a scalar offset and the lane's byte offset in the block
  // is fixed.  (Offsets are passed as int, the builtin's parameter type: an
  // implicit conversion there makes the host pass drop the launch stub.)
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, N * D * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, N * D * 2, kBufDword3);
  const std::integral_constant<bool, false> kIsK;
  const std::integral_constant<bool, true> kIsV;
  int ld_off[LOADS];
#pragma unroll
  for (int t = 0; t < LOADS; ++t) {
    const int row = 4 * (w + NW * t) + (lane >> 4);
    ld_off[t] = (row * D + 8 * ((lane & 15) ^ swz(row))) * 2;
  }
  auto issue = [&](auto is_v, int kb, char* dst) {
    const __amdgpu_buffer_rsrc_t rs = decltype(is_v)::value ? vrs : krs;
    const int soff = kb * kBc * D * 2;
    if (kb * kBc + kBc <= N) {
#pragma unroll
      for (int t = 0; t < LOADS; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (w + NW * t) * 1024),
                                                 16, (int)ld_off[t], (int)soff, 0, 0);
    } else {
      // Last, partial block: rows past N read row N - 1 (they are masked).
#pragma unroll
      for (int t = 0; t < LOADS; ++t) {
        const int row = 4 * (w + NW * t) + (lane >> 4);
        const int over = kb * kBc + row - (N - 1);
        const int off = over > 0 ? ld_off[t] - over * D * 2 : ld_off[t];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (w + NW * t) * 1024),
                                                 16, (int)off, (int)soff, 0, 0);
      }
    }
  };

  if (nblk > 0) {
    issue(kIsK, kb_lo, k0);
    issue(kIsV, kb_lo, v0);
    if (nblk > 1) issue(kIsK, kb_lo + 1, k1);
  }

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
  float m_ref = kNegInf;  // reference of l_run, l_bf and oacc, log2 units
  float l_run = 0.0f;     // running normalizer over the float32 P (LSE)
  float l_bf = 0.0f;      // the same over the bf16 P that enters P V (divides O)
  float pend_alpha = 1.0f;  // factor still to be applied to oacc
  bool pend = false;
  const float c = p.c;
  const int qa = q0 + 32 * w, qb = qa + 31;
  const int krow = perm_key(l32);
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int tr_rowoff = 8 * (tr_g >> 1) + (tr_j >> 2);
  const int tr_col = 16 * (tr_g & 1) + 4 * (tr_j & 3);
  const int tr_byte = (tr_j & 1) * 8;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

  // S^T = K Q^T for the block in `kl` (MFMA only, K fragments from LDS).
  auto scores = [&](const char* kl, f32x16 (&s)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + kv_off(32 * kt + krow, 2 * kk + hf));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[kk], s[kt], 0, 0, 0);
      }
    }
  };
  // Masks of key block j0 for this lane's query: key offset
  // t = 32 kt + 16 (r / 8) + 8 hf + r % 8 is visible iff lo < t <= hi.
  // Decided per 32-key half kt from the bounds' extremes over the wave's
  // rows (wave-uniform): a half that every row sees fully is left alone, a
  // half that no row sees is set to -inf, and only a half that a bound cuts
  // into takes a compare and a select per score.  Query tiles start at
  // multiples of 32, so a causal diagonal or a window edge cuts into one half.
  auto mask = [&](f32x16 (&s)[2], int j0) { mask_block(p, kr, qi, qa, qb, hf, s, j0); };
  // Row maximum of a block and the lazy reference update (sets the pending
  // accumulator factor; l is rescaled here).
  auto update_ref = [&](const f32x16 (&s)[2]) {
    float m4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x16& sq = s[q >> 1];
      const int o = 8 * (q & 1);
      m4[q] = vmax3(vmax3(vmax3(sq[o], sq[o + 1], sq[o + 2]), sq[o + 3], sq[o + 4]), sq[o + 5], sq[o + 6]);
    }
    const float mx = vmax3(vmax3(m4[0], m4[1], s[0][7]), vmax3(m4[2], m4[3], s[0][15]), vmax(s[1][7], s[1][15]));
    const float mblk = max_halves(mx) * c;
    const bool move = mblk > m_ref + kTau;
    // A lane that does not move keeps factor 1 exactly (a lane that has seen
    // no key must not form exp2(-inf - (-inf))).
    const float alpha = move ? fast_exp2(m_ref - mblk) : 1.0f;
    m_ref = move ? mblk : m_ref;
    l_run *= alpha;
    l_bf *= alpha;
    pend_alpha = alpha;
    pend = __any(move);
  };
  // exp2 of half a block (the 16 registers of one kt) against the current
  // reference, packed to bf16; the row sum is taken in float32.
  // Pair q (registers 2q, 2q + 1) of a half block takes the FMA-pipe
  // exponential in the POLY variants.
  auto on_fma = [](int q) { return POLY > 0 && q % POLY == POLY - 1; };
  auto exp_half = [&](f32x16& s, bf16x8 (&pk)[2]) {
    const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;
    float part[2] = {0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = fmaf(s[8 * t + e], c, -mr);
        f[e] = on_fma(4 * t + e / 2) ? exp2_fma(x) : fast_exp2(x);
      }
      pk[t] = __builtin_convertvector(f, bf16x8);
#pragma unroll
      for (int e = 0; e < 8; ++e) part[t] += f[e];
      const u32x4 w4 = __builtin_bit_cast(u32x4, pk[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) l_bf = sum_bf16x2(w4[e], l_bf);
    }
    l_run += part[0] + part[1];
  };
  // K fragment i (kt = i / 8, kk = i % 8) of the S^T MFMAs; V^T fragment i
  // (md = i / 4, 8-key group i % 4) of the P V MFMAs.
  auto kread = [&](const char* kl, int i) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(kl + kv_off(32 * (i >> 3) + krow, 2 * (i & 7) + hf));
  };
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  // The swizzle of row 16 g + R (R < 16) equals that of R, so the transposed
  // reads of group g are those of group 0 moved by 4096 g bytes: 8 per-lane
  // offsets (r, md) and an immediate per group.
  int voff[2][NMD];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int md = 0; md < NMD; ++md) voff[r][md] = kv_off(4 * r + tr_rowoff, (32 * md + tr_col) >> 3) + tr_byte;
  auto vread = [&](const char* vl, int i) -> bf16x8 {
    const int md = i >> 2, g = i & 3;
    s16x4 h[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const char* a = vl + voff[r][md] + 4096 * g;
      h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
    }
    const s16x8 hv = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, hv);
  };
  // Exponentials of a half block in three stages per pair p of score
  // registers (2p, 2p + 1), each in its own slot so that no slot waits on a
  // result of the same slot: the scaled, shifted exponent (in place), the
  // exp2 (in place), then the bf16 packing into word p of `pw` and the
  // float32 row-sum.
  auto st1 = [&](f32x16& s, int p, float mr) {
    s[2 * p] = fmaf(s[2 * p], c, -mr);
    s[2 * p + 1] = fmaf(s[2 * p + 1], c, -mr);
    OSFA_KEEP(s[2 * p]);
    OSFA_KEEP(s[2 * p + 1]);
  };
  auto st2 = [&](f32x16& s, int p) {
    if (on_fma(p)) {
      s[2 * p] = exp2_fma(s[2 * p]);
      s[2 * p + 1] = exp2_fma(s[2 * p + 1]);
    } else {
      s[2 * p] = fast_exp2(s[2 * p]);
      s[2 * p + 1] = fast_exp2(s[2 * p + 1]);
    }
    OSFA_KEEP(s[2 * p]);
    OSFA_KEEP(s[2 * p + 1]);
  };
  auto st3 = [&](const f32x16& s, int p, u32x4 (&pw)[2], float& acc, float& accb) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = {s[2 * p], s[2 * p + 1]};
    uint32_t wd = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    acc += f[0] + f[1];
    accb = sum_bf16x2(wd, accb);
    OSFA_KEEP(wd);
    OSFA_KEEP(acc);
    OSFA_KEEP(accb);
    pw[p >> 2][p & 3] = wd;
  };
  auto to_p = [&](const u32x4 (&pw)[2], bf16x8 (&pk)[2]) {
    pk[0] = __builtin_bit_cast(bf16x8, pw[0]);
    pk[1] = __builtin_bit_cast(bf16x8, pw[1]);
  };

  // One step j: kn holds K_{j+1}, vc holds V_j; kd and vd receive K_{j+2}
  // and V_{j+1}.  sc = S_j (masked, reference already updated, first half
  // exponentiated into pc), sn receives S_{j+1}, pn its first-half P.  Each
  // phase is written as 16 slots of one MFMA plus a few VALU instructions,
  // with LDS reads issued a fixed number of slots ahead; sched_barrier keeps
  // the slots in this order.
  auto step = [&](auto has_next, int j, const char* kn, const char* vc, char* kd, char* vd, f32x16 (&sc)[2],
                  f32x16 (&sn)[2], const bf16x8 (&pc)[2], bf16x8 (&pn)[2]) {
    constexpr bool NEXT = decltype(has_next)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // (A wave that does not see block j + 1 runs this step without NEXT but
    // still loads its share of V_{j+1} for the others.)
    if (j + 2 < nblk) issue(kIsK, kb_lo + j + 2, kd);
    if (j + 1 < nblk) issue(kIsV, kb_lo + j + 1, vd);
    // Phase A: S_{j+1} on the matrix core, second half of P_j on the VALU.
    bf16x8 p1[2];
    {
      const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;
      u32x4 pw[2];
      float acc = 0.0f, accb = 0.0f;
      bf16x8 kf[16];
      if constexpr (NEXT) {
#pragma unroll
        for (int i = 0; i < KAHEAD; ++i) kf[i] = kread(kn, i);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (NEXT) {
          if (i + KAHEAD < 16) kf[i + KAHEAD] = kread(kn, i + KAHEAD);
          if ((i & 7) == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sn[i >> 3][r] = 0.0f;
          }
          sn[i >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qreg[i & 7], sn[i >> 3], 0, 0, 0);
        }
        // Pair p: stage 1 in slot 2p, stage 2 in slot 2p + 1, stage 3 in
        // slot 2p + 2 (the last one after the loop).
        if ((i & 1) == 0) st1(sc[1], i >> 1, mr);
        if (i & 1) st2(sc[1], i >> 1);
        if ((i & 1) == 0 && i >= 2) st3(sc[1], (i >> 1) - 1, pw, acc, accb);
        __builtin_amdgcn_sched_barrier(0);
      }
      st3(sc[1], 7, pw, acc, accb);
      l_run += acc;
      l_bf += accb;
      to_p(pw, p1);
    }
    if constexpr (NEXT) mask(sn, (kb_lo + j + 1) * kBc);
    // Phase B: P_j V_j on the matrix core; max of S_{j+1}, the reference
    // update and the first half of P_{j+1} on the VALU.
    if (pend) {
#pragma unroll
      for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[md][r] *= pend_alpha;
    }
    {
      bf16x8 vf[16];
#pragma unroll
      for (int i = 0; i < VAHEAD; ++i) vf[i] = vread(vc, i);
      float m4[4], mx = 0.0f, mblk = 0.0f, alpha = 1.0f;
      bool move = false;
      float mr = 0.0f, acc = 0.0f, accb = 0.0f;
      u32x4 pw[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + VAHEAD < 16) vf[i + VAHEAD] = vread(vc, i + VAHEAD);
        const bf16x8 pb = ((i & 3) < 2) ? pc[i & 1] : p1[i & 1];
        oacc[i >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pb, oacc[i >> 2], 0, 0, 0);
        if constexpr (NEXT) {
          // Row maximum of the 32 scores in 16 three-input maxima: four
          // independent chains over the 8-register groups q, one link per
          // slot, then the four chains and their last registers.
          if (i == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x16& sq = sn[q >> 1];
              const int o = 8 * (q & 1);
              m4[q] = vmax3(sq[o], sq[o + 1], sq[o + 2]);
            }
          } else if (i <= 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x16& sq = sn[q >> 1];
              const int o = 8 * (q & 1) + 2 * i + 1;
              m4[q] = vmax3(m4[q], sq[o], sq[o + 1]);
            }
          } else if (i == 3) {
            m4[0] = vmax3(m4[0], m4[1], sn[0][7]);
            m4[2] = vmax3(m4[2], m4[3], sn[0][15]);
            m4[1] = vmax(sn[1][7], sn[1][15]);
          } else if (i == 4) {
            mx = vmax3(m4[0], m4[2], m4[1]);
          } else if (i == 5) {
            mblk = max_halves(mx) * c;
          } else if (i == 6) {
            move = mblk > m_ref + kTau;
            // Formed for every lane; lanes that do not move take 1 below
            // (a lane that has seen no key would form exp2(-inf - (-inf))).
            alpha = fast_exp2(m_ref - mblk);
          } else if (i == 7) {
            alpha = move ? alpha : 1.0f;
            m_ref = move ? mblk : m_ref;
            l_run *= alpha;
            l_bf *= alpha;
            pend_alpha = alpha;
            pend = __any(move);
            mr = (m_ref == kNegInf) ? 0.0f : m_ref;
            OSFA_KEEP(mr);
            OSFA_KEEP(m_ref);
            OSFA_KEEP(l_run);
            OSFA_KEEP(pend_alpha);
          } else {
            // Pair k = i - 8: stage 1 now, stage 2 of pair k - 1, stage 3 of
            // pair k - 2 (the last ones after the loop).
            const int k = i - 8;
            st1(sn[0], k, mr);
            if (k >= 1) st2(sn[0], k - 1);
            if (k >= 2) st3(sn[0], k - 2, pw, acc, accb);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NEXT) {
        st2(sn[0], 7);
        st3(sn[0], 6, pw, acc, accb);
        st3(sn[0], 7, pw, acc, accb);
        l_run += acc;
        l_bf += accb;
        to_p(pw, pn);
      } else {
        pend = false;
      }
    }
  };

  if (nblk > 0) {
    f32x16 sA[2], sB[2];
    bf16x8 pA[2], pB[2];
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // A wave skips the matrix work of the range's first or last block when
    // none of its 32 rows sees it (a window edge, a causal diagonal).
    if (rows_see_block(p, kr.jmax, qa, qb, kb_lo * kBc)) {
      scores(k0, sA);
      mask(sA, kb_lo * kBc);
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[kt][r] = kNegInf;
    }
    update_ref(sA);
    pend = false;  // the accumulator is still zero
    exp_half(sA[0], pA);
    const std::integral_constant<bool, true> yes;
    const std::integral_constant<bool, false> no;
    // Steps in pairs (static buffer roles); the last step has no next block.
    int j = 0;
    for (; j + 2 < nblk; j += 2) {
      step(yes, j, k1, v0, k0, v1, sA, sB, pA, pB);
      step(yes, j + 1, k0, v1, k1, v0, sB, sA, pB, pA);
    }
    // The last block: a wave that sees none of it neither scores it (the
    // step before runs without a next block) nor multiplies it with V (its
    // step is only the barrier every wave takes).
    const bool see_last = rows_see_block(p, kr.jmax, qa, qb, (kb_lo + nblk - 1) * kBc);
    auto barrier_step = [&]() {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    };
    if (j + 1 < nblk) {
      if (see_last) {
        step(yes, j, k1, v0, k0, v1, sA, sB, pA, pB);
        step(no, j + 1, k0, v1, k1, v0, sB, sA, pB, pA);
      } else {
        step(no, j, k1, v0, k0, v1, sA, sB, pA, pB);
        barrier_step();
      }
    } else if (see_last) {
      step(no, j, k1, v0, k0, v1, sA, sB, pA, pB);
    } else {
      barrier_step();
    }
  }

  // O divides by the sum of the bf16 P it accumulated (their rounding
  // cancels in the ratio); LSE takes the float32 sum.
  const float l_tot = sum_halves(l_run);
  const float l_div = sum_halves(l_bf);
  const float inv = l_div > 0.0f ? 1.0f / l_div : 0.0f;
  // O rows through LDS: a lane holds 8-byte pieces of one row (columns
  // 32 md + 8 rq + 4 hf .. + 3), which stored directly would be 16-byte runs
  // scattered over 32 rows per instruction.  Once every wave is past its
  // last K/V read and no load to LDS is in flight, each wave writes its 32
  // rows (8 KB, swizzled block layout) to its own part of the K buffers and
  // stores them back as whole 256-byte rows.
  static_assert(NW * 32 * D * 2 <= 2 * BLK && NW % 2 == 0, "the O rows fit in the two K buffers");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  char* orow = (w < NW / 2 ? k0 : k1) + (w % (NW / 2)) * (32 * D * 2);
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      u32x2 wv;
      wv[0] = pack_bf16x2(oacc[md][4 * rq + 0] * inv, oacc[md][4 * rq + 1] * inv);
      wv[1] = pack_bf16x2(oacc[md][4 * rq + 2] * inv, oacc[md][4 * rq + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + kv_off(l32, 4 * md + rq) + 8 * hf) = wv;
    }
  u32x4 rows[8];  // 4 rows per instruction
#pragma unroll
  for (int t = 0; t < 8; ++t) rows[t] = *reinterpret_cast<const u32x4*>(orow + kv_off(4 * t + (lane >> 4), lane & 15));
  __bf16* Og = static_cast<__bf16*>(p.o) + head_off;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int qr = q0 + 32 * w + 4 * t + (lane >> 4);
    if (qr < N) *reinterpret_cast<u32x4*>(Og + (size_t)qr * D + 8 * (lane & 15)) = rows[t];
  }
  if (qi < N && hf == 0)
    p.lse[(size_t)tile.bh * N + qi] = l_tot > 0.0f ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
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



// ---------------------------------------------------------------------------
// float32, few query tiles: the waves of a workgroup split the key range
//
// When a launch has fewer 128-query tiles than the chip has CUs, the tile
// kernel above leaves most SIMDs idle.  Here a workgroup owns 32 queries and
// its S waves take the 32-key blocks of their range in turn (wave w: blocks
// w, w + S, ...), each staging its blocks in its own LDS region (no
// barrier), and each keeps its own partial (m, l, O).  At the end the S
// partial states are merged through LDS by the rescale rule of split-KV
// (page "Derive online softmax, prove it is exact", "What interviewers probe
// next"; article "Online softmax", Step 4): M = max m_w, O = sum 2^(m_w - M)
// O_w / sum 2^(m_w - M) l_w.
// ---------------------------------------------------------------------------

// The keys query i sees form one interval [lo, hi] (hi = lo - 1 when empty):
// j < jmax, j <= i when causal, |i - j| < window when windowed -- the rule of
// visible(), evaluated once per query instead of once per score.
struct KeySpan {
  int lo, hi;
};
__device__ __forceinline__ KeySpan key_span(const FwdParams& p, int jmax, int i) {
  long long lo = 0, hi = (long long)jmax - 1;
  if (p.causal) hi = min(hi, (long long)i);
  if (p.window > 0) {
    lo = max(lo, (long long)i - p.window + 1);
    hi = min(hi, (long long)i + p.window - 1);
  }
  KeySpan k;
  k.lo = (int)lo;
  k.hi = (int)max(hi, lo - 1);
  return k;
}

// Orders a wave's earlier LDS accesses before its later ones across lanes:
// wavefront-scope release and acquire around the wave's own barrier.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int S>
__global__ __launch_bounds__(64 * S, 1) void fwd_f32_split_kernel(FwdParams p) {
  constexpr int BC = 32;        // keys per block
  constexpr int RS = D + 4;     // LDS row stride (floats), +16 B pad
  constexpr int NKK = D / 2;
  constexpr int NMD = D / 32;
  constexpr int WREG = 2 * BC * RS;  // floats of one wave's region (K and V rows)
  static_assert(32 * (D + 2) <= WREG, "the merge state fits in a wave's region");
  __shared__ __attribute__((aligned(16))) float lds[S * WREG];

  const Tile tile = map_tile(p);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.q0;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int N = p.N;
  const size_t head_off = (size_t)tile.bh * (size_t)N * D;
  const float* Kg = static_cast<const float*>(p.k) + head_off;
  const float* Vg = static_cast<const float*>(p.v) + head_off;

  // MFMA step kk pairs d = kk (lower half) with d = kk + D/2 (upper half).
  const int qi = q0 + l32;
  float qreg[NKK];
  {
    const bool ok = qi < N;
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + head_off +
                                                      (size_t)(ok ? qi : 0) * D + (D / 2) * hf);
#pragma unroll
    for (int i = 0; i < NKK / 4; ++i) {
      f32x4 v = ok ? src[i] : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) qreg[4 * i + e] = v[e];
    }
  }

  const KeyRange kr = key_range(p, b, q0);
  const KeySpan span = key_span(p, kr.jmax, qi);
  const int kb_lo = kr.kbeg / BC;
  const int kb_hi = (kr.kend > kr.kbeg) ? (kr.kend + BC - 1) / BC : kb_lo;
  float* ks = lds + w * WREG;
  float* vs = ks + BC * RS;

  f32x16 oacc[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  const float c = p.c;

  // A block's K and V rows pass through registers on their way to LDS; the
  // next block's are loaded while the current one is computed, so a wave
  // waits on global memory once, before its first block.  Lane `lane` holds
  // the 16-byte chunks lane + 64 t of the block (rows past N read row
  // N - 1; they are masked).
  constexpr int NLD = BC * D / 4 / 64;
  f32x4 kbuf[NLD], vbuf[NLD];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int idx = lane + 64 * t;
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      const int j = min(kb * BC + row, N - 1);
      kbuf[t] = *reinterpret_cast<const f32x4*>(Kg + (size_t)j * D + 4 * c4);
      vbuf[t] = *reinterpret_cast<const f32x4*>(Vg + (size_t)j * D + 4 * c4);
    }
  };
  if (kb_lo + w < kb_hi) fetch(kb_lo + w);
  for (int kb = kb_lo + w; kb < kb_hi; kb += S) {
    const int j0 = kb * BC;
    // This wave's block into its own region.  Other lanes read the previous
    // block's rows from it, so the writes wait for those reads, and the
    // reads below for the writes.
    wave_sync();
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int idx = lane + 64 * t;
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      *reinterpret_cast<f32x4*>(ks + row * RS + 4 * c4) = kbuf[t];
      *reinterpret_cast<f32x4*>(vs + row * RS + 4 * c4) = vbuf[t];
    }
    wave_sync();
    if (kb + S < kb_hi) fetch(kb + S);
    // S^T: lane l, register r holds key j0 + 8 (r/4) + 4 hf + r%4 of query qi.
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    const float* krow = ks + l32 * RS + (D / 2) * hf;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[kk], qreg[kk], s, 0, 0, 0);
    // Every block is masked, by selects: with a branch here (masked blocks
    // only) the compiler read the last score register of the d = 128
    // instance on the masked path 17 wait states after the MFMA that writes
    // it, one fewer than the 18 it inserts in straight-line code, and wrote
    // the stale value back.  Selects keep the reads in the MFMAs' own block.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      s[r] = (j < span.lo || j > span.hi) ? kNegInf : s[r];
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_ref = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    float rs = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(s[r], c, -m_ref));
      s[r] = e;
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
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
      for (int md = 0; md < NMD; ++md)
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * RS + 32 * md + l32], s[r], oacc[md], 0, 0, 0);
    }
  }

  // This wave's state into its region: m[32], l[32], O[32][D] (query-major).
  const float l_tot = sum_halves(l_run);
  float* st = ks;
  if (hf == 0) {
    st[l32] = m_run;
    st[32 + l32] = l_tot;
  }
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) st[64 + l32 * D + 32 * md + 8 * (r >> 2) + 4 * hf + (r & 3)] = oacc[md][r];
  __syncthreads();
  // Merge: thread t takes elements t, t + 64 S, ... of the tile's 32 x D outputs.
  for (int e = threadIdx.x; e < 32 * D; e += 64 * S) {
    const int q = e / D, d = e % D;
    float M = kNegInf;
#pragma unroll
    for (int u = 0; u < S; ++u) M = fmaxf(M, lds[u * WREG + q]);
    float lsum = 0.0f, osum = 0.0f;
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const float mu = lds[u * WREG + q];
      const float wgt = (mu == kNegInf) ? 0.0f : fast_exp2(mu - M);
      lsum += wgt * lds[u * WREG + 32 + q];
      osum += wgt * lds[u * WREG + 64 + q * D + d];
    }
    const int qq = q0 + q;
    if (qq < N) {
      static_cast<float*>(p.o)[head_off + (size_t)qq * D + d] = lsum > 0.0f ? osum / lsum : 0.0f;
      if (d == 0) p.lse[(size_t)tile.bh * N + qq] = lsum > 0.0f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
    }
  }
}


// ---------------------------------------------------------------------------
// float32, smallest launches: 16-query workgroups on v_mfma_f32_16x16x4_f32.
//
// The key-split kernel above runs one 32-query tile per workgroup; a single
// head of 1000 queries is then 32 workgroups, and their matrix time (the
// per-CU MFMA work is fixed by the tile) sets the launch's time.  With 16
// queries per workgroup the same work spreads over twice as many CUs at the
// same MFMA rate per query-key pair.  Structure as above: S waves take the
// 16-key blocks of the range in turn, each keeps its own (m, l, O), and the
// partial states are merged through LDS by the split-KV rescale rule.
//
// Layouts (lane l, g = l / 16, c = l % 16): an MFMA step takes A[c][g],
// B[g][c] and leaves D[4 g + i][c] in register i.  Scores are S^T = K Q^T
// with the K rows permuted (A row r holds key 4 (r % 4) + r / 4), so that
// register i of lane l holds key 4 i + g of query c: exactly the B operand
// of P V step i (keys 4 i .. 4 i + 3), with no data movement.
// ---------------------------------------------------------------------------
template <int D, int S>
__global__ __launch_bounds__(64 * S, 1) void fwd_f32_split16_kernel(FwdParams p) {
  constexpr int BC = 16;       // keys per block
  constexpr int RK = D + 4;    // K row stride (floats): an S step's 16 rows x 4 columns hit 64 distinct banks
  constexpr int RV = D + 16;   // V row stride: a P V step's 4 rows x 16 columns hit 64 distinct banks
  constexpr int NKK = D / 4;   // S steps (4 d each)
  constexpr int NMD = D / 16;  // 16-row d tiles of O^T
  constexpr int WREG = BC * RK + BC * RV;  // floats of one wave's region (K rows, then V rows)
  static_assert(32 + 16 * D <= WREG, "the merge state fits in a wave's region");
  __shared__ __attribute__((aligned(16))) float lds[S * WREG];

  const Tile tile = map_tile(p);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.q0;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int g = lane >> 4;
  const int N = p.N;
  const size_t head_off = (size_t)tile.bh * (size_t)N * D;
  const float* Kg = static_cast<const float*>(p.k) + head_off;
  const float* Vg = static_cast<const float*>(p.v) + head_off;

  const int qi = q0 + c16;
  float qreg[NKK];  // Q[qi][4 kk + g]
  {
    const bool ok = qi < N;
    const float* src = static_cast<const float*>(p.q) + head_off + (size_t)(ok ? qi : 0) * D + g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qreg[kk] = ok ? src[4 * kk] : 0.0f;
  }

  const KeyRange kr = key_range(p, b, q0);
  const KeySpan span = key_span(p, kr.jmax, qi);
  const int kb_lo = kr.kbeg / BC;
  const int kb_hi = (kr.kend > kr.kbeg) ? (kr.kend + BC - 1) / BC : kb_lo;
  float* ks = lds + w * WREG;
  float* vs = ks + BC * RK;
  const int krow = 4 * (c16 & 3) + (c16 >> 2);  // the key this lane feeds as A row c16

  f32x4 oacc[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md) oacc[md] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf, l_run = 0.0f;
  const float c = p.c;

  // K and V rows of a block pass through registers on their way to the
  // wave's LDS region; the next block's are loaded while the current one is
  // computed.  Lane `lane` holds the 16-byte chunks lane + 64 t of the
  // block (rows past N read row N - 1; they are masked).
  constexpr int NLD = BC * D / 4 / 64;
  f32x4 kbuf[NLD], vbuf[NLD];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int idx = lane + 64 * t;
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      const int j = min(kb * BC + row, N - 1);
      kbuf[t] = *reinterpret_cast<const f32x4*>(Kg + (size_t)j * D + 4 * c4);
      vbuf[t] = *reinterpret_cast<const f32x4*>(Vg + (size_t)j * D + 4 * c4);
    }
  };
  if (kb_lo + w < kb_hi) fetch(kb_lo + w);
  for (int kb = kb_lo + w; kb < kb_hi; kb += S) {
    const int j0 = kb * BC;
    // Other lanes read the previous block's rows from this region: the
    // writes wait for those reads, and the reads below for the writes.
    wave_sync();
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int idx = lane + 64 * t;
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      *reinterpret_cast<f32x4*>(ks + row * RK + 4 * c4) = kbuf[t];
      *reinterpret_cast<f32x4*>(vs + row * RV + 4 * c4) = vbuf[t];
    }
    wave_sync();
    if (kb + S < kb_hi) fetch(kb + S);
    f32x4 s = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float* kr_row = ks + krow * RK + g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x4f32(kr_row[4 * kk], qreg[kk], s, 0, 0, 0);
    // Masks by selects on every block (no branch between the MFMAs and the
    // first read of their result).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * i + g;
      s[i] = (j < span.lo || j > span.hi) ? kNegInf : s[i];
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // the block's maximum for query c16
    const float m_new = fmaxf(m_run, mx * c);
    const float m_ref = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(fmaf(s[i], c, -m_ref));
      s[i] = e;
      rs += e;
    }
    l_run = l_run * alpha + rs;  // this lane's keys only; summed over g at the end
    m_run = m_new;
#pragma unroll
    for (int md = 0; md < NMD; ++md) oacc[md] *= alpha;
    // O^T += V^T P^T: step i takes keys 4 i .. 4 i + 3 (A[c][g] = V[4 i + g][16 md + c]).
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int md = 0; md < NMD; ++md)
        oacc[md] = __builtin_amdgcn_mfma_f32_16x16x4f32(vs[(4 * i + g) * RV + 16 * md + c16], s[i], oacc[md], 0, 0, 0);
  }

  // This wave's state into its region: m[16], l[16], O[16][D] (query-major).
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  float* st = ks;
  if (g == 0) {
    st[c16] = m_run;
    st[16 + c16] = l_tot;
  }
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int i = 0; i < 4; ++i) st[32 + c16 * D + 16 * md + 4 * g + i] = oacc[md][i];
  __syncthreads();
  // Merge: thread t takes elements t, t + 64 S, ... of the tile's 16 x D outputs.
  for (int e = threadIdx.x; e < 16 * D; e += 64 * S) {
    const int q = e / D, d = e % D;
    float M = kNegInf;
#pragma unroll
    for (int u = 0; u < S; ++u) M = fmaxf(M, lds[u * WREG + q]);
    float lsum = 0.0f, osum = 0.0f;
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const float mu = lds[u * WREG + q];
      const float wgt = (mu == kNegInf) ? 0.0f : fast_exp2(mu - M);
      lsum += wgt * lds[u * WREG + 16 + q];
      osum += wgt * lds[u * WREG + 32 + q * D + d];
    }
    const int qq = q0 + q;
    if (qq < N) {
      static_cast<float*>(p.o)[head_off + (size_t)qq * D + d] = lsum > 0.0f ? osum / lsum : 0.0f;
      if (d == 0) p.lse[(size_t)tile.bh * N + qq] = lsum > 0.0f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) {
    const FwdParams p = make_params(a, 32 * kV2Waves);
    hipLaunchKernelGGL((fwd_bf16_d128_kernel<kV2Waves, 0>), dim3(grid_for(p)), dim3(64 * kV2Waves), 0, stream, p);
  } else {
    const FwdParams p = make_params(a, kBr);
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid_for(p)), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_bf16_exp2_offload(const FwdArgs& a, int poly_every, hipStream_t stream) {
  const FwdParams p = make_params(a, 32 * kV2Waves);
  const dim3 grid(grid_for(p)), block(64 * kV2Waves);
  if (poly_every == 2)
    hipLaunchKernelGGL((fwd_bf16_d128_kernel<kV2Waves, 2>), grid, block, 0, stream, p);
  else if (poly_every == 4)
    hipLaunchKernelGGL((fwd_bf16_d128_kernel<kV2Waves, 4>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_bf16_d128_kernel<kV2Waves, 8>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  // Fewer 32-query tiles than CUs: 16-query workgroups of 8 waves that split
  // the keys.  Fewer 128-query tiles than CUs: 32-query workgroups whose
  // waves split the keys (8 waves at d = 64; 4 at d = 128, whose per-wave K
  // and V regions take 33 KB of LDS each).
  const long long tiles128 = (long long)a.B * a.H * ((a.N + kBr - 1) / kBr);
  const long long tiles32 = (long long)a.B * a.H * ((a.N + 31) / 32);
  if (tiles32 < kSplitTilesBelow) {
    const FwdParams p = make_params(a, 16);
    if (a.d == 128)
      hipLaunchKernelGGL((fwd_f32_split16_kernel<128, 8>), dim3(grid_for(p)), dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_f32_split16_kernel<64, 8>), dim3(grid_for(p)), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
  if (tiles128 < kSplitTilesBelow) {
    const FwdParams p = make_params(a, 32);
    if (a.d == 128)
      hipLaunchKernelGGL((fwd_f32_split_kernel<128, 4>), dim3(grid_for(p)), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_f32_split_kernel<64, 8>), dim3(grid_for(p)), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
  const FwdParams p = make_params(a, kBr);
  const dim3 grid(grid_for(p)), block(kThreads);
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace osfa
