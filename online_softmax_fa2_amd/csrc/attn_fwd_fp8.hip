// Attention forward with FP8 (OCP e4m3) Q, K and V on gfx950: the query-tile
// online-softmax recurrence of attn_fwd (masks, guard, deferred division,
// LSE) with both products on the FP8 matrix core
// (v_mfma_scale_f32_32x32x64_f8f6f4) and float32 statistics.  The pages name
// FP8 as the precision step of FA3 (page "Derive online softmax, prove it is
// exact", "What interviewers probe next"; article "Online softmax",
// "Trade-offs and edge cases").
//
// Inputs are e4m3 codes with one float32 descale per tensor (value = code x
// descale).  The scores are scale * qd * kd * (q8 . k8); qd * kd is folded
// into the exp2 factor, vd into the final normalization.
//
// P enters P V as e4m3 too.  Its dynamic range is managed per (query, key
// block) through the MFMA's E8M0 operand scale: the block's row maximum is
// mapped into (128, 256] (the exponent frame m_ref - u for an integer u), the
// block's P are formed and rounded in that frame, and the MFMA multiplies
// them back by 2^-u, so no P below the block maximum by less than 2^17 is
// lost to underflow.  The sum that divides O is taken over the same rounded
// P by one more MFMA against a row of ones (the rounding of a dominant P
// cancels in the ratio); LSE uses the float32 sum of the unrounded P.
//
// Layout: one workgroup per 128-query tile, each of its 4 waves owning 32
// queries (lane = query, as in the bf16 kernels: S^T = K Q^T, O^T += V^T
// P^T).  K and V blocks of 64 keys x 128 B are copied to LDS by buffer loads
// straight to LDS, double buffered, in a layout where 16-byte chunk c of row
// r sits at r * 128 + ((c ^ f8_swz(r)) << 4); K is read by rows, V
// transposed with ds_read_b64_tr_b8 (8 consecutive keys of one column per
// lane).
//
// MFMA operand layout used here (checked on the device): for
// 32x32x64 with 8-bit operands, lane l holds 32 bytes of row (A) or column
// (B) l % 32; the two halves of the wave hold different k.  Both operands of
// a product are loaded with the same (half, byte) -> k assignment, so it
// need not be known, except for the B scale: bytes 0-15 of both halves of
// column j take the scale of lane j, bytes 16-31 that of lane j + 32.  Here
// every lane of a query supplies the same scale.
#include "device_common.h"
#include "fwd_common.h"
#include "launch.h"

namespace osfa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kD8 = 128;                  // head dim = bytes per fp8 row
constexpr int kBlk8 = kBc * kD8;          // 8 KB per 64-key block
constexpr int kScale1 = 127;              // E8M0 encoding of 1.0
constexpr uint32_t kOnes4 = 0x38383838u;  // four e4m3 1.0

// Chunk slot of a 128-byte row: XOR with f(row) = ((row >> 1) & 3) << 1 |
// (row >> 3) & 1.  With 64 four-byte banks (two rows per bank line), the
// 16 rows of a K fragment read (16 lanes x 16 B) and the 8 rows x 2 chunks
// of a transposed V read (32 lanes x 8 B) each touch every bank once.
__device__ __forceinline__ int f8_swz(int row) { return (((row >> 1) & 3) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int f8_off(int row, int chunk) { return row * kD8 + ((chunk ^ f8_swz(row)) << 4); }

__device__ __forceinline__ i32x8 join(u32x4 a, u32x4 b) {
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// Rows [r0, r0 + 64) of an [N, 128] byte matrix into a staged block: load t
// of wave w fills 1 KB = rows 8 (w + 4 t) .. + 7, lane L taking row
// (L >> 3) of the group and the chunk that belongs at slot L & 7.  Rows past
// N read row N - 1 (their scores are masked).
__device__ __forceinline__ void stage8(__amdgpu_buffer_rsrc_t rs, char* dst, int r0, int N, int w, int lane) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 8 * (w + 4 * t) + (lane >> 3);
    const int grow = min(r0 + row, N - 1);
    const int off = grow * kD8 + 16 * ((lane & 7) ^ f8_swz(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (w + 4 * t) * 1024),
                                             16, off, 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads, 2) void fwd_fp8_d128_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) char k0[kBlk8];
  __shared__ __attribute__((aligned(1024))) char k1[kBlk8];
  __shared__ __attribute__((aligned(1024))) char v0[kBlk8];
  __shared__ __attribute__((aligned(1024))) char v1[kBlk8];

  const Tile tile = map_tile(p);
  if (!tile.valid) return;
  const int b = tile.bh / p.H;
  const int q0 = tile.q0;
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)tile.bh * N;

  const KeyRange kr = key_range(p, b, q0);
  const int kb_lo = kr.kbeg / kBc;
  const int nblk = kr.kend > kr.kbeg ? (kr.kend + kBc - 1) / kBc - kb_lo : 0;

  const char* kbase = static_cast<const char*>(p.k) + head * kD8;
  const char* vbase = static_cast<const char*>(p.v) + head * kD8;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, N * kD8, kBufDword3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, N * kD8, kBufDword3);
  auto load_block = [&](int j, char* kd, char* vd) {
    stage8(krs, kd, (kb_lo + j) * kBc, N, w, lane);
    stage8(vrs, vd, (kb_lo + j) * kBc, N, w, lane);
  };
  if (nblk > 0) load_block(0, k0, v0);

  // Q bytes 64 kk + 32 hf + [0, 32) of query qi, the B operand of S^T.
  const int qi = q0 + 32 * w + l32;
  const bool qok = qi < N;
  i32x8 qreg[2];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q) + (head + (qok ? qi : 0)) * kD8 + 32 * hf);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 z{0, 0, 0, 0};
      qreg[kk] = join(qok ? src[4 * kk] : z, qok ? src[4 * kk + 1] : z);
    }
  }

  // Transposed V reads: group g = lane >> 4 of 16 lanes, lane j in it; read
  // (kt, t) yields keys 32 kt + 16 t + 8 hf + [0, 8) of column 32 md + l32.
  const int tg = lane >> 4, tj = lane & 15;
  int voff[4][2][2];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = 8 * (tg >> 1) + 16 * t + 32 * kt + (tj >> 1);
        voff[md][kt][t] = f8_off(row, 2 * md + (tg & 1)) + 8 * (tj & 1);
      }

  f32x16 oacc[4], lacc;
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.0f;
  const i32x8 ones = l32 == 0 ? i32x8{(int)kOnes4, (int)kOnes4, (int)kOnes4, (int)kOnes4, (int)kOnes4, (int)kOnes4,
                                      (int)kOnes4, (int)kOnes4}
                              : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  float m_ref = kNegInf;  // reference of l_run, lacc and oacc (log2 units)
  float l_run = 0.0f;     // this half's share of sum P (float32 P: LSE)
  const float c = p.c;
  const int krow = perm_key(l32);
  const int qa = q0 + 32 * w, qb = qa + 31;

  auto block = [&](int j, const char* kl, const char* vl) {
    const int j0 = (kb_lo + j) * kBc;
    if (!rows_see_block(p, kr.jmax, qa, qb, j0)) return;
    // S^T = K Q^T: two 32-key groups, two 64-byte k-steps each.
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
      const int row = 32 * kt + krow;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const i32x8 kf = join(*reinterpret_cast<const u32x4*>(kl + f8_off(row, 4 * kk + 2 * hf)),
                              *reinterpret_cast<const u32x4*>(kl + f8_off(row, 4 * kk + 2 * hf + 1)));
        s[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qreg[kk], s[kt], 0, 0, 0, kScale1, 0, kScale1);
      }
    }
    // Register r of group kt holds key j0 + 32 kt + 16 (r / 8) + 8 hf + r % 8.
    mask_block(p, kr, qi, qa, qb, hf, s, j0);
    // Lane maximum of the 32 scores: four independent v_max3 chains.
    float m4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& x = s[g >> 1];
      const int o = 8 * (g & 1);
      m4[g] = vmax3(vmax3(vmax3(x[o], x[o + 1], x[o + 2]), x[o + 3], x[o + 4]), x[o + 5], x[o + 6]);
    }
    const float mx = vmax3(vmax3(m4[0], m4[1], s[0][7]), vmax3(m4[2], m4[3], s[0][15]), vmax(s[1][7], s[1][15]));
    const float mblk = max_halves(mx) * c;
    const bool move = mblk > m_ref + kTau;
    if (__any(move)) {
      const float alpha = move ? fast_exp2(m_ref - mblk) : 1.0f;
      l_run *= alpha;
      lacc[0] *= alpha;  // the other registers of lacc stay 0
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
      m_ref = move ? mblk : m_ref;
    }
    // Frame of this block: its maximum maps into (128, 256] (e4m3 max 448).
    // A query that sees no key of the block gets u = 127 (its P are 0).
    const bool live = mblk != kNegInf;
    int u = live ? 8 - (int)ceilf(mblk - m_ref) : 127;
    u = u > 127 ? 127 : u;
    const float mr = (live ? m_ref : 0.0f) - (float)u;
    float rs = 0.0f;
    i32x8 pb;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = fast_exp2(fmaf(s[kt][r + i], c, -mr));
          rs += e[i];
        }
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], wd, true);
        pb[4 * kt + (r >> 2)] = wd;  // bytes 16 kt + r .. + 3: keys 32 kt + 16 (r / 8) + 8 hf + r % 8 ..
      }
    l_run += __builtin_amdgcn_ldexpf(rs, -u);
    const int sb = kScale1 - u;
    // O^T += V^T P^T and the row of ones for sum(P) (both scaled by 2^-u).
#pragma unroll
    for (int md = 0; md < 4; ++md) {
      i32x2 h[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          h[kt][t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(vl + voff[md][kt][t]));
      const i32x8 vf{h[0][0][0], h[0][0][1], h[0][1][0], h[0][1][1], h[1][0][0], h[1][0][1], h[1][1][0], h[1][1][1]};
      oacc[md] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pb, oacc[md], 0, 0, 0, kScale1, 0, sb);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb, lacc, 0, 0, 0, kScale1, 0, sb);
  };

  // Two blocks per trip, one call site per buffer: with an if/else on the
  // parity the accumulators came out of the join in different registers
  // and were copied every block.
  auto iter = [&](int j, const char* kl, const char* vl, char* kn, char* vn) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (j + 1 < nblk) load_block(j + 1, kn, vn);
    block(j, kl, vl);
  };
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    iter(j, k0, v0, k1, v1);
    iter(j + 1, k1, v1, k0, v0);
  }
  if (j < nblk) iter(j, k0, v0, k1, v1);

  // Row 0 of lacc (lane l32 of the first half, register 0) is sum(rounded P)
  // for query l32; both halves need it.
  const float lq = __shfl(lacc[0], l32, 64);
  const float l_tot = sum_halves(l_run);
  const float inv = lq > 0.0f ? p.o_scale / lq : 0.0f;
  // O rows through LDS: a lane holds 8-byte pieces of one bf16 row (columns
  // 32 md + 8 rq + 4 hf .. + 3), which stored directly would be 16-byte runs
  // scattered over 32 rows per instruction.  Once every wave is past its
  // last K/V read and no load to LDS is in flight, each wave writes its 32
  // rows (8 KB, the 256-byte-row swizzle of tile_layout.h) to one of the four
  // K/V buffers and stores them back as whole rows.
  static_assert(kThreads == 256 && kBlk8 == 32 * kD8 * 2, "one 8 KB buffer per wave");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  char* orow = w == 0 ? k0 : w == 1 ? k1 : w == 2 ? v0 : v1;
#pragma unroll
  for (int md = 0; md < 4; ++md)
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
  __bf16* Og = static_cast<__bf16*>(p.o) + head * kD8;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int qr = q0 + 32 * w + 4 * t + (lane >> 4);
    if (qr < N) *reinterpret_cast<u32x4*>(Og + (size_t)qr * kD8 + 8 * (lane & 15)) = rows[t];
  }
  if (qok && hf == 0) p.lse[head + qi] = l_tot > 0.0f ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const FwdArgs& a, float qk_descale, float v_descale, hipStream_t stream) {
  FwdParams p = make_params(a, kBr);
  p.c *= qk_descale;
  p.o_scale = v_descale;
  hipLaunchKernelGGL(fwd_fp8_d128_kernel, dim3(grid_for(p)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace osfa
