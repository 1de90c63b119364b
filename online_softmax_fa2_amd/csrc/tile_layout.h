// K/V (or Q/dO) blocks staged in LDS by the attention kernels (forward and
// backward), and the row order of MFMA operands.
//
// A block is 64 rows of 128 bf16 (256 B per row).  It is copied from global
// memory by buffer_load_dwordx4 ... lds (16 B per lane, no VGPR staging):
// each load instruction fills 1 KB of LDS = 4 rows in lane order, the lane
// fetching whichever 16-byte chunk belongs at its LDS slot under the layout
//     byte(row, chunk) = row * 256 + ((chunk ^ f(row)) * 16),
//     f(row) = ((row & 3) << 2) | ((row >> 2) & 3),
// an XOR swizzle under which both access patterns touch every LDS bank once:
// row fragments (32 rows, one 16-byte chunk each: an MFMA operand holding 8
// consecutive columns of one row) and transposed reads (ds_read_b64_tr_b16
// over 8 rows x 64 B: in each group of 16 lanes, lane i receives 4
// consecutive rows of one column, so two such reads form an MFMA operand
// holding 8 consecutive rows of one column).
#pragma once

namespace osfa {

constexpr int kBc = 64;  // rows (keys or queries) per staged block
// s_waitcnt immediate for gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;
// Word 3 of a raw buffer resource (gfx9 family: 32-bit data format).
constexpr int kBufDword3 = 0x00020000;
// Cache-policy operand of a buffer load: the non-temporal bit (gfx94x/gfx950
// encoding), for data read once that should not displace reused lines.
constexpr int kCpolNT = 2;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int kv_off(int row, int chunk) { return row * 256 + ((chunk ^ swz(row)) << 4); }

// Row m of a 32-row MFMA operand takes row perm_key(m) of the 32-row group:
// bits 2 and 3 swapped.  With the 32x32 accumulator layout (lane l, register
// r holds output row 8(r/4) + 4(l/32) + r%4) this puts rows 16(r/8) +
// 8(l/32) + r%8 in register r: 8 consecutive registers hold 8 consecutive
// rows, which is the 8-element group the next MFMA takes as its B operand.
__device__ __forceinline__ int perm_key(int m) { return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1); }

}  // namespace osfa
