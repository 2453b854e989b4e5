// Matrix-core operand fragments of row-major bf16 tiles in LDS, head
// dimension 128, for the 32x32x16 bf16 product (shared by the backward
// kernels and the forward's short-tail pass).
//
// A tile holds 32 (or more) rows of 128 bf16; its 16-byte granules are
// XOR-swizzled per row.  A tile is read by rows (ds_read_b128) for an operand
// whose contraction runs along the features, or by the transpose read
// ds_read_b64_tr_b16 for one whose contraction runs along the rows; the
// latter hands out the rows in the order in which a 32x32 product's output
// keeps them, so the output block of one product, packed to bf16 pairs, is
// the second operand of the next one without any exchange between lanes.
#pragma once

#include "rha_device.hpp"
#include "rha_fwd_common.hpp"

namespace rha {
namespace frag {

using fwd::i16x4;
using fwd::lds_i16x4;

constexpr int BD = 128;            // head dimension
constexpr int RB = 32;             // rows (or keys) per matrix-core block
constexpr int ROWT = RB * BD * 2;  // one 32-row bf16 tile in LDS

// Granule swizzle serving both reads: 16 consecutive rows read at one
// granule (ds_read_b128, one row per lane) hit 16 distinct 16-byte slots, and
// 4 consecutive rows read by the transpose read (64 bytes each) hit 4
// distinct 64-byte bank groups.
__device__ __forceinline__ int fsw(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// byte offset of granule g (8 bf16) of row r
__device__ __forceinline__ int gran_off(int r, int g) { return r * BD * 2 + ((g ^ fsw(r)) * 16); }

__device__ __forceinline__ void put_granule(unsigned char* t, int r, int g, const u32x4& x) {
  *reinterpret_cast<u32x4*>(t + gran_off(r, g)) = x;
}

// Operand with m = row (row0 + lane % 32) of the tile, k = features 16 ks + 8 (lane / 32) + 0..7.
__device__ __forceinline__ bf16x8 row_frag(const unsigned char* t, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31), g = 2 * ks + (lane >> 5);
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(t + gran_off(r, g)));
}

// Operand of the transposed tile: m = feature 32 nb + .., k = 16 rows from
// 16 ks, in the order in which a 32x32 matrix-core output holds its rows
// (the order the packed probabilities below follow).
__device__ __forceinline__ bf16x8 col_frag(const unsigned char* t, int ks, int nb, int lane) {
  const int hh = lane >> 5, vj = lane & 15;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (vj & 3);
  const int vrow0 = 4 * hh + (vj >> 2);
  const int col = nb * 32 + vcol;
  const int r0 = vrow0 + 16 * ks, r1 = r0 + 8;
  const unsigned char* pa = t + gran_off(r0, col >> 3) + (col & 7) * 2;
  const unsigned char* pb = t + gran_off(r1, col >> 3) + (col & 7) * 2;
  const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pa);
  const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pb);
  const u32x2 w0 = __builtin_bit_cast(u32x2, x0), w1 = __builtin_bit_cast(u32x2, x1);
  return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
}

// Packed bf16 pairs of an output block as the second operand of the next
// product (elements 8 ks .. 8 ks + 7).
__device__ __forceinline__ bf16x8 pack_b(const uint32_t (&pk)[8], int ks) {
  return __builtin_bit_cast(bf16x8, u32x4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]});
}

// element i of a 32x32 output block sits in row 8 (i / 4) + 4 (lane / 32) + i % 4
__device__ __forceinline__ int out_row(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

}  // namespace frag
}  // namespace rha
