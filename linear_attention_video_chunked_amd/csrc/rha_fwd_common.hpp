// Helpers shared by the bf16 forward kernels (rha_fwd_bf16.hip,
// rha_fwd_bf16_qb2.hip): tile geometry, LDS swizzles, wait immediates.
#pragma once

#include "rha_device.hpp"

namespace rha {
namespace fwd {

constexpr int BN = 64;                 // keys per LDS tile (two 32-key blocks)
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr float kLn2 = 0.6931471805599453f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = bid & 7, local = bid >> 3;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + local;
}

// phi of 8 bf16 values, rounded back to bf16.
__device__ __forceinline__ bf16x8 phi8(const bf16x8& x) {
  const u32x4 w = __builtin_bit_cast(u32x4, x);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16(phi(bf16_lo(w[i])), phi(bf16_hi(w[i])));
  return __builtin_bit_cast(bf16x8, r);
}

// Granule swizzles (16-byte granule g of row r is stored at slot g ^ sw(r)).
// K: ds_read_b128 of 16 consecutive rows at one granule hits 16 distinct slots.
template <int D> __device__ __forceinline__ int ksw(int r) { return r & (D / 8 - 1); }
// V: a transpose read covers 4 consecutive rows x 4 granules (D = 128) or
// 4 rows x 4 granules of a 128-byte row (D = 64); the swizzle puts them in
// distinct bank ranges.
template <int D> __device__ __forceinline__ int vsw(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// s_waitcnt immediate (gfx9 encoding) for "at most n vector-memory loads
// outstanding", leaving the other counters alone.
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkm0 = 0xC07F;
// Fourth word of a raw buffer descriptor on gfx9-class GPUs (32-bit format,
// no swizzle); out-of-range reads return zero.
constexpr int kBufWord3 = 0x00020000;

}  // namespace fwd
}  // namespace rha
