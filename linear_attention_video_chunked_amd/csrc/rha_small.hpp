// Bodies of the small memory-bound steps, shared by their own kernels and by
// the launches that run them next to other work (the streaming step fuses
// the cache copy with the fold and the two merges into one launch).
#pragma once

#include "rha_device.hpp"
#include "rha_launch.hpp"

namespace rha {

// One 16-byte unit of the cache copy: tensor `which` (0: src -> dst, 1: src2
// -> dst2), head bh, unit i of that head's C * d * elem_bytes / 16.
// Source and destination of that unit.
__device__ __forceinline__ void copy_addr(const CopyParams& p, int which, int bh, int i, const unsigned char*& src,
                                          unsigned char*& dst) {
  const int row_vecs = p.d * p.elem_bytes / 16;
  const void* srcp = which ? p.src2 : p.src;
  void* dstp = which ? p.dst2 : p.dst;
  const int t = i / row_vecs, vcol = i - t * row_vecs;
  const int b = bh / p.H, h = bh - b * p.H;
  src = (const unsigned char*)srcp + ((int64_t)b * p.sb + (int64_t)h * p.sh + (int64_t)t * p.st) * p.elem_bytes +
        vcol * 16;
  dst = (unsigned char*)dstp + ((((int64_t)bh * p.w + p.slot) * p.C + t) * (int64_t)p.d) * p.elem_bytes + vcol * 16;
}

__device__ __forceinline__ void copy_unit(const CopyParams& p, int which, int bh, int i) {
  if (i >= p.C * (p.d * p.elem_bytes / 16)) return;
  const unsigned char* src;
  unsigned char* dst;
  copy_addr(p, which, bh, i, src, dst);
  st16(dst, ld16(src));
}

// One float4 of the state merge: S[bh] += sum_g part_S[bh][g] (likewise z),
// the partial sums added in g order first; idx runs over B*H*(d*d + d)/4.
__device__ __forceinline__ void state_combine_unit(const StateCombineParams& p, int64_t idx) {
  const int per = (p.d * p.d + p.d) / 4;  // float4 units per head
  if (idx >= (int64_t)p.BH * per) return;
  const int bh = (int)(idx / per), r = (int)(idx - (int64_t)bh * per);
  const int sq = p.d * p.d / 4;
  const float* src;
  int64_t gstride;
  float* dst;
  if (r < sq) {
    src = p.part + ((int64_t)bh * p.G * p.d * p.d) + 4 * r;
    gstride = (int64_t)p.d * p.d;
    dst = p.S + (int64_t)bh * p.d * p.d + 4 * r;
  } else {
    src = p.part + (int64_t)p.BH * p.G * p.d * p.d + (int64_t)bh * p.G * p.d + 4 * (r - sq);
    gstride = p.d;
    dst = p.z + (int64_t)bh * p.d + 4 * (r - sq);
  }
  // groups of eight loads in flight, added in g order
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int g = 0;
  for (; g + 8 <= p.G; g += 8) {
    f32x4 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = *reinterpret_cast<const f32x4*>(src + (g + i) * gstride);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += x[i];
  }
  for (; g < p.G; ++g) acc += *reinterpret_cast<const f32x4*>(src + g * gstride);
  *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(dst) + acc;
}

}  // namespace rha
