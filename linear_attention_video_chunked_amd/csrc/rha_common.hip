// Small memory-bound kernels: the lagged prefix over chunk states and the
// copy of a new chunk into the streaming KV cache.
#include "rha_device.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace {

// ReHyAt (abstract): the chunk-wise recurrence carries one state from chunk to
// chunk.  Slots c >= w hold per-chunk contributions on entry; on exit slot c
// holds their running sum over slots w..c, i.e. the state of every chunk up to
// c - w.  Slots c < w see no folded history and are zeroed.  Sequential float32
// sum in chunk order, the same order the streaming fold uses.
// Each thread owns 4 consecutive floats of one head's S (or z) and walks the
// slots in groups of 8: all loads of a group are issued before the running
// sum touches them, so the HBM latency is paid once per group, not per slot.
__global__ __launch_bounds__(256) void prefix_kernel(const PrefixParams p) {
  const int64_t per4 = ((int64_t)p.d * p.d + p.d) / 4;  // float4 units per head (d is a multiple of 4)
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.BH * per4) return;
  const int64_t bh = idx / per4, e4 = idx % per4;
  const int64_t dd4 = (int64_t)p.d * p.d / 4;
  f32x4* base;
  int64_t stride;  // in float4 units
  if (e4 < dd4) {
    stride = dd4;
    base = reinterpret_cast<f32x4*>(p.S) + bh * p.N * stride + e4;
  } else {
    stride = p.d / 4;
    base = reinterpret_cast<f32x4*>(p.z) + bh * p.N * stride + (e4 - dd4);
  }
  const int w = min(p.w, p.N);
  for (int c = 0; c < w; ++c) base[c * stride] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int G = 8;
  for (int c0 = w; c0 < p.N; c0 += G) {
    f32x4 v[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (c0 + g < p.N) v[g] = base[(c0 + g) * stride];
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (c0 + g < p.N) {
        acc = (c0 + g == w) ? v[g] : acc + v[g];
        base[(c0 + g) * stride] = acc;
      }
  }
}

// 16-byte copy of one [B,H,C,d] chunk (strided rows) into slot `slot` of a
// contiguous [B,H,w,C,d] cache; with src2 set, a second chunk into dst2 in
// the same launch (the upper half of the grid).
__global__ __launch_bounds__(256) void copy_chunk_kernel(const CopyParams p) {
  const int row_vecs = p.d * p.elem_bytes / 16;
  const int64_t total = (int64_t)p.B * p.H * p.C * row_vecs;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const void* srcp = p.src;
  void* dstp = p.dst;
  if (idx >= total) {
    if (p.src2 == nullptr || idx >= 2 * total) return;
    idx -= total;
    srcp = p.src2;
    dstp = p.dst2;
  }
  const int vcol = (int)(idx % row_vecs);
  const int64_t r = idx / row_vecs;
  const int t = (int)(r % p.C);
  const int64_t bh = r / p.C;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const unsigned char* src = (const unsigned char*)srcp +
                             ((int64_t)b * p.sb + (int64_t)h * p.sh + (int64_t)t * p.st) * p.elem_bytes +
                             vcol * 16;
  unsigned char* dst = (unsigned char*)dstp +
                       (((bh * p.w + p.slot) * p.C + t) * (int64_t)p.d) * p.elem_bytes + vcol * 16;
  st16(dst, ld16(src));
}

}  // namespace

hipError_t launch_prefix(const PrefixParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.BH * ((int64_t)p.d * p.d + p.d) / 4;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(prefix_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_copy_chunk(const CopyParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.H * p.C * (p.d * p.elem_bytes / 16) * (p.src2 != nullptr ? 2 : 1);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_chunk_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace rha
