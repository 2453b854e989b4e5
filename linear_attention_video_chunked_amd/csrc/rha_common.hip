// Small memory-bound kernels: the lagged prefix over chunk states and the
// copy of a new chunk into the streaming KV cache.
#include "rha_device.hpp"
#include "rha_launch.hpp"
#include "rha_small.hpp"

namespace rha {
namespace {

// ReHyAt (abstract): the chunk-wise recurrence carries one state from chunk to
// chunk.  Slots c >= w hold per-chunk contributions on entry; on exit slot c
// holds their running sum over slots w..c, i.e. the state of every chunk up to
// c - w.  Slots c < w see no folded history and are zeroed.  Sequential float32
// sum in chunk order, the same order the streaming fold uses.  With reverse
// the slots are walked from the last (the future part of a bidirectional
// state: slot c sums the contributions stored in slots c .. N-1-w).
// Each thread owns 4 consecutive floats of one head's S (or z) and walks the
// slots in groups of 24: all loads of a group are issued before the running
// sum touches them, so the HBM latency is paid once per group, not per slot
// (once in all for up to 24 summed slots); 128-thread workgroups spread the
// few threads over more compute units.
__global__ __launch_bounds__(128) void prefix_kernel(const PrefixParams p) {
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
  if (p.reverse) {  // the same walk over slots N-1, N-2, .. 0 (a suffix)
    base += (int64_t)(p.N - 1) * stride;
    stride = -stride;
  }
  const int w = min(p.w, p.N);
  for (int c = 0; c < w; ++c) base[c * stride] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int G = 24;
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
// contiguous [B,H,w,C,d] cache; with src2 set, a second chunk into dst2
// (blockIdx.y = 1).  blockIdx.x = bh * blocks_per_bh + block within the head,
// so every per-thread index is 32-bit.
__global__ __launch_bounds__(256) void copy_chunk_kernel(const CopyParams p, int blocks_per_bh) {
  const int bh = blockIdx.x / blocks_per_bh;
  copy_unit(p, blockIdx.y, bh, (blockIdx.x - bh * blocks_per_bh) * 256 + threadIdx.x);
}

__global__ __launch_bounds__(64) void state_combine_kernel(const StateCombineParams p) {
  state_combine_unit(p, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

}  // namespace

hipError_t launch_prefix(const PrefixParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.BH * ((int64_t)p.d * p.d + p.d) / 4;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(prefix_kernel, dim3((unsigned)((total + 127) / 128)), dim3(128), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_copy_chunk(const CopyParams& p, hipStream_t s) {
  const int64_t per_bh = (int64_t)p.C * (p.d * p.elem_bytes / 16);
  const int64_t BH = (int64_t)p.B * p.H;
  if (per_bh == 0 || BH == 0) return hipSuccess;
  const int blocks_per_bh = (int)((per_bh + 255) / 256);
  hipLaunchKernelGGL(copy_chunk_kernel, dim3((unsigned)(BH * blocks_per_bh), p.src2 != nullptr ? 2u : 1u), dim3(256), 0, s,
                     p, blocks_per_bh);
  return hipGetLastError();
}

hipError_t launch_state_combine(const StateCombineParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.BH * ((int64_t)p.d * p.d + p.d) / 4;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(state_combine_kernel, dim3((unsigned)((total + 63) / 64)), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace rha
