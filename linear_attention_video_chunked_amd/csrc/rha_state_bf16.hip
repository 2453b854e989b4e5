// Per-chunk linear-attention state contributions for bf16 inputs on gfx950.
//
// For every requested chunk c: U_c = phi(K_c)^T V_c (d x d, float32) and
// u_c = sum_{t in c} phi(k_t) (d, float32) -- the linear-attention state of
// "Transformers are RNNs" restricted to one chunk.  "Long-Horizon Streaming
// Video Generation via Hybrid Attention with Decoupled Distillation"
// (explainer, section 2.A) folds each frame that leaves the sliding window into
// this state; "ReHyAt" (abstract) evaluates the same quantity chunk by chunk.
// The workgroup-level computation is chunk_state_unit (rha_state_unit.hpp);
// this kernel runs it for every (head, chunk, slice) and, in extra
// workgroups, an optional cache copy.
#include "rha_device.hpp"
#include "rha_fwd_common.hpp"
#include "rha_launch.hpp"
#include "rha_small.hpp"
#include "rha_state_unit.hpp"

namespace rha {
namespace {

using namespace state;

template <int D, bool SCALED>
__global__ __launch_bounds__(THREADS) void chunk_state_bf16_kernel(const ChunkStateParams p) {
  using Cfg = StateCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char kt_s[2][Cfg::KBYTES];  // phi(K) slice, 2 buffers
  __shared__ __attribute__((aligned(1024))) unsigned char vt_s[2][Cfg::VBYTES];  // V, 2 buffers
  __shared__ float zred[THREADS / (ESLICE / 8)][ESLICE];
  // slices of one chunk are adjacent in the logical order, which keeps them
  // on one XCD (one L2) so V is fetched from HBM once
  const int total = p.B * p.H * p.n_chunks * Cfg::ES;
  if ((int)blockIdx.x >= total) {  // the launch's extra workgroups: the cache copy
    const int cb = blockIdx.x - total;
    const int pair = cb / p.copy_blocks_per_bh;  // (tensor, head)
    const int BH = p.B * p.H;
    copy_unit(p.copy, pair / BH, pair % BH, (cb - pair * p.copy_blocks_per_bh) * THREADS + (int)threadIdx.x);
    return;
  }
  chunk_state_unit<D, SCALED>(p, fwd::xcd_remap(blockIdx.x, total), &kt_s[0][0], vt_s[0], vt_s[1], &zred[0][0]);
}

// Head dimension 128 without a cache copy: one workgroup per (head, chunk)
// with a thread group per slice of e, so each chunk's V is loaded and staged
// once (the same bits as the one-slice workgroups).
template <bool SCALED>
__global__ __launch_bounds__(2 * THREADS) void chunk_state_bf16_both_kernel(const ChunkStateParams p) {
  using Cfg = StateCfg<128>;
  static_assert(Cfg::ES == 2, "two slices of 64 rows");
  __shared__ __attribute__((aligned(1024))) unsigned char kt_s[2][2][Cfg::KBYTES];  // per slice, 2 buffers
  __shared__ __attribute__((aligned(1024))) unsigned char vt_s[2][Cfg::VBYTES];
  __shared__ float zred[2][THREADS / (ESLICE / 8)][ESLICE];
  const int total = p.B * p.H * p.n_chunks;
  chunk_state_unit<128, SCALED, 2, 4>(p, fwd::xcd_remap(blockIdx.x, total), &kt_s[0][0][0], vt_s[0], vt_s[1],
                                      &zred[0][0][0]);
}

}  // namespace

hipError_t launch_chunk_state_bf16(const ChunkStateParams& p, int d, hipStream_t s) {
  const int64_t heads_chunks = (int64_t)p.B * p.H * p.n_chunks;
  // extra workgroups for a cache copy in the same launch (2 tensors x B*H heads)
  const int64_t copy_blocks = p.copy.src != nullptr ? 2 * (int64_t)p.B * p.H * p.copy_blocks_per_bh : 0;
  const bool scaled = p.vscale != nullptr;
  const dim3 g128((unsigned)(heads_chunks * StateCfg<128>::ES + copy_blocks));
  const dim3 g64((unsigned)(heads_chunks * StateCfg<64>::ES + copy_blocks));
  if (d == 128 && copy_blocks == 0 && !scaled) {
    hipLaunchKernelGGL((chunk_state_bf16_both_kernel<false>), dim3((unsigned)heads_chunks), dim3(2 * THREADS), 0, s, p);
  } else if (d == 128 && copy_blocks == 0) {  // scaled (the backward pass's state gradients)
    hipLaunchKernelGGL((chunk_state_bf16_both_kernel<true>), dim3((unsigned)heads_chunks), dim3(2 * THREADS), 0, s, p);
  } else if (d == 128 && scaled)
    hipLaunchKernelGGL((chunk_state_bf16_kernel<128, true>), g128, dim3(THREADS), 0, s, p);
  else if (d == 128)
    hipLaunchKernelGGL((chunk_state_bf16_kernel<128, false>), g128, dim3(THREADS), 0, s, p);
  else if (scaled)
    hipLaunchKernelGGL((chunk_state_bf16_kernel<64, true>), g64, dim3(THREADS), 0, s, p);
  else
    hipLaunchKernelGGL((chunk_state_bf16_kernel<64, false>), g64, dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace rha
