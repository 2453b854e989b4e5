// The hybrid forward without a softmax window (window of 0 chunks), bf16,
// head_dim 128, on gfx950.
//
// With no window every key is in the linear term, and the state of chunk c
// includes chunk c itself: out_i = phi(q_i)^T S_c / phi(q_i).z_c.  This is
// chunk-causal linear attention ("Transformers are RNNs", section 3.2, with
// the state taken at chunk granularity: ReHyAt and the Hybrid Forcing
// explainer, section 2.A, with the softmax window emptied).
//
// The work per row is one 128 x 128 product against the chunk's state, so
// the call reads q and writes out at about 64 flops per byte moved: it is
// bound by HBM, not by the matrix cores.  A light workgroup (128 rows, 4 waves of
// 32 rows, about 150 registers a lane) lets three workgroups share a compute
// unit and hide each other's load latency; the windowed kernel, built for
// long windows, holds a compute unit alone.  The workgroups of a chunk run on
// one XCD (consecutive logical tiles per XCD), so each workgroup's copy of S_c
// after the first comes from that XCD's L2 rather than from memory: 42 us
// instead of 54-60 us for 21 chunks of 1560 rows and 12 heads, where the
// state slots re-read by every 128-row workgroup would otherwise move about
// as many bytes as q and out.  The arithmetic is the windowed kernel's
// seeding step at reference 0: S_c rounded to bf16, phi(q) rounded to bf16,
// float32 products in the same order, the denominator summed in float32.
#include "rha_device.hpp"
#include "rha_frag.hpp"
#include "rha_fwd_common.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace {

using namespace frag;

constexpr int NWL = 4;           // waves per workgroup
constexpr int TBL = NWL * 64;    // threads per workgroup
constexpr int LQB = 1;           // 32-row query blocks per wave (2: one wave per SIMD, 70% slower)
constexpr bool LXCD = true;      // tiles of a chunk on one XCD
constexpr int RPW = NWL * 32 * LQB;  // rows per workgroup

__global__ __launch_bounds__(TBL) void fwd_linear_bf16_kernel(const FwdParams p) {
  // S_c^T as bf16 rows (row m = column m of S_c); afterwards each wave's
  // 32 output rows at a time (8 KiB per wave)
  __shared__ __attribute__((aligned(1024))) unsigned char st[BD * BD * 2];
  __shared__ __attribute__((aligned(16))) float zs[BD];  // z_c
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int rtiles = (p.C + RPW - 1) / RPW;
  const int logical = LXCD ? fwd::xcd_remap(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int tile = logical % rtiles, rest = logical / rtiles;
  const int c = rest % p.n_qchunks, bh = rest / p.n_qchunks;
  const int b = bh / p.H, h = bh % p.H;
  const float* S = p.S + ((int64_t)bh * p.n_qchunks + c) * BD * BD;
  const float* z = p.z + ((int64_t)bh * p.n_qchunks + c) * BD;

  // S_c^T: unit u covers rows e = 8 eg .. 8 eg + 7 and columns n = 4 ng .. 4 ng + 3
  // of S_c; column n becomes granule eg of LDS row n
  constexpr int UNITS = (BD / 8) * (BD / 4), UPT = UNITS / TBL;
  static_assert(UPT * TBL == UNITS, "whole units per thread");
  f32x4 rows[UPT][8];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = tid + TBL * k, eg = u / (BD / 4), ng = u % (BD / 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) rows[k][i] = *reinterpret_cast<const f32x4*>(S + (int64_t)(eg * 8 + i) * BD + ng * 4);
  }
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = tid + TBL * k, eg = u / (BD / 4), ng = u % (BD / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16(rows[k][2 * i][j], rows[k][2 * i + 1][j]);
      put_granule(st, ng * 4 + j, eg, w);
    }
  }
  if (tid < BD) zs[tid] = z[tid];
  // this lane's q rows (features 16 ks + 8 hh .. + 7), loaded once the S
  // values are in LDS (fewer registers live at once); query block qb of the
  // wave covers rows r0(qb) .. r0(qb) + 31 of the chunk
  auto r0 = [&](int qb) { return RPW * tile + 32 * (LQB * wave + qb); };
  u32x4 qw[LQB][8];
#pragma unroll
  for (int qb = 0; qb < LQB; ++qb) {
    const bool ok = l32 < p.C - r0(qb);
    const bf16_t* qrow = (const bf16_t*)p.q + b * p.q_sb + h * p.q_sh + ((int64_t)c * p.C + r0(qb) + l32) * p.q_st;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qw[qb][ks] = ok ? ld16(qrow + 16 * ks + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // O^T = S_c^T phi(Q)^T (output feature m on the rows, query on the lanes)
  f32x16 o[LQB][4];
  float lz[LQB];
#pragma unroll
  for (int qb = 0; qb < LQB; ++qb) {
    lz[qb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) o[qb][mb] = f32x16{};
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(zs + 16 * ks + 8 * hh);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(zs + 16 * ks + 8 * hh + 4);
    bf16x8 pf[LQB];
#pragma unroll
    for (int qb = 0; qb < LQB; ++qb) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = phi(bf16_lo(qw[qb][ks][i]));
        f[2 * i + 1] = phi(bf16_hi(qw[qb][ks][i]));
      }
      lz[qb] += f[0] * z0[0] + f[1] * z0[1] + f[2] * z0[2] + f[3] * z0[3] + f[4] * z1[0] + f[5] * z1[1] +
                f[6] * z1[2] + f[7] * z1[3];
      pf[qb] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                                                pack_bf16(f[6], f[7])});
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const bf16x8 sf = row_frag(st, 32 * mb, ks, lane);
#pragma unroll
      for (int qb = 0; qb < LQB; ++qb) o[qb][mb] = mfma32(sf, pf[qb], o[qb][mb]);
    }
  }

  // normalise, stage the wave's rows in LDS (one query block at a time),
  // write them out a row per 16 lanes
  __syncthreads();  // every wave is done reading S_c^T
  unsigned char* ob = st + wave * ROWT;
#pragma unroll
  for (int qb = 0; qb < LQB; ++qb) {
    const int nr = max(0, min(32, p.C - r0(qb)));
    const int64_t tok0 = (int64_t)c * p.C + r0(qb);  // token of the block's first row
    const float ltot = half_sum(lz[qb]);  // the two halves of the features
    const float inv = 1.0f / ltot;
    if (qb > 0) __builtin_amdgcn_wave_barrier();  // the previous block's rows are read out
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int f = 32 * mb + 8 * rr + 4 * hh;
        const u32x2 pr = {pack_bf16(o[qb][mb][4 * rr] * inv, o[qb][mb][4 * rr + 1] * inv),
                          pack_bf16(o[qb][mb][4 * rr + 2] * inv, o[qb][mb][4 * rr + 3] * inv)};
        *reinterpret_cast<u32x2*>(ob + gran_off(l32, f >> 3) + (f & 7) * 2) = pr;
      }
    if (p.lse != nullptr && hh == 0 && l32 < nr) {
      const int64_t L = (int64_t)p.n_qchunks * p.C;
      p.lse[(int64_t)bh * L + tok0 + l32] = __log2f(ltot) * fwd::kLn2;
    }
    __builtin_amdgcn_s_waitcnt(fwd::kWaitLgkm0);  // this wave's staging writes are complete
    __builtin_amdgcn_wave_barrier();
    bf16_t* obase = (bf16_t*)p.out + b * p.q_sb + h * p.q_sh + tok0 * p.q_st;
#pragma unroll
    for (int idx = lane; idx < 32 * (BD / 8); idx += 64) {
      const int r = idx / (BD / 8), g = idx % (BD / 8);
      if (r < nr) st16(obase + (int64_t)r * p.q_st + g * 8, *reinterpret_cast<const u32x4*>(ob + gran_off(r, g)));
    }
    __builtin_amdgcn_s_waitcnt(fwd::kWaitLgkm0);  // the staged rows are read
  }
}

}  // namespace

hipError_t launch_fwd_linear_bf16(const FwdParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.H * p.n_qchunks * ((p.C + RPW - 1) / RPW);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_linear_bf16_kernel, dim3((unsigned)blocks), dim3(TBL), 0, s, p);
  return hipGetLastError();
}

}  // namespace rha
