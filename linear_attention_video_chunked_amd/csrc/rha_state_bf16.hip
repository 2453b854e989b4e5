// Per-chunk linear-attention state contributions for bf16 inputs on gfx950.
//
// For every requested chunk c: U_c = phi(K_c)^T V_c (d x d, float32) and
// u_c = sum_{t in c} phi(k_t) (d, float32) -- the linear-attention state of
// "Transformers are RNNs" restricted to one chunk.  "Long-Horizon Streaming
// Video Generation via Hybrid Attention with Decoupled Distillation"
// (explainer, section 2.A) folds each frame that leaves the sliding window into
// this state; "ReHyAt" (abstract) evaluates the same quantity chunk by chunk.
//
// One workgroup per (head, chunk): 4 waves, each owning a 32-row block of the
// feature axis e of U (all of n for d = 128).  Tokens stream through LDS in
// tiles of 64; both operands are contracted over tokens, so both phi(K) and V
// are stored transposed (8 consecutive tokens per 16-byte MFMA fragment) by an
// in-register 4x8 transpose of the 16-byte global loads.  phi is evaluated in
// float32 and rounded to bf16 for the product; u is summed from the float32
// phi values in a fixed order.  With `accumulate` the result is added into
// the destination (the streaming fold), otherwise it is stored.
#include "rha_device.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace {

constexpr int NW = 4;
constexpr int THREADS = NW * kWave;
constexpr int BT = 64;  // tokens per tile

template <int D>
struct StateCfg {
  static constexpr int TBYTES = BT * D * 2;        // one transposed tile
  static constexpr int UNITS = (BT / 4) * (D / 8);  // 4-token x 8-feature load units
  static constexpr int EB = D / 32;
  static constexpr int NBW = EB * EB / NW;          // output 32x32 blocks per wave
  static_assert(UNITS <= THREADS, "one unit per thread at most");
  static_assert(NBW >= 1, "at least one block per wave");
};

// Store a 4-token x 8-feature unit transposed: tokens 4*tq .. +3 of the tile.
// Layout: element (token t, feature f) of the tile at ((ks*2 + g)*D + f)*8 + i
// where ks = t/16 and (g, i) follow the MFMA k-order used for both operands.
template <int D>
__device__ __forceinline__ void store_unit_t(unsigned char* tbuf, int tq, int fo, const uint32_t (&w)[4][4]) {
  const int ks = tq >> 2, m = tq & 3;
  const int g = m & 1, e0 = (m >> 1) * 4;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int wd = f >> 1, sh = (f & 1) * 16;
    const uint32_t x0 = (w[0][wd] >> sh) & 0xffffu, x1 = (w[1][wd] >> sh) & 0xffffu;
    const uint32_t x2 = (w[2][wd] >> sh) & 0xffffu, x3 = (w[3][wd] >> sh) & 0xffffu;
    u32x2 pr = {x0 | (x1 << 16), x2 | (x3 << 16)};
    *reinterpret_cast<u32x2*>(tbuf + (((size_t)(ks * 2 + g) * D + fo * 8 + f) * 8 + e0) * 2) = pr;
  }
}

template <int D>
__global__ __launch_bounds__(THREADS) void chunk_state_bf16_kernel(const ChunkStateParams p) {
  using Cfg = StateCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * Cfg::TBYTES];
  __shared__ float zred[BT / 4][D];
  unsigned char* const kt0 = smem;                      // phi(K)^T, 2 buffers
  unsigned char* const vt0 = smem + 2 * Cfg::TBYTES;    // V^T, 2 buffers

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  const int jc = blockIdx.x % p.n_chunks;
  const int bh = blockIdx.x / p.n_chunks;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t t0 = (int64_t)(p.chunk0 + jc) * p.C;
  const bf16_t* kbase = (const bf16_t*)p.k + b * p.kv_sb + h * p.kv_sh + t0 * p.kv_st;
  const bf16_t* vbase = (const bf16_t*)p.v + b * p.kv_sb + h * p.kv_sh + t0 * p.kv_st;

  const bool active = Cfg::UNITS == THREADS || tid < Cfg::UNITS;
  const int fo = tid % (D / 8), tq = tid / (D / 8);

  int eb, nb0;
  if (Cfg::EB == 4) {
    eb = wave;
    nb0 = 0;
  } else {
    eb = wave >> 1;
    nb0 = wave & 1;
  }

  f32x16 acc[Cfg::NBW];
#pragma unroll
  for (int i = 0; i < Cfg::NBW; ++i) acc[i] = f32x16{};
  float zacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zacc[i] = 0.f;

  const int ntiles = (p.C + BT - 1) / BT;
  uint32_t kw[4][4], vw[4][4];

  auto gload = [&](int j) {
    if (!active) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = j * BT + tq * 4 + r;
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (t < p.C) {
        xk = ld16(kbase + (int64_t)t * p.kv_st + fo * 8);
        xv = ld16(vbase + (int64_t)t * p.kv_st + fo * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kw[r][i] = xk[i];
        vw[r][i] = xv[i];
      }
    }
  };
  auto lstore = [&](int j, int buf) {
    if (!active) return;
    uint32_t fw[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = j * BT + tq * 4 + r < p.C;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = ok ? phi(bf16_lo(kw[r][i])) : 0.f;
        const float c = ok ? phi(bf16_hi(kw[r][i])) : 0.f;
        zacc[2 * i] += a;
        zacc[2 * i + 1] += c;
        fw[r][i] = pack_bf16(a, c);
      }
    }
    store_unit_t<D>(kt0 + buf * Cfg::TBYTES, tq, fo, fw);
    store_unit_t<D>(vt0 + buf * Cfg::TBYTES, tq, fo, vw);
  };

  gload(0);
  lstore(0, 0);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    const unsigned char* kt = kt0 + buf * Cfg::TBYTES;
    const unsigned char* vt = vt0 + buf * Cfg::TBYTES;
#pragma unroll
    for (int ks = 0; ks < BT / 16; ++ks) {
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(kt + ((size_t)(ks * 2 + hh) * D + eb * 32 + l32) * 16));
#pragma unroll
      for (int i = 0; i < Cfg::NBW; ++i) {
        const int nb = nb0 + i;
        const bf16x8 bb = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(vt + ((size_t)(ks * 2 + hh) * D + nb * 32 + l32) * 16));
        acc[i] = mfma32(a, bb, acc[i]);
      }
    }
    if (j + 1 < ntiles) lstore(j + 1, buf ^ 1);
    __syncthreads();
  }

  // U: acc[i] reg 4r+q <-> e = eb*32 + 8r + 4hh + q, n = (nb0+i)*32 + l32
  float* Sdst = p.S + (int64_t)bh * p.s_bh + (int64_t)(jc + p.slot_offset) * D * D;
#pragma unroll
  for (int i = 0; i < Cfg::NBW; ++i) {
    const int n = (nb0 + i) * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = eb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      float* dst = Sdst + (int64_t)e * D + n;
      const float val = acc[i][r];
      *dst = p.accumulate ? *dst + val : val;
    }
  }

  // u: fixed-order reduction of the per-thread partial sums
  if (active) {
#pragma unroll
    for (int i = 0; i < 8; ++i) zred[tq][fo * 8 + i] = zacc[i];
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < BT / 4; ++r) s += zred[r][tid];
    float* zd = p.z + (int64_t)bh * p.z_bh + (int64_t)(jc + p.slot_offset) * D + tid;
    *zd = p.accumulate ? *zd + s : s;
  }
}

}  // namespace

hipError_t launch_chunk_state_bf16(const ChunkStateParams& p, int d, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.H * p.n_chunks));
  if (d == 128)
    hipLaunchKernelGGL(chunk_state_bf16_kernel<128>, grid, dim3(THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(chunk_state_bf16_kernel<64>, grid, dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace rha
