// Fused hybrid-attention forward for bf16 inputs on gfx950 matrix cores.
//
// Computes, per query row i of chunk c (window and history as defined in
// include/rha.h):
//   out_i = (sum_{j in window} exp(s_ij) v_j + phi(q_i)^T S_c)
//         / (sum_{j in window} exp(s_ij)     + phi(q_i)^T z_c)
// following "Long-Horizon Streaming Video Generation via Hybrid Attention with
// Decoupled Distillation" (explainer, section 2.A: window attention computed
// in FlashAttention-style blocks, folded linear state for evicted frames).
//
// Design (gfx950, wave64, 32x32x16 bf16 MFMA):
//  * one workgroup = 4 waves = one query tile of 128*QB rows inside one chunk;
//    each wave owns 32*QB query rows, kept in registers as MFMA B operands.
//  * scores are produced transposed, S^T = K Q^T (M = keys, N = queries), so
//    every lane holds one query's scores: the row max and row sum need one
//    lane-pair exchange (v_permlane32_swap) instead of a 32-lane reduction,
//    and the probabilities are already laid out as the B operand of
//    O^T += V^T P^T.  The output accumulators are O^T, again one query per
//    lane, so rescaling and normalisation are lane-local.
//  * the linear term seeds the accumulators: O^T = S_c^T phi(Q)^T and
//    l = phi(Q).z_c at reference maximum 0 (the same as multiplying it by
//    exp(-m) at the end), then the window keys are streamed in tiles of 64
//    with an online maximum.  Rescaling is lazy: the reference maximum only
//    moves when a new score exceeds it by more than 2^8, which keeps every
//    probability <= 256 and leaves the result unchanged.
//  * K tiles live in LDS row-major (padded rows); V tiles live in LDS
//    transposed into the 8-keys-per-lane order the MFMA A operand wants,
//    built from 16-byte global loads by an in-register 4x8 transpose.
//    Tiles are double-buffered: the global loads of tile j+1 are in flight
//    while tile j is multiplied.
//  * workgroup ids are remapped so that each of the 8 XCDs gets a contiguous
//    range of tiles; neighbouring tiles share their window keys in that XCD's
//    L2.
#include "rha_device.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace {

constexpr int NW = 4;
constexpr int THREADS = NW * kWave;
constexpr int BN = 64;            // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = bid & 7, local = bid >> 3;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + local;
}

__device__ __forceinline__ bf16x8 lds_frag(const unsigned char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// phi of 8 bf16 values, rounded back to bf16.
__device__ __forceinline__ bf16x8 phi8(const bf16x8& x) {
  const u32x4 w = __builtin_bit_cast(u32x4, x);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16(phi(bf16_lo(w[i])), phi(bf16_hi(w[i])));
  return __builtin_bit_cast(bf16x8, r);
}

template <int D, int QB>
struct FwdCfg {
  static constexpr int BM = NW * 32 * QB;
  static constexpr int DS = D / 16;                 // MFMA k-steps over features
  static constexpr int DB = D / 32;                 // 32-wide feature blocks
  static constexpr int KPITCH = D * 2 + 16;         // padded K row in LDS (bytes)
  static constexpr int KBYTES = BN * KPITCH;
  static constexpr int VTBYTES = BN * D * 2;
  static constexpr int STBYTES = D * D * 2;         // bf16 state staged for the linear term
  static constexpr int OPITCH = D * 2 + 16;
  static constexpr int MAIN = 2 * KBYTES + 2 * VTBYTES;
  static constexpr int OUT = BM * OPITCH;
  static constexpr int LDS = MAIN > OUT ? MAIN : OUT;
  static constexpr int KCH = BN * (D / 8) / THREADS;   // 16-byte K chunks per thread
  static constexpr int VUNITS = (BN / 4) * (D / 8);    // 4-key x 8-feature V units
  static_assert(2 * VTBYTES >= STBYTES, "state staging must fit the V buffers");
  static_assert(KCH * THREADS == BN * (D / 8), "K tile must split evenly");
  static_assert(VUNITS <= THREADS, "one V unit per thread at most");
};

template <int D, int QB>
__global__ __launch_bounds__(THREADS) void fwd_bf16_kernel(const FwdParams p) {
  using Cfg = FwdCfg<D, QB>;
  constexpr int BM = Cfg::BM, DS = Cfg::DS, DB = Cfg::DB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::LDS];
  unsigned char* const kbuf0 = smem;
  unsigned char* const vtbuf0 = smem + 2 * Cfg::KBYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- which tile
  const int logical = xcd_remap(blockIdx.x, p.total_tiles);
  const int tile = logical % p.tiles_per_chunk;
  const int rest = logical / p.tiles_per_chunk;
  const int c = p.n_qchunks - 1 - rest % p.n_qchunks;  // later chunks (longer windows) first
  const int bh = rest / p.n_qchunks;
  const int b = bh / p.H, h = bh % p.H;
  const int qrow0 = tile * BM;
  const int nrows = min(BM, p.C - qrow0);
  const int64_t qtok0 = (int64_t)c * p.C + qrow0;

  const bf16_t* qbase = (const bf16_t*)p.q + b * p.q_sb + h * p.q_sh + qtok0 * p.q_st;
  const bf16_t* kbase = (const bf16_t*)p.k + b * p.kv_sb + h * p.kv_sh;
  const bf16_t* vbase = (const bf16_t*)p.v + b * p.kv_sb + h * p.kv_sh;

  int64_t kbeg, kend;
  bool has_state;
  const float* Sp;
  const float* zp;
  if (!p.stream_mode) {
    if (p.w > 0) {
      kbeg = (int64_t)max(0, c - p.w + 1) * p.C;
      kend = (int64_t)(c + 1) * p.C;
    } else {
      kbeg = kend = 0;
    }
    has_state = (p.w == 0) || (c >= p.w);
    Sp = p.S + ((int64_t)bh * p.n_qchunks + c) * D * D;
    zp = p.z + ((int64_t)bh * p.n_qchunks + c) * D;
  } else {
    kbeg = 0;
    kend = p.n_keys;
    has_state = p.has_state != 0;
    Sp = p.S + (int64_t)bh * D * D;
    zp = p.z + (int64_t)bh * D;
  }

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[row l32][16s + 8hh .. +7]
  bf16x8 qf[QB][DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wave * 32 * QB + qb * 32 + l32;
    const bool ok = row < nrows;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = ld16(qbase + (int64_t)row * p.q_st + s * 16 + hh * 8);
      qf[qb][s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 o[QB][DB];
  float lsum[QB], mrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    lsum[qb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < DB; ++nb) o[qb][nb] = f32x16{};
  }

  // ---- linear term: O^T = S^T phi(Q)^T, l = phi(Q).z, at reference max 0
  if (has_state) {
    // Stage S (float32 [D][D]) as bf16 in LDS, laid out as MFMA A fragments:
    // element (e = 16s + 8g + i, n) at ((s*2 + g)*D + n)*8 + i.
    constexpr int SUNITS = (D / 8) * (D / 4);  // 8 rows x 4 columns each
    for (int u = tid; u < SUNITS; u += THREADS) {
      const int eg = u / (D / 4), ng = u % (D / 4);
      f32x4 rows[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rows[i] = *reinterpret_cast<const f32x4*>(Sp + (int64_t)(eg * 8 + i) * D + ng * 4);
      const int s = eg >> 1, g = eg & 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack_bf16(rows[2 * i][j], rows[2 * i + 1][j]);
        st16(vtbuf0 + ((size_t)(s * 2 + g) * D + ng * 4 + j) * 16, pk);
      }
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float lz = 0.f;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 pf = phi8(qf[qb][s]);
        const u32x4 qw = __builtin_bit_cast(u32x4, qf[qb][s]);
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zp + s * 16 + hh * 8);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(zp + s * 16 + hh * 8 + 4);
        lz += phi(bf16_lo(qw[0])) * z0[0] + phi(bf16_hi(qw[0])) * z0[1] +
              phi(bf16_lo(qw[1])) * z0[2] + phi(bf16_hi(qw[1])) * z0[3] +
              phi(bf16_lo(qw[2])) * z1[0] + phi(bf16_hi(qw[2])) * z1[1] +
              phi(bf16_lo(qw[3])) * z1[2] + phi(bf16_hi(qw[3])) * z1[3];
#pragma unroll
        for (int nb = 0; nb < DB; ++nb) {
          const bf16x8 a = lds_frag(vtbuf0 + ((size_t)(s * 2 + hh) * D + nb * 32 + l32) * 16);
          o[qb][nb] = mfma32(a, pf, o[qb][nb]);
        }
      }
      lsum[qb] = lz;  // this lane's half of the features; halves are summed at the end
      mrun[qb] = 0.f;
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mrun[qb] = -INFINITY;
  }

  // ---- window keys
  const int ntiles = (int)((kend - kbeg + BN - 1) / BN);
  u32x4 kreg[Cfg::KCH];
  u32x4 vreg[4];
  const int vfo = tid % (D / 8), vkq = tid / (D / 8);

  auto gload = [&](int j) {
    const int64_t k0 = kbeg + (int64_t)j * BN;
#pragma unroll
    for (int i = 0; i < Cfg::KCH; ++i) {
      const int idx = tid + i * THREADS;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      const int64_t key = k0 + row;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < kend) x = ld16(kbase + key * p.kv_st + ch * 8);
      kreg[i] = x;
    }
    if (Cfg::VUNITS == THREADS || tid < Cfg::VUNITS) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t key = k0 + vkq * 4 + jj;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < kend) x = ld16(vbase + key * p.kv_st + vfo * 8);
        vreg[jj] = x;
      }
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* kb = kbuf0 + buf * Cfg::KBYTES;
    unsigned char* vt = vtbuf0 + buf * Cfg::VTBYTES;
#pragma unroll
    for (int i = 0; i < Cfg::KCH; ++i) {
      const int idx = tid + i * THREADS;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      st16(kb + row * Cfg::KPITCH + ch * 16, kreg[i]);
    }
    if (Cfg::VUNITS == THREADS || tid < Cfg::VUNITS) {
      // keys 4*vkq .. +3 of the tile: 16-key step ks, quarter m of that step.
      // MFMA k-order inside a 16-key step: lane half g takes keys
      // {4g..4g+3, 8+4g..8+4g+3}; quarter m -> half g = m & 1, slot 4*(m >> 1).
      const int ks = vkq >> 2, m = vkq & 3;
      const int g = m & 1, e0 = (m >> 1) * 4;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int wd = f >> 1;
        const int sh = (f & 1) * 16;
        const uint32_t x0 = (vreg[0][wd] >> sh) & 0xffffu, x1 = (vreg[1][wd] >> sh) & 0xffffu;
        const uint32_t x2 = (vreg[2][wd] >> sh) & 0xffffu, x3 = (vreg[3][wd] >> sh) & 0xffffu;
        u32x2 pr = {x0 | (x1 << 16), x2 | (x3 << 16)};
        *reinterpret_cast<u32x2*>(vt + (((size_t)(ks * 2 + g) * D + vfo * 8 + f) * 8 + e0) * 2) = pr;
      }
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    const int valid = (int)min((int64_t)BN, kend - (kbeg + (int64_t)j * BN));
    const unsigned char* kb = kbuf0 + buf * Cfg::KBYTES;
    const unsigned char* vt = vtbuf0 + buf * Cfg::VTBYTES;

    // S^T = K Q^T : sacc[qb][kb] reg 4r+i <-> key kb*32 + 8r + 4hh + i, query l32
    f32x16 sacc[QB][BN / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb2 = 0; kb2 < BN / 32; ++kb2) sacc[qb][kb2] = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int kb2 = 0; kb2 < BN / 32; ++kb2) {
        const bf16x8 a = lds_frag(kb + (kb2 * 32 + l32) * Cfg::KPITCH + (s * 16 + hh * 8) * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][kb2] = mfma32(a, qf[qb][s], sacc[qb][kb2]);
      }
    }

    // online softmax (log2 domain), probabilities packed to bf16 pairs
    uint32_t pk[QB][BN / 32][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (valid < BN) {
#pragma unroll
        for (int kb2 = 0; kb2 < BN / 32; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb2 * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (key >= valid) sacc[qb][kb2][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < BN / 32; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[qb][kb2][i]);
      mx = half_max(mx) * p.scale_log2;
      const float mnew = fmaxf(mrun[qb], mx);
      if (__any(mnew > mrun[qb] + kRescaleSlack)) {
        const float alpha = __builtin_amdgcn_exp2f(mrun[qb] - mnew);
        mrun[qb] = mnew;
        lsum[qb] *= alpha;
#pragma unroll
        for (int nb = 0; nb < DB; ++nb) o[qb][nb] *= alpha;
      }
      const float mneg = -mrun[qb];
      float ps = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < BN / 32; ++kb2)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb2][2 * i], p.scale_log2, mneg));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb2][2 * i + 1], p.scale_log2, mneg));
          ps += p0 + p1;
          pk[qb][kb2][i] = pack_bf16(p0, p1);
        }
      lsum[qb] += ps;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const int kb2 = ks >> 1, r0 = (ks & 1) * 2;
      bf16x8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        u32x4 w4 = {pk[qb][kb2][r0 * 2], pk[qb][kb2][r0 * 2 + 1], pk[qb][kb2][r0 * 2 + 2],
                    pk[qb][kb2][r0 * 2 + 3]};
        pf[qb] = __builtin_bit_cast(bf16x8, w4);
      }
#pragma unroll
      for (int nb = 0; nb < DB; ++nb) {
        const bf16x8 a = lds_frag(vt + ((size_t)(ks * 2 + hh) * D + nb * 32 + l32) * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][nb] = mfma32(a, pf[qb], o[qb][nb]);
      }
    }

    if (j + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, stage bf16 rows in LDS, write coalesced
  __syncthreads();
  bf16_t* obase = (bf16_t*)p.out + b * p.q_sb + h * p.q_sh + qtok0 * p.q_st;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = half_sum(lsum[qb]);
    const float inv = 1.0f / ltot;
    const int row = wave * 32 * QB + qb * 32 + l32;
#pragma unroll
    for (int nb = 0; nb < DB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = nb * 32 + 8 * r + 4 * hh;
        u32x2 pr = {pack_bf16(o[qb][nb][4 * r] * inv, o[qb][nb][4 * r + 1] * inv),
                    pack_bf16(o[qb][nb][4 * r + 2] * inv, o[qb][nb][4 * r + 3] * inv)};
        *reinterpret_cast<u32x2*>(smem + row * Cfg::OPITCH + col * 2) = pr;
      }
    if (p.lse != nullptr && hh == 0 && row < nrows) {
      const int64_t L = (int64_t)p.n_qchunks * p.C;
      p.lse[(int64_t)bh * L + qtok0 + row] = (mrun[qb] + __log2f(ltot)) * kLn2;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < BM * (D / 8); idx += THREADS) {
    const int row = idx / (D / 8), ch = idx % (D / 8);
    if (row < nrows)
      st16(obase + (int64_t)row * p.q_st + ch * 8,
           *reinterpret_cast<const u32x4*>(smem + row * Cfg::OPITCH + ch * 16));
  }
}

template <int D, int QB>
hipError_t launch(FwdParams& p, hipStream_t s) {
  p.tiles_per_chunk = (p.C + FwdCfg<D, QB>::BM - 1) / FwdCfg<D, QB>::BM;
  p.total_tiles = p.B * p.H * p.n_qchunks * p.tiles_per_chunk;
  if (p.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB>), dim3(p.total_tiles), dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(FwdParams& p, int d, hipStream_t s) {
  if (d == 128) return launch<128, 1>(p, s);
  return launch<64, 1>(p, s);
}

}  // namespace rha
