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
//  * one workgroup = 4 waves = one query tile of 128 rows inside one chunk;
//    each wave owns 32 query rows, kept in registers as MFMA B operands.
//    Two workgroups share a CU (<= 256 registers per wave, 64 KB LDS each),
//    so one wave's softmax overlaps another's matrix products.
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
//  * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4:
//    no registers, no VALU), row-major with an XOR swizzle of the 16-byte
//    granules.  K fragments are read with ds_read_b128; V fragments are read
//    transposed with ds_read_b64_tr_b16, which hands each lane 4 keys of one
//    feature column.  Tiles are double-buffered: the loads of tile j+1 are in
//    flight while tile j is multiplied.  Keys past the window end are loaded
//    from the last valid row (finite values) and masked to -inf.
//  * workgroup ids are remapped so that each of the 8 XCDs gets a contiguous
//    range of tiles; neighbouring tiles share their window keys in that XCD's
//    L2.
#include "rha_device.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace {

constexpr int NW = 4;
constexpr int THREADS = NW * kWave;
constexpr int BM = NW * 32;       // query rows per workgroup
constexpr int BN = 64;            // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr float kLn2 = 0.6931471805599453f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

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

template <int D>
struct FwdCfg {
  static constexpr int DS = D / 16;               // MFMA k-steps over features
  static constexpr int DB = D / 32;               // 32-wide feature blocks
  static constexpr int GR = D / 8;                // 16-byte granules per row
  static constexpr int TILE = BN * D * 2;         // bytes of one K or V tile
  static constexpr int LPW = BN * GR / (NW * 64); // direct loads per wave per tile
  static_assert(LPW * NW * 64 == BN * GR, "tile must split into whole wave loads");
  static_assert(TILE >= D * D, "half of the state staging must fit one V buffer");
  static_assert(TILE >= 2 * 32 * D * 2, "two waves' output rows must fit one K buffer");
};

// Granule swizzles (16-byte granule g of row r is stored at slot g ^ sw(r)).
// K: ds_read_b128 of 16 consecutive rows at one granule hits 16 distinct slots.
template <int D> __device__ __forceinline__ int ksw(int r) { return r & (D / 8 - 1); }
// V: a transpose read covers 4 consecutive rows x 4 granules (D = 128) or
// 4 rows x 4 granules of a 128-byte row (D = 64); the swizzle puts them in
// distinct bank ranges.
template <int D> __device__ __forceinline__ int vsw(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// s_waitcnt immediates (gfx9 encoding): wait for all vector-memory loads,
// or for all LDS operations, leaving the other counters alone.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

template <int D>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const FwdParams p) {
  using Cfg = FwdCfg<D>;
  constexpr int DS = Cfg::DS, DB = Cfg::DB, GR = Cfg::GR;
  __shared__ __attribute__((aligned(1024))) unsigned char kb0[Cfg::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char kb1[Cfg::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[Cfg::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[Cfg::TILE];

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

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[row l32][16s + 8hh .. +7].
  // Rows past the chunk re-read the last valid row; their results are not stored.
  bf16x8 qf[DS];
  {
    const int row = min(wave * 32 + l32, nrows - 1);
    const bf16_t* qr = qbase + (int64_t)row * p.q_st + hh * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld16(qr + s * 16));
  }

  f32x16 o[DB];
#pragma unroll
  for (int nb = 0; nb < DB; ++nb) o[nb] = f32x16{};
  float lsum = 0.f, mrun;

  // ---- linear term: O^T = S^T phi(Q)^T, l = phi(Q).z, at reference max 0
  if (has_state) {
    // Stage S (float32 [D][D]) as bf16 A fragments: element (e = 8*eg + i, n)
    // at byte eg*D*16 + n*16 + 2i; groups eg < DS in vb0, the rest in vb1.
    constexpr int SUNITS = (D / 8) * (D / 4);  // 8 rows x 4 columns each
    for (int u = tid; u < SUNITS; u += THREADS) {
      const int eg = u / (D / 4), ng = u % (D / 4);
      f32x4 rows[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rows[i] = *reinterpret_cast<const f32x4*>(Sp + (int64_t)(eg * 8 + i) * D + ng * 4);
      unsigned char* dst = eg < DS ? vb0 + (size_t)eg * D * 16 : vb1 + (size_t)(eg - DS) * D * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack_bf16(rows[2 * i][j], rows[2 * i + 1][j]);
        *reinterpret_cast<u32x4*>(dst + (size_t)(ng * 4 + j) * 16) = pk;
      }
    }
    __syncthreads();
    float lz = 0.f;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 pf = phi8(qf[s]);
      const u32x4 qw = __builtin_bit_cast(u32x4, qf[s]);
      const f32x4 z0 = *reinterpret_cast<const f32x4*>(zp + s * 16 + hh * 8);
      const f32x4 z1 = *reinterpret_cast<const f32x4*>(zp + s * 16 + hh * 8 + 4);
      lz += phi(bf16_lo(qw[0])) * z0[0] + phi(bf16_hi(qw[0])) * z0[1] + phi(bf16_lo(qw[1])) * z0[2] +
            phi(bf16_hi(qw[1])) * z0[3] + phi(bf16_lo(qw[2])) * z1[0] + phi(bf16_hi(qw[2])) * z1[1] +
            phi(bf16_lo(qw[3])) * z1[2] + phi(bf16_hi(qw[3])) * z1[3];
      const int eg = s * 2 + hh;
      const unsigned char* src = eg < DS ? vb0 + (size_t)eg * D * 16 : vb1 + (size_t)(eg - DS) * D * 16;
#pragma unroll
      for (int nb = 0; nb < DB; ++nb) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + (nb * 32 + l32) * 16));
        o[nb] = mfma32(a, pf, o[nb]);
      }
    }
    lsum = lz;  // this lane's half of the features; the halves are summed at the end
    mrun = 0.f;
    __syncthreads();
  } else {
    mrun = -INFINITY;
  }

  // ---- window keys
  const int ntiles = (int)((kend - kbeg + BN - 1) / BN);

  // Direct loads: load i of wave `wave` writes physical granules
  // (wave*LPW + i)*64 + lane of the tile; granule slot ps of row r holds
  // logical granule ps ^ sw(r).
  int krow[Cfg::LPW], kgo[Cfg::LPW], vgo[Cfg::LPW];
#pragma unroll
  for (int i = 0; i < Cfg::LPW; ++i) {
    const int pg = (wave * Cfg::LPW + i) * 64 + lane;
    krow[i] = pg / GR;
    const int ps = pg % GR;
    kgo[i] = (ps ^ ksw<D>(krow[i])) * 8;
    vgo[i] = (ps ^ vsw<D>(krow[i])) * 8;
  }
  auto issue = [&](int j, unsigned char* kdst, unsigned char* vdst) {
    const int64_t k0 = kbeg + (int64_t)j * BN;
#pragma unroll
    for (int i = 0; i < Cfg::LPW; ++i) {
      const int64_t key = min(k0 + krow[i], kend - 1);
      const int64_t off = key * p.kv_st;
      const int dst = (wave * Cfg::LPW + i) * 1024;
      __builtin_amdgcn_global_load_lds((const void*)(kbase + off + kgo[i]), (lds_void*)(kdst + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vbase + off + vgo[i]), (lds_void*)(vdst + dst), 16, 0, 0);
    }
  };

  // K fragment (A of S^T): row kb*32 + l32, granule 2s + hh.
  const int kswz = ksw<D>(l32);  // same for rows l32 and 32 + l32
  // V fragment (A of O^T, transposed read): in each 16-lane group, source
  // lane 4e + r supplies row 16ks + 8t + 4hh + e, columns nb*32 + 16*(group&1) + 4r;
  // lane j of the group then holds column nb*32 + 16*(group&1) + j, rows e = 0..3.
  const int vj = lane & 15;
  const int ve = vj >> 2, vr = vj & 3;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * vr;  // + nb*32
  const int vrow0 = 4 * hh + ve;                      // + 16ks + 8t

  if (ntiles > 0) issue(0, kb0, vb0);

  for (int j = 0; j < ntiles; ++j) {
    unsigned char* kcur = (j & 1) ? kb1 : kb0;
    unsigned char* vcur = (j & 1) ? vb1 : vb0;
    // tile j has landed (own loads), and every wave's loads are visible after the barrier
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (j + 1 < ntiles) issue(j + 1, (j & 1) ? kb0 : kb1, (j & 1) ? vb0 : vb1);
    const int valid = (int)min((int64_t)BN, kend - (kbeg + (int64_t)j * BN));

    // S^T = K Q^T : sacc[kb] reg 4r+i <-> key kb*32 + 8r + 4hh + i, query l32
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const int slot = ((2 * s + hh) ^ kswz) * 16;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kcur + (kb2 * 32 + l32) * D * 2 + slot));
        sacc[kb2] = mfma32(a, qf[s], sacc[kb2]);
      }
    }

    // online softmax (log2 domain), probabilities packed to bf16 pairs
    if (valid < BN) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb2 * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= valid) sacc[kb2][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb2][i]);
    mx = half_max(mx) * p.scale_log2;
    const float mnew = fmaxf(mrun, mx);
    if (__any(mnew > mrun + kRescaleSlack)) {
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int nb = 0; nb < DB; ++nb) o[nb] *= alpha;
    }
    const float mneg = -mrun;
    uint32_t pk[2][8];
    float ps = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][2 * i], p.scale_log2, mneg));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][2 * i + 1], p.scale_log2, mneg));
        ps += p0 + p1;
        pk[kb2][i] = pack_bf16(p0, p1);
      }
    lsum += ps;

    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const int kb2 = ks >> 1, r0 = (ks & 1) * 2;
      const u32x4 w4 = {pk[kb2][r0 * 2], pk[kb2][r0 * 2 + 1], pk[kb2][r0 * 2 + 2], pk[kb2][r0 * 2 + 3]};
      const bf16x8 pf = __builtin_bit_cast(bf16x8, w4);
      const int r_a = 16 * ks + vrow0, r_b = r_a + 8;
#pragma unroll
      for (int nb = 0; nb < DB; ++nb) {
        const int col = nb * 32 + vcol;
        const int ga = col >> 3, cb = (col & 7) * 2;
        const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vcur + r_a * D * 2 + ((ga ^ vsw<D>(r_a)) * 16) + cb));
        const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vcur + r_b * D * 2 + ((ga ^ vsw<D>(r_b)) * 16) + cb));
        const u32x2 w0 = __builtin_bit_cast(u32x2, x0), w1 = __builtin_bit_cast(u32x2, x1);
        const u32x4 av = {w0[0], w0[1], w1[0], w1[1]};
        o[nb] = mfma32(__builtin_bit_cast(bf16x8, av), pf, o[nb]);
      }
    }
  }

  // ---- epilogue: normalise, stage bf16 rows in LDS (per wave), write coalesced
  __syncthreads();
  const float ltot = half_sum(lsum);
  const float inv = 1.0f / ltot;
  unsigned char* stage = ((wave < 2) ? kb0 : kb1) + (wave & 1) * 32 * D * 2;
#pragma unroll
  for (int nb = 0; nb < DB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = nb * 32 + 8 * r + 4 * hh;
      const int g = col >> 3;
      u32x2 pr = {pack_bf16(o[nb][4 * r] * inv, o[nb][4 * r + 1] * inv),
                  pack_bf16(o[nb][4 * r + 2] * inv, o[nb][4 * r + 3] * inv)};
      *reinterpret_cast<u32x2*>(stage + l32 * D * 2 + ((g ^ ksw<D>(l32)) * 16) + (col & 7) * 2) = pr;
    }
  const int myrow = wave * 32 + l32;
  if (p.lse != nullptr && hh == 0 && myrow < nrows) {
    const int64_t L = (int64_t)p.n_qchunks * p.C;
    p.lse[(int64_t)bh * L + qtok0 + myrow] = (mrun + __log2f(ltot)) * kLn2;
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's staging writes are complete
  __builtin_amdgcn_wave_barrier();
  bf16_t* obase = (bf16_t*)p.out + b * p.q_sb + h * p.q_sh + qtok0 * p.q_st;
  for (int idx = lane; idx < 32 * GR; idx += 64) {
    const int r = idx / GR, g = idx % GR;
    const int row = wave * 32 + r;
    if (row < nrows)
      st16(obase + (int64_t)row * p.q_st + g * 8,
           *reinterpret_cast<const u32x4*>(stage + r * D * 2 + ((g ^ ksw<D>(r)) * 16)));
  }
}

template <int D>
hipError_t launch(FwdParams& p, hipStream_t s) {
  p.tiles_per_chunk = (p.C + BM - 1) / BM;
  p.total_tiles = p.B * p.H * p.n_qchunks * p.tiles_per_chunk;
  if (p.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_bf16_kernel<D>), dim3(p.total_tiles), dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(FwdParams& p, int d, hipStream_t s) {
  if (d == 128) return launch<128>(p, s);
  return launch<64>(p, s);
}

}  // namespace rha
