// Backward pass of the causal hybrid attention (head_dim 128, bf16) on gfx950.
//
// The forward output is out_i = N_i / D_i with N_i = sum_W e^{s_ij} v_j +
// phi(q_i)^T S_c and D_i = sum_W e^{s_ij} + phi(q_i).z_c (the shared
// normaliser of the hybrid: ReHyAt, abstract; Hybrid Forcing explainer,
// section 2.A; phi and the state from "Transformers are RNNs").  With
// lse_i = ln D_i, P_ij = e^{s_ij - lse_i}, delta_i = dout_i . out_i:
//   window:  dv_j += sum_i P_ij dout_i
//            ds_ij = P_ij (dout_i . v_j - delta_i)
//            dq_i += sum_j ds_ij k_j / sqrt(d),  dk_j += sum_i ds_ij q_i / sqrt(d)
//   linear:  dphi(q_i) = (S_c dout_i - z_c delta_i) / D_i
//            dS_c = sum_i phi(q_i) dout_i^T / D_i,  dz_c = -sum_i phi(q_i) delta_i / D_i
//            dU_j = sum_{c >= j + w} dS_c  (likewise du_j)
//            dv_t += dU_j^T phi(k_t),  dphi(k_t) = dU_j v_t + du_j
// and phi'(x) = 1 (x > 0), e^x (otherwise).
//
// Kernels (all products on the bf16 matrix cores, float32 accumulation):
//   bwd_prep_kernel      delta, 1/D and -delta/D per row
//   chunk state (rha_state_bf16.hip, scaled rows) for dS_c, dz_c, then a
//   running sum from the last slot for dU_j, du_j
//   bwd_dkdv_kernel      per 128 keys (32 per wave, rows of K and V held as
//                        operands): every 32-row query block of the chunks
//                        that see them -- S = Q K^T and dP = dO V^T with keys
//                        on the lanes, then dV^T += dO^T P and dK^T += Q^T dS;
//                        then the linear term of those keys (dU_j, du_j)
//   bwd_dq_kernel        per 128 query rows (32 per wave): every 32-key block
//                        of the window -- S^T = K Q^T and dP^T = V dO^T with
//                        queries on the lanes, then dQ^T += K^T dS^T; then the
//                        linear term of those queries (S_c, z_c)
// Each of dq, dk, dv is written once, window and linear term together.
// Operand layouts are those of the forward kernels: a row-major LDS tile
// (16-byte granules XOR-swizzled) is read by rows (ds_read_b128) or, for a
// transposed operand, by the transpose read ds_read_b64_tr_b16, which hands
// out the rows in the order the matrix-core output keeps them.
#include "rha_device.hpp"
#include "rha_frag.hpp"
#include "rha_fwd_common.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace {

using fwd::xcd_remap;
using namespace frag;

constexpr int NWB = 4;               // waves per workgroup
constexpr int TB = NWB * 64;         // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;

// ---- delta_i = dout_i . out_i, 1 / D_i = exp(-lse_i), -delta_i / D_i
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p) {
  const int64_t L = (int64_t)p.N * p.C;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.B * p.H * L) return;
  const int64_t bh = idx / L, t = idx - bh * L;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const int64_t off = b * p.sb + h * p.sh + t * p.st;
  const bf16_t* o = (const bf16_t*)p.out + off;
  const bf16_t* g = (const bf16_t*)p.dout + off;
  float acc = 0.f;
#pragma unroll 4
  for (int gr = 0; gr < BD / 8; ++gr) {
    const u32x4 a = ld16(o + gr * 8), c = ld16(g + gr * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(a[i]) * bf16_lo(c[i]) + bf16_hi(a[i]) * bf16_hi(c[i]);
  }
  const float r = __expf(-p.lse[idx]);
  p.delta[idx] = acc;
  p.rsc[idx] = r;
  p.zw[idx] = -acc * r;
}

// ---- the linear term: rows times a d x d state M (float32, row-major),
// staged in LDS as bf16 rows e = M[e][:] (mr) and, if TRANS, rows n = M[:][n]
// (mt); every thread of the workgroup takes part.
template <bool TRANS>
__device__ __forceinline__ void stage_state(unsigned char* mr, unsigned char* mt, const float* M, int tid) {
  for (int u = tid; u < BD * BD / 8; u += TB) {
    const int e = u / (BD / 8), g = u % (BD / 8);
    const f32x4 a = *reinterpret_cast<const f32x4*>(M + (int64_t)e * BD + g * 8);
    const f32x4 c4 = *reinterpret_cast<const f32x4*>(M + (int64_t)e * BD + g * 8 + 4);
    put_granule(mr, e, g, u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(c4[0], c4[1]), pack_bf16(c4[2], c4[3])});
    if constexpr (TRANS) {
      const float vals[8] = {a[0], a[1], a[2], a[3], c4[0], c4[1], c4[2], c4[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = g * 8 + i;  // row n of the transpose, column e
        *reinterpret_cast<uint16_t*>(mt + gran_off(n, e >> 3) + (e & 7) * 2) = (uint16_t)(pack_bf16(vals[i], 0.f) & 0xffffu);
      }
    }
  }
}

// phi'(x) of the four features f .. f+3 of a bf16 row
__device__ __forceinline__ void dphi4(const bf16_t* row, int f, float out[4]) {
  const u32x2 xw = *reinterpret_cast<const u32x2*>(row + f);
  const float xs[4] = {bf16_lo(xw[0]), bf16_hi(xw[0]), bf16_lo(xw[1]), bf16_hi(xw[1])};
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = xs[i] > 0.f ? 1.f : __expf(xs[i]);
}

// ---- window gradients of keys and values, then their linear term
//   (key chunks j <= N-1-w): dv_t += dU_j^T phi(k_t),  dk_t += (dU_j v_t + du_j) * phi'(k_t)
__global__ __launch_bounds__(TB) void bwd_dkdv_kernel(const BwdParams p) {
  // two buffers of (Q rows, dout rows, lse, delta) for one 32-row query block
  __shared__ __attribute__((aligned(1024))) unsigned char qs[2][ROWT];
  __shared__ __attribute__((aligned(1024))) unsigned char gs[2][ROWT];
  __shared__ float lse_s[2][RB], del_s[2][RB];
  // dU_j as bf16 rows, and its transpose
  __shared__ __attribute__((aligned(1024))) unsigned char um[BD * BD * 2];
  __shared__ __attribute__((aligned(1024))) unsigned char ut[BD * BD * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int ktiles = (p.C + 127) / 128;
  const int total = p.B * p.H * p.N * ktiles;
  const int logical = xcd_remap(blockIdx.x, total);
  const int tile = logical % ktiles, rest = logical / ktiles;
  const int j = rest % p.N, bh = rest / p.N;  // earlier key chunks (more query chunks see them) first
  const int b = bh / p.H, h = bh % p.H;
  const int64_t L = (int64_t)p.N * p.C;
  const int64_t head = b * p.sb + h * p.sh;
  const bf16_t* qb = (const bf16_t*)p.q + head;
  const bf16_t* kb = (const bf16_t*)p.k + head;
  const bf16_t* vb = (const bf16_t*)p.v + head;
  const bf16_t* gb = (const bf16_t*)p.dout + head;

  const int64_t key0 = (int64_t)j * p.C + 128 * tile + 32 * wave;  // this wave's first key
  const int nk = (int)max((int64_t)0, min((int64_t)32, (int64_t)(j + 1) * p.C - key0));
  bf16x8 kr[8], vr[8];  // rows of K and V for this lane's key
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (l32 < nk) {
      a = ld16(kb + (key0 + l32) * p.st + 16 * ks + 8 * hh);
      c = ld16(vb + (key0 + l32) * p.st + 16 * ks + 8 * hh);
    }
    kr[ks] = __builtin_bit_cast(bf16x8, a);
    vr[ks] = __builtin_bit_cast(bf16x8, c);
  }
  f32x16 dv[4], dk[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) dv[nb] = dk[nb] = f32x16{};

  // query blocks of the chunks whose window holds chunk j (j .. j + w - 1),
  // 32 rows each, numbered qi = (c - j) * nqb + block
  const int c_hi = p.w > 0 ? min(p.N - 1, j + p.w - 1) : j - 1;
  const int nqb = (p.C + RB - 1) / RB;
  const int nblk = (c_hi - j + 1) * nqb;
  // staging: thread tid moves granules u = tid + 256 i (i < 4) of the block's
  // 32 Q rows (u < 512) and 32 dout rows (u >= 512); threads < 32 the lse, delta
  u32x4 stg[4];
  float lse_r = 0.f, del_r = 0.f;
  auto fetch = [&](int qi) {
    const int c = j + qi / nqb, blk = qi % nqb;
    const int64_t row0 = (int64_t)c * p.C + RB * blk;
    const int nq = min(RB, p.C - RB * blk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + TB * i, which = u >> 9, rem = u & 511, r = rem >> 4, g = rem & 15;
      stg[i] = u32x4{0u, 0u, 0u, 0u};
      if (r < nq) stg[i] = ld16((which ? gb : qb) + (row0 + r) * p.st + g * 8);
    }
    if (tid < RB) {
      const bool ok = tid < nq;
      lse_r = ok ? p.lse[bh * L + row0 + tid] * kLog2e : INFINITY;  // rows past the chunk: P = 0
      del_r = ok ? p.delta[bh * L + row0 + tid] : 0.f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + TB * i, which = u >> 9, rem = u & 511, r = rem >> 4, g = rem & 15;
      put_granule(which ? gs[buf] : qs[buf], r, g, stg[i]);
    }
    if (tid < RB) {
      lse_s[buf][tid] = lse_r;
      del_s[buf][tid] = del_r;
    }
  };
  if (nblk > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int qi = 0; qi < nblk; ++qi) {
    const int buf = qi & 1;
    if (qi + 1 < nblk) fetch(qi + 1);  // in flight while this block is multiplied
    const unsigned char* qt = qs[buf];
    const unsigned char* gt = gs[buf];
    f32x16 sa = {}, pa = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sa = mfma32(row_frag(qt, 0, ks, lane), kr[ks], sa);  // S = Q K^T, keys on the lanes
      pa = mfma32(row_frag(gt, 0, ks, lane), vr[ks], pa);  // dP = dO V^T
    }
    uint32_t pp[8], dd[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const int m0 = out_row(i, hh), m1 = out_row(i + 1, hh);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sa[i], p.scale_log2, -lse_s[buf][m0]));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sa[i + 1], p.scale_log2, -lse_s[buf][m1]));
      pp[i >> 1] = pack_bf16(p0, p1);
      dd[i >> 1] = pack_bf16(p0 * (pa[i] - del_s[buf][m0]), p1 * (pa[i + 1] - del_s[buf][m1]));
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        dv[nb] = mfma32(col_frag(gt, ks, nb, lane), pack_b(pp, ks), dv[nb]);  // dV^T += dO^T P
        dk[nb] = mfma32(col_frag(qt, ks, nb, lane), pack_b(dd, ks), dk[nb]);  // dK^T += Q^T dS
      }
    // the other buffer was last read in the previous block, before the barrier that ended it
    if (qi + 1 < nblk) stash(buf ^ 1);
    __syncthreads();
  }
  // lane = key; element i of block nb = feature 32 nb + out_row(i)
  float* dvr = p.dv + (bh * L + key0 + l32) * BD;
  float* dkr = p.dk + (bh * L + key0 + l32) * BD;
  if (j < p.N - p.w) {  // the chunk is in the state of chunks j + w .. N-1
    stage_state<true>(um, ut, p.dS + ((int64_t)bh * p.N + j) * BD * BD, tid);
    __syncthreads();
    f32x16 o1[4], o2[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) o1[mb] = o2[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 pk = l32 < nk ? fwd::phi8(kr[ks]) : kr[ks];  // phi(k_t) (0 past the chunk)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        o1[mb] = mfma32(row_frag(ut, 32 * mb, ks, lane), pk, o1[mb]);      // dU^T phi(k)^T: m = n
        o2[mb] = mfma32(row_frag(um, 32 * mb, ks, lane), vr[ks], o2[mb]);  // dU v^T: m = e
      }
    }
    if (l32 < nk) {
      const bf16_t* kt = kb + (key0 + l32) * p.st;  // phi' argument
      const float* dz = p.dz + ((int64_t)bh * p.N + j) * BD;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int f = 32 * nb + 8 * rr + 4 * hh;
          const f32x4 zz = *reinterpret_cast<const f32x4*>(dz + f);
          float dphi[4];
          dphi4(kt, f, dphi);
          f32x4 a, k4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = dv[nb][4 * rr + i];
            k4[i] = dk[nb][4 * rr + i] * p.scale;
            a[i] += o1[nb][4 * rr + i];
            k4[i] += (o2[nb][4 * rr + i] + zz[i]) * dphi[i];
          }
          *reinterpret_cast<f32x4*>(dvr + f) = a;
          *reinterpret_cast<f32x4*>(dkr + f) = k4;
        }
    }
  } else if (l32 < nk) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int f = 32 * nb + 8 * rr + 4 * hh;
        *reinterpret_cast<f32x4*>(dvr + f) = f32x4{dv[nb][4 * rr], dv[nb][4 * rr + 1], dv[nb][4 * rr + 2], dv[nb][4 * rr + 3]};
        *reinterpret_cast<f32x4*>(dkr + f) = f32x4{dk[nb][4 * rr] * p.scale, dk[nb][4 * rr + 1] * p.scale,
                                                   dk[nb][4 * rr + 2] * p.scale, dk[nb][4 * rr + 3] * p.scale};
      }
  }
}

// ---- window gradient of the queries, then their linear term
//   (query chunks c >= w): dq_i += ((dout_i / D_i) S_c^T - z_c delta_i / D_i) * phi'(q_i)
__global__ __launch_bounds__(TB) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char ks_t[2][ROWT];
  __shared__ __attribute__((aligned(1024))) unsigned char vs_t[2][ROWT];
  __shared__ __attribute__((aligned(1024))) unsigned char sm[BD * BD * 2];  // S_c as bf16 rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int qtiles = (p.C + 127) / 128;
  const int total = p.B * p.H * p.N * qtiles;
  const int logical = xcd_remap(blockIdx.x, total);
  const int tile = logical % qtiles, rest = logical / qtiles;
  const int c = p.N - 1 - rest % p.N, bh = rest / p.N;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t L = (int64_t)p.N * p.C;
  const int64_t head = b * p.sb + h * p.sh;
  const bf16_t* qb = (const bf16_t*)p.q + head;
  const bf16_t* kb = (const bf16_t*)p.k + head;
  const bf16_t* vb = (const bf16_t*)p.v + head;
  const bf16_t* gb = (const bf16_t*)p.dout + head;

  const int64_t row0 = (int64_t)c * p.C + 128 * tile + 32 * wave;  // this wave's first query
  const int nq = (int)max((int64_t)0, min((int64_t)32, (int64_t)(c + 1) * p.C - row0));
  const bool qok = l32 < nq;
  bf16x8 qr[8], gr[8];  // this lane's rows of Q and dO
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
    if (qok) {
      a = ld16(qb + (row0 + l32) * p.st + 16 * ks + 8 * hh);
      g = ld16(gb + (row0 + l32) * p.st + 16 * ks + 8 * hh);
    }
    qr[ks] = __builtin_bit_cast(bf16x8, a);
    gr[ks] = __builtin_bit_cast(bf16x8, g);
  }
  const float lse2 = qok ? p.lse[bh * L + row0 + l32] * kLog2e : INFINITY;
  const float del = qok ? p.delta[bh * L + row0 + l32] : 0.f;
  f32x16 dq[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) dq[nb] = f32x16{};

  const int64_t kbeg = p.w > 0 ? (int64_t)max(0, c - p.w + 1) * p.C : 0;
  const int64_t kend = p.w > 0 ? (int64_t)(c + 1) * p.C : 0;
  const int nblk = (int)((kend - kbeg + RB - 1) / RB);
  // staging of 32-key blocks: thread tid moves granules u = tid + 256 i of
  // the block's 32 K rows (u < 512) and 32 V rows (u >= 512)
  u32x4 stg[4];
  auto fetch = [&](int bi) {
    const int64_t k0 = kbeg + (int64_t)RB * bi;
    const int nk = (int)min((int64_t)RB, kend - k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + TB * i, which = u >> 9, rem = u & 511, r = rem >> 4, g = rem & 15;
      stg[i] = u32x4{0u, 0u, 0u, 0u};
      if (r < nk) stg[i] = ld16((which ? vb : kb) + (k0 + r) * p.st + g * 8);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + TB * i, which = u >> 9, rem = u & 511, r = rem >> 4, g = rem & 15;
      put_granule(which ? vs_t[buf] : ks_t[buf], r, g, stg[i]);
    }
  };
  if (nblk > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int bi = 0; bi < nblk; ++bi) {
    const int buf = bi & 1;
    const int nk = (int)min((int64_t)RB, kend - (kbeg + (int64_t)RB * bi));
    if (bi + 1 < nblk) fetch(bi + 1);  // in flight while this block is multiplied
    const unsigned char* kt = ks_t[buf];
    const unsigned char* vt = vs_t[buf];
    f32x16 sa = {}, pa = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sa = mfma32(row_frag(kt, 0, ks, lane), qr[ks], sa);  // S^T = K Q^T, queries on the lanes
      pa = mfma32(row_frag(vt, 0, ks, lane), gr[ks], pa);  // dP^T = V dO^T
    }
    uint32_t dd[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const int m0 = out_row(i, hh), m1 = out_row(i + 1, hh);
      const float p0 = m0 < nk ? __builtin_amdgcn_exp2f(fmaf(sa[i], p.scale_log2, -lse2)) : 0.f;
      const float p1 = m1 < nk ? __builtin_amdgcn_exp2f(fmaf(sa[i + 1], p.scale_log2, -lse2)) : 0.f;
      dd[i >> 1] = pack_bf16(p0 * (pa[i] - del), p1 * (pa[i + 1] - del));
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) dq[nb] = mfma32(col_frag(kt, ks, nb, lane), pack_b(dd, ks), dq[nb]);  // dQ^T += K^T dS^T
    if (bi + 1 < nblk) stash(buf ^ 1);
    __syncthreads();
  }
  float* dqr = p.dq + (bh * L + row0 + l32) * BD;
  if (c >= p.w) {  // the chunk has a state (every chunk for w = 0)
    stage_state<false>(sm, nullptr, p.S + ((int64_t)bh * p.N + c) * BD * BD, tid);
    __syncthreads();
    const float rs = qok ? p.rsc[bh * L + row0 + l32] : 0.f;  // 1 / D_i
    const bf16_t* qt = qb + (row0 + l32) * p.st;                // phi' argument
    const float* zc = p.z + ((int64_t)bh * p.N + c) * BD;
    const float dD = qok ? p.zw[bh * L + row0 + l32] : 0.f;     // -delta_i / D_i
    // one 32-feature block at a time (16 more accumulators, not 64: the
    // kernel keeps two waves per SIMD)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x16 o1 = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4 x = __builtin_bit_cast(u32x4, gr[ks]);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = pack_bf16(bf16_lo(x[i]) * rs, bf16_hi(x[i]) * rs);  // dout_i / D_i
        o1 = mfma32(row_frag(sm, 32 * nb, ks, lane), __builtin_bit_cast(bf16x8, x), o1);
      }
      if (qok) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int f = 32 * nb + 8 * rr + 4 * hh;
          const f32x4 zz = *reinterpret_cast<const f32x4*>(zc + f);
          float dphi[4];
          dphi4(qt, f, dphi);
          f32x4 a;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = dq[nb][4 * rr + i] * p.scale;
            a[i] += (o1[4 * rr + i] + zz[i] * dD) * dphi[i];
          }
          *reinterpret_cast<f32x4*>(dqr + f) = a;
        }
      }
    }
  } else if (qok) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int f = 32 * nb + 8 * rr + 4 * hh;
        *reinterpret_cast<f32x4*>(dqr + f) = f32x4{dq[nb][4 * rr] * p.scale, dq[nb][4 * rr + 1] * p.scale,
                                                   dq[nb][4 * rr + 2] * p.scale, dq[nb][4 * rr + 3] * p.scale};
      }
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s) {
  const int64_t BH = (int64_t)p.B * p.H;
  const int64_t L = (int64_t)p.N * p.C;
  if (BH == 0 || L == 0) return hipSuccess;
  const int tiles128 = (p.C + 127) / 128;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((BH * L + 255) / 256)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.w < p.N) {  // some chunk has a state: the linear term
    // dS_c, dz_c of chunks c >= w into slot c - w, then slot j <- sum over slots j .. N-1-w = dU_j
    ChunkStateParams c{};
    c.k = p.q;
    c.v = p.dout;
    c.S = p.dS;
    c.z = p.dz;
    c.kv_sb = p.sb;
    c.kv_sh = p.sh;
    c.kv_st = p.st;
    c.s_bh = (int64_t)p.N * BD * BD;
    c.z_bh = (int64_t)p.N * BD;
    c.B = p.B;
    c.H = p.H;
    c.C = p.C;
    c.chunk0 = 0;
    c.n_chunks = p.N;
    c.slot_offset = -p.w;
    c.n_slots = p.N;
    c.accumulate = 0;
    c.tok_end = L;
    c.vscale = p.rsc;
    c.zweight = p.zw;
    c.scale_bh = L;
    e = launch_chunk_state_bf16(c, BD, s);
    if (e != hipSuccess) return e;
    PrefixParams pr{p.dS, p.dz, (int)BH, p.N, p.w, BD, 1};
    e = launch_prefix(pr, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(BH * p.N * tiles128)), dim3(TB), 0, s, p);
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)(BH * p.N * tiles128)), dim3(TB), 0, s, p);
  return hipGetLastError();
}

}  // namespace rha
