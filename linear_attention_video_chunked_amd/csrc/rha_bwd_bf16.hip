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
//   bwd_dkdv_pp_kernel   per 128 keys, two waves per SIMD for each 32 of them:
//                        a score wave (rows of K and V held as operands)
//                        computes, per 32-row query block of the chunks that
//                        see them, S = Q K^T and dP = dO V^T with keys on the
//                        lanes, then P and dS; a gradient wave accumulates
//                        dV^T += dO^T P and dK^T += Q^T dS, then adds the
//                        linear term of those keys (dU_j, du_j)
//   bwd_dq_kernel        per 128 query rows (32 per wave): every 32-key block
//                        of the window -- S^T = K Q^T and dP^T = V dO^T with
//                        queries on the lanes, then dQ^T += K^T dS^T; then the
//                        linear term of those queries (S_c, z_c)
// Each of dq, dk, dv is written once, window and linear term together.
// The bidirectional hybrid uses the same kernels with a symmetric window and
// the past and future states (and their gradients) summed in float32.
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

// 32x32x16 bf16 products whose accumulator lives in vector registers (the
// first of a chain starts from zero)
__device__ __forceinline__ void mfma_v_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// ---- delta_i = dout_i . out_i, 1 / D_i = exp(-lse_i), -delta_i / D_i, lse_i log2(e)
// 16 lanes per row (one 16-byte granule of out and of dout each), so that a
// wave's loads cover four whole rows; the partial dot products meet by lane
// swaps within each group of 16.
constexpr int kPrepRowsPerBlock = 16;
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p) {
  const int64_t L = (int64_t)p.N * p.C;
  const int gl = threadIdx.x & 15;
  const int64_t idx = (int64_t)blockIdx.x * kPrepRowsPerBlock + (threadIdx.x >> 4);
  const bool ok = idx < (int64_t)p.B * p.H * L;
  float acc = 0.f;
  if (ok) {
    const int64_t bh = idx / L, t = idx - bh * L;
    const int b = (int)(bh / p.H), h = (int)(bh % p.H);
    const int64_t off = b * p.sb + h * p.sh + t * p.st + gl * 8;
    const u32x4 a = ld16((const bf16_t*)p.out + off), c = ld16((const bf16_t*)p.dout + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(a[i]) * bf16_lo(c[i]) + bf16_hi(a[i]) * bf16_hi(c[i]);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (!ok || gl >= 4) return;
  // lanes 0..3 of the group write the row's four values
  const float lse = p.lse[idx];
  // (a row left with no weight by a pruned window has lse = -inf, out = 0)
  const float r = lse == -INFINITY ? 0.f : __expf(-lse);
  float* const dst = gl == 0 ? p.lse2 : gl == 1 ? p.delta : gl == 2 ? p.rsc : p.zw;
  dst[idx] = gl == 0 ? lse * kLog2e : gl == 1 ? acc : gl == 2 ? r : -acc * r;
}

// ---- the linear term: rows times a d x d state M (float32, row-major),
// staged in LDS as bf16 rows e = M[e][:] (mr) and, if TRANS, rows n = M[:][n]
// (mt); every thread of the workgroup takes part.
// With M2 set, the staged matrix is M + M2, summed in float32 (the
// bidirectional pass's past and future parts).
template <bool TRANS, int NT = TB>
__device__ __forceinline__ void stage_state(unsigned char* mr, unsigned char* mt, const float* M, const float* M2,
                                            int tid) {
  for (int u = tid; u < BD * BD / 8; u += NT) {
    const int e = u / (BD / 8), g = u % (BD / 8);
    f32x4 a = *reinterpret_cast<const f32x4*>(M + (int64_t)e * BD + g * 8);
    f32x4 c4 = *reinterpret_cast<const f32x4*>(M + (int64_t)e * BD + g * 8 + 4);
    if (M2 != nullptr) {
      a += *reinterpret_cast<const f32x4*>(M2 + (int64_t)e * BD + g * 8);
      c4 += *reinterpret_cast<const f32x4*>(M2 + (int64_t)e * BD + g * 8 + 4);
    }
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

// The same staging with S split into two bf16 parts, S = hi + lo (exact to
// about 2^-16 relative): hi rows into mr, lo rows 0..63 into lo0 and 64..127
// into lo1 (64 rows each).
__device__ __forceinline__ void stage_state_split(unsigned char* mr, unsigned char* lo0, unsigned char* lo1,
                                                  const float* M, const float* M2, int tid) {
  for (int u = tid; u < BD * BD / 8; u += TB) {
    const int e = u / (BD / 8), g = u % (BD / 8);
    f32x4 a = *reinterpret_cast<const f32x4*>(M + (int64_t)e * BD + g * 8);
    f32x4 c4 = *reinterpret_cast<const f32x4*>(M + (int64_t)e * BD + g * 8 + 4);
    if (M2 != nullptr) {
      a += *reinterpret_cast<const f32x4*>(M2 + (int64_t)e * BD + g * 8);
      c4 += *reinterpret_cast<const f32x4*>(M2 + (int64_t)e * BD + g * 8 + 4);
    }
    const float x[8] = {a[0], a[1], a[2], a[3], c4[0], c4[1], c4[2], c4[3]};
    u32x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
      lo[i] = pack_bf16(x[2 * i] - bf16_lo(hi[i]), x[2 * i + 1] - bf16_hi(hi[i]));
    }
    put_granule(mr, e, g, hi);
    put_granule(e < 64 ? lo0 : lo1, e & 63, g, lo);
  }
}

// phi'(x) of the four features f .. f+3 of a bf16 row
__device__ __forceinline__ void dphi4(const bf16_t* row, int f, float out[4]) {
  const u32x2 xw = *reinterpret_cast<const u32x2*>(row + f);
  const float xs[4] = {bf16_lo(xw[0]), bf16_hi(xw[0]), bf16_lo(xw[1]), bf16_hi(xw[1])};
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = xs[i] > 0.f ? 1.f : __expf(xs[i]);
}

// ---- dK, dV with two waves per SIMD (eight per workgroup, 128 keys).
// Waves 0-3 (score waves) each hold the K and V rows of 32 keys as operands
// and compute, per 32-row query block, S = Q K^T and dP = dO V^T (keys on the
// lanes), then P and dS = P (dP - delta); they hand P and dS, packed to bf16
// pairs in register order, to the gradient wave of the same keys (wave 4 +
// the same index) through LDS.  The gradient wave accumulates dV^T += dO^T P
// and dK^T += Q^T dS one block behind, then adds the keys' linear term.  On a
// SIMD the score wave's vector work (exponentials, dS) runs beside the
// gradient wave's products: each step has two barriers, the score waves'
// products before the second and their vector work after it, beside the
// gradient waves' products.
// Query blocks of the chunks whose window holds chunk j (j .. j + w - 1;
// bidirectional j - w + 1 .. j + w - 1; an anchor chunk: every chunk from j
// on), 32 rows each, reach LDS through buffer loads that write LDS directly,
// two blocks ahead (four buffers; each wave one 4-row slice of the Q and the
// dO tile, whose descriptors end at the chunk's last row: rows past it read as
// zero, and such rows (q = dout = 0, lse = delta = 0: P = 1, dP = 0) add
// nothing).  A pruned pass visits only the query blocks for which some key
// tile of the workgroup is kept (listed in LDS) and gives a pruned key P = 0
// lane by lane.  Anchor chunks' workgroups come first in every XCD's queue.
template <bool SPARSE>
__global__ __launch_bounds__(2 * TB) void bwd_dkdv_pp_kernel(const BwdParams p) {
  constexpr int NW = 2 * NWB;  // waves per workgroup
  // Q tiles 0..3 and dO tiles 4..7 of the ring; in the epilogue dU as bf16
  // rows (the first half) and its transpose (the second)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[8][ROWT];
  __shared__ __attribute__((aligned(256))) float lse_s[4][64];
  __shared__ __attribute__((aligned(256))) float del_s[4][64];
  // P and dS of a block from score wave k to gradient wave k: [buffer][k][P, dS][half][lane]
  __shared__ __attribute__((aligned(16))) u32x4 xch[2][NWB][2][2][64];
  __shared__ unsigned short qlist[SPARSE ? kMaxListedQBlocks : 1];
  __shared__ int qlist_n;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grad = wv >= NWB;  // gradient wave
  const int kw = wv & (NWB - 1);  // the wave's 32 keys within the workgroup's 128
  const int ktiles = (p.C + 127) / 128;
  const int total = p.B * p.H * p.N * ktiles;
  int tile, j, bh;
  if (p.anchors > 0 && p.anchors < p.N) {
    // anchor chunks' workgroups first in every XCD's queue (each XCD a
    // contiguous range of them, and of the others)
    const int bid = blockIdx.x, x = bid & 7;
    const int heavy = p.B * p.H * p.anchors * ktiles;
    if (bid < heavy) {
      const int hi = xcd_remap(bid, heavy);
      tile = hi % ktiles;
      const int rest = hi / ktiles;
      j = rest % p.anchors;
      bh = rest / p.anchors;
    } else {
      auto per_xcd = [](int n, int xx) { return n > xx ? (n - xx + 7) / 8 : 0; };
      int start = 0;
      for (int xx = 0; xx < x; ++xx) start += per_xcd(total, xx) - per_xcd(heavy, xx);
      const int li = start + (bid >> 3) - per_xcd(heavy, x);
      const int nl = p.N - p.anchors;
      tile = li % ktiles;
      const int rest = li / ktiles;
      j = p.anchors + rest % nl;
      bh = rest / nl;
    }
  } else {
    const int logical = xcd_remap(blockIdx.x, total);
    tile = logical % ktiles;
    const int rest = logical / ktiles;
    j = rest % p.N;
    bh = rest / p.N;
  }
  const int b = bh / p.H, h = bh % p.H;
  const int64_t L = (int64_t)p.N * p.C;
  const int64_t head = b * p.sb + h * p.sh;
  const bf16_t* qb = (const bf16_t*)p.q + head;
  const bf16_t* kb = (const bf16_t*)p.k + head;
  const bf16_t* vb = (const bf16_t*)p.v + head;
  const bf16_t* gb = (const bf16_t*)p.dout + head;

  const int64_t key0 = (int64_t)j * p.C + 128 * tile + 32 * kw;  // the wave's first key
  const int nk = (int)max((int64_t)0, min((int64_t)32, (int64_t)(j + 1) * p.C - key0));

  const int c_lo = p.bidir ? max(0, j - p.w + 1) : j;
  const int c_hi = j < p.anchors ? p.N - 1 : p.w > 0 ? min(p.N - 1, j + p.w - 1) : j - 1;
  const int nqb = (p.C + RB - 1) / RB;
  int nblk = max(0, c_hi - c_lo + 1) * nqb;
  bool listed = false;
  if constexpr (SPARSE) {
    if (nblk <= kMaxListedQBlocks) {
      listed = true;
      if (wv == 0) {
        const int64_t kw0 = (int64_t)j * p.C + 128 * tile;  // the workgroup's first key
        const int nkw = min(128, p.C - 128 * tile);
        int base = 0;
        for (int x0 = 0; x0 < nblk; x0 += 64) {
          const int x = x0 + lane;
          bool keep = false;
          if (x < nblk) {
            const int cq = c_lo + x / nqb, blk = x - (x / nqb) * nqb;
            const int64_t ws = (int64_t)max(0, cq - p.w + 1) * p.C;
            const int t0 = (int)((kw0 - ws) >> 6), t1 = min((int)((kw0 + nkw - 1 - ws) >> 6), p.nkt - 1);
            const unsigned char* mrow = p.kmask + (((int64_t)bh * p.N + cq) * p.mask_qtiles + (blk >> 3)) * p.nkt;
            for (int t = t0; t <= t1; ++t) keep = keep || mrow[t] != 0;
          }
          const uint64_t bal = __ballot(keep);
          if (keep) qlist[base + __popcll(bal & ((1ull << lane) - 1ull))] = (unsigned short)x;
          base += __popcll(bal);
        }
        if (lane == 0) qlist_n = base;
      }
      __syncthreads();
      nblk = __builtin_amdgcn_readfirstlane(qlist_n);
    }
  }
  auto qidx = [&](int i) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE)
      if (listed) return __builtin_amdgcn_readfirstlane(qlist[i]);
    return i;
  };
  // loads: each wave one 4-row load of the Q tile and one of the dO tile;
  // waves 0 and 1 the block's lse log2(e) and delta
  typedef __attribute__((address_space(3))) void lds_void;
  const int st2 = (int)p.st * 2;
  int doff;
  {
    const int row = 4 * wv + (lane >> 4);
    doff = row * st2 + (((lane & 15) ^ fsw(row)) * 16);
  }
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int bo = i & 3;
    const int qi = qidx(i);
    const int cq = c_lo + qi / nqb, blk = qi - (qi / nqb) * nqb;
    const int64_t row0 = (int64_t)cq * p.C + RB * blk;
    const int nq = min(RB, p.C - RB * blk);
    const int nbytes = (nq - 1) * st2 + BD * 2;
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(qb + row0 * p.st), (short)0, nbytes, fwd::kBufWord3);
    const __amdgpu_buffer_rsrc_t grs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(gb + row0 * p.st), (short)0, nbytes, fwd::kBufWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void*)(ring[bo] + wv * 1024), 16, doff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, (lds_void*)(ring[4 + bo] + wv * 1024), 16, doff, 0, 0, 0);
    if (wv < 2) {
      const float* src = (wv == 0 ? p.lse2 : p.delta) + bh * L + row0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nq * 4, fwd::kBufWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(wv == 0 ? lse_s[bo] : del_s[bo]), 4, lane * 4, 0, 0, 0);
    }
  };

  // every wave issues its slices of the first two blocks
  if (nblk > 0) {
    issue(0);
    if (nblk > 1) issue(1);
  }
  if (!grad) {
    // ---- score wave
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
    for (int s = 0; s <= nblk; ++s) {
      __builtin_amdgcn_s_waitcnt(fwd::wait_vm(0));
      __syncthreads();
      if (s + 2 < nblk) issue(s + 2);
      if (s >= nblk) {
        __syncthreads();  // the step's second barrier
        continue;
      }
      {
        const int x = s;
        uint32_t kc = 1;
        if constexpr (SPARSE) {
          const int qi = qidx(x);
          const int cq = c_lo + qi / nqb, blk = qi - (qi / nqb) * nqb;
          const int64_t ws = (int64_t)max(0, cq - p.w + 1) * p.C;
          const int kt = min((int)((key0 + l32 - ws) >> 6), p.nkt - 1);
          kc = p.kmask[(((int64_t)bh * p.N + cq) * p.mask_qtiles + (blk >> 3)) * p.nkt + kt] != 0;
        }
        const unsigned char* qt = ring[x & 3];
        const unsigned char* gt = ring[4 + (x & 3)];
        f32x4 lr[4], dr[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          lr[g] = *reinterpret_cast<const f32x4*>(lse_s[x & 3] + 8 * g + 4 * hh);
          dr[g] = *reinterpret_cast<const f32x4*>(del_s[x & 3] + 8 * g + 4 * hh);
        }
        bf16x8 qf[8], gf[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          qf[ks] = row_frag(qt, 0, ks, lane);
          gf[ks] = row_frag(gt, 0, ks, lane);
        }
        f32x16 sa, pa;
        mfma_v_first(sa, qf[0], kr[0]);
        mfma_v_first(pa, gf[0], vr[0]);
#pragma unroll
        for (int ks = 1; ks < 8; ++ks) {
          mfma_v(sa, qf[ks], kr[ks]);
          mfma_v(pa, gf[ks], vr[ks]);
        }
        // the products go first on the SIMD: the gradient wave starts its own
        // after this barrier, beside this wave's vector work
        __syncthreads();
        uint32_t pk[8], dk8[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int g = e >> 2, ee = e & 3;
          float p0 = __builtin_amdgcn_exp2f(fmaf(sa[e], p.scale_log2, -lr[g][ee]));
          float p1 = __builtin_amdgcn_exp2f(fmaf(sa[e + 1], p.scale_log2, -lr[g][ee + 1]));
          if constexpr (SPARSE) {
            p0 = kc ? p0 : 0.f;
            p1 = kc ? p1 : 0.f;
          }
          pk[e >> 1] = pack_bf16(p0, p1);
          dk8[e >> 1] = pack_bf16(p0 * (pa[e] - dr[g][ee]), p1 * (pa[e + 1] - dr[g][ee + 1]));
        }
        u32x4* xo = &xch[x & 1][kw][0][0][0];
        xo[lane] = u32x4{pk[0], pk[1], pk[2], pk[3]};
        xo[64 + lane] = u32x4{pk[4], pk[5], pk[6], pk[7]};
        xo[128 + lane] = u32x4{dk8[0], dk8[1], dk8[2], dk8[3]};
        xo[192 + lane] = u32x4{dk8[4], dk8[5], dk8[6], dk8[7]};
      }
    }
  } else {
    // ---- gradient wave
    f32x16 dv[4], dk[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) dv[nb] = dk[nb] = f32x16{};
    for (int s = 0; s <= nblk; ++s) {
      __builtin_amdgcn_s_waitcnt(fwd::wait_vm(0));
      __syncthreads();
      if (s + 2 < nblk) issue(s + 2);
      if (s < 1) {
        __syncthreads();  // the step's second barrier
        continue;
      }
      {
        const int x = s - 1;
        const unsigned char* qt = ring[x & 3];
        const unsigned char* gt = ring[4 + (x & 3)];
        const u32x4* xi = &xch[x & 1][kw][0][0][0];
        const u32x4 ph0 = xi[lane], ph1 = xi[64 + lane], dh0 = xi[128 + lane], dh1 = xi[192 + lane];
        bf16x8 gc[2][4], qc[2][4];  // the block's transposed fragments, read before the barrier
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            gc[ks][nb] = col_frag(gt, ks, nb, lane);
            qc[ks][nb] = col_frag(qt, ks, nb, lane);
          }
        __syncthreads();  // the score wave's products are done
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          dv[nb] = mfma32(gc[0][nb], __builtin_bit_cast(bf16x8, ph0), dv[nb]);
          dk[nb] = mfma32(qc[0][nb], __builtin_bit_cast(bf16x8, dh0), dk[nb]);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          dv[nb] = mfma32(gc[1][nb], __builtin_bit_cast(bf16x8, ph1), dv[nb]);
          dk[nb] = mfma32(qc[1][nb], __builtin_bit_cast(bf16x8, dh1), dk[nb]);
        }
      }
    }
    // the loads issued by this wave are complete (nothing after the last wait)
    // ---- epilogue below, after the staging shared with the score waves
    const bool lin = (j >= p.anchors && j < p.N - p.w) || (p.bidir && j >= max(p.w, 1));
    float* dvr = p.dv + (bh * L + key0 + l32) * BD;
    float* dkr = p.dk + (bh * L + key0 + l32) * BD;
    if (lin) {
      __syncthreads();  // every wave is done with the ring
      const int64_t slot = (int64_t)bh * p.N + j;
      unsigned char* um = ring[0];
      unsigned char* ut = ring[4];
      stage_state<true, 2 * TB>(um, ut, p.dS + slot * BD * BD, p.bidir ? p.dS2 + slot * BD * BD : nullptr, tid);
      __syncthreads();
      // this lane's key row (lanes past the chunk read its last row; their
      // columns of the products are not written)
      const int64_t krw = min(key0 + l32, (int64_t)(j + 1) * p.C - 1);
      const bf16_t* krow = kb + krw * p.st;
      const bf16_t* vrow = vb + krw * p.st;
      const float* dz = p.dz + ((int64_t)bh * p.N + j) * BD;
      const float* dz2 = p.bidir ? p.dz2 + ((int64_t)bh * p.N + j) * BD : nullptr;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x16 o1 = {}, o2 = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 kk = __builtin_bit_cast(bf16x8, ld16(krow + 16 * ks + 8 * hh));
          const bf16x8 vv = __builtin_bit_cast(bf16x8, ld16(vrow + 16 * ks + 8 * hh));
          o1 = mfma32(row_frag(ut, 32 * nb, ks, lane), fwd::phi8(kk), o1);  // dU^T phi(k)^T: m = n
          o2 = mfma32(row_frag(um, 32 * nb, ks, lane), vv, o2);             // dU v^T: m = e
        }
        if (l32 < nk) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int f = 32 * nb + 8 * rr + 4 * hh;
            f32x4 zz = *reinterpret_cast<const f32x4*>(dz + f);
            if (dz2 != nullptr) zz += *reinterpret_cast<const f32x4*>(dz2 + f);
            float dphi[4];
            dphi4(krow, f, dphi);
            f32x4 a, k4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              a[i] = dv[nb][4 * rr + i] + o1[4 * rr + i];
              k4[i] = dk[nb][4 * rr + i] * p.scale + (o2[4 * rr + i] + zz[i]) * dphi[i];
            }
            *reinterpret_cast<f32x4*>(dvr + f) = a;
            *reinterpret_cast<f32x4*>(dkr + f) = k4;
          }
        }
      }
    } else if (l32 < nk) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int f = 32 * nb + 8 * rr + 4 * hh;
          *reinterpret_cast<f32x4*>(dvr + f) =
              f32x4{dv[nb][4 * rr], dv[nb][4 * rr + 1], dv[nb][4 * rr + 2], dv[nb][4 * rr + 3]};
          *reinterpret_cast<f32x4*>(dkr + f) = f32x4{dk[nb][4 * rr] * p.scale, dk[nb][4 * rr + 1] * p.scale,
                                                     dk[nb][4 * rr + 2] * p.scale, dk[nb][4 * rr + 3] * p.scale};
        }
    }
    return;
  }
  // score waves: take part in the staging of dU, then leave
  const bool lin = (j >= p.anchors && j < p.N - p.w) || (p.bidir && j >= max(p.w, 1));
  if (lin) {
    __syncthreads();
    const int64_t slot = (int64_t)bh * p.N + j;
    stage_state<true, 2 * TB>(ring[0], ring[4], p.dS + slot * BD * BD, p.bidir ? p.dS2 + slot * BD * BD : nullptr, tid);
    __syncthreads();
  }
}

// ---- window gradient of the queries, then their linear term
//   (query chunks c >= w): dq_i += ((dout_i / D_i) S_c^T - z_c delta_i / D_i) * phi'(q_i)
template <bool SPARSE>
__global__ __launch_bounds__(TB) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(const BwdParams p) {
  // pruned pass: the kept 64-key tiles of the workgroup's query tile, in order
  __shared__ unsigned short kept_s[SPARSE ? kSparseMaxKeyTiles : 1];
  __shared__ int kept_n;
  // One 64 KiB arena: during the key loop three buffers of a 32-key block's
  // K and V rows (8 KiB each); in the epilogue S_c as bf16 rows (32 KiB) and
  // its low parts (two 16 KiB halves).
  __shared__ __attribute__((aligned(1024))) unsigned char arena[4 * BD * BD];
  auto ks_t = [&](int buf) __attribute__((always_inline)) { return arena + buf * (2 * ROWT); };
  auto vs_t = [&](int buf) __attribute__((always_inline)) { return arena + buf * (2 * ROWT) + ROWT; };
  unsigned char* const sm = arena;                         // S_c as bf16 rows
  unsigned char* const slo_k = arena + BD * BD * 2;        // low parts, rows 0..63
  unsigned char* const slo_v = arena + BD * BD * 2 + BD * BD;  // low parts, rows 64..127
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

  int64_t kbeg = p.w > 0 ? (int64_t)max(0, c - p.w + 1) * p.C : 0;
  int64_t kend = p.w > 0 ? (int64_t)(p.bidir ? min(p.N, c + p.w) : c + 1) * p.C : 0;
  // Anchored: the anchor keys not in the query's future, [0, a_end), come
  // first as a range of their own, or join the window when the two touch.
  int64_t a_end = p.anchors > 0 ? (int64_t)min(p.anchors, c + 1) * p.C : 0;
  if (a_end > 0 && (kend <= kbeg || kbeg <= a_end)) {  // one range [0, max(a_end, kend))
    kend = max(kend, a_end);
    kbeg = 0;
    a_end = 0;
  }
  const int nba = (int)((a_end + RB - 1) / RB);  // blocks of the separate anchor range
  int nblk = nba + (int)((kend - kbeg + RB - 1) / RB);
  if constexpr (SPARSE) {
    // the workgroup's 128 rows lie in one 256-row query tile: list its kept
    // key tiles (ballot + prefix count), then visit both 32-key halves of each
    const unsigned char* mrow = p.kmask + (((int64_t)bh * p.N + c) * p.mask_qtiles + (tile >> 1)) * p.nkt;
    const int T = (int)((kend - kbeg + 63) / 64);
    if (wave == 0) {
      int base = 0;
      for (int j0 = 0; j0 < T; j0 += 64) {
        const int jt = j0 + lane;
        const bool keep = jt < T && mrow[jt] != 0;
        const uint64_t bal = __ballot(keep);
        if (keep) kept_s[base + __popcll(bal & ((1ull << lane) - 1ull))] = (unsigned short)jt;
        base += __popcll(bal);
      }
      if (lane == 0) kept_n = base;
    }
    __syncthreads();
    nblk = 2 * __builtin_amdgcn_readfirstlane(kept_n);
  }
  // first key and key count of block bi (a pruned pass's second half of the
  // window's last tile may hold no key: count <= 0, the block is skipped)
  auto blk_k0 = [&](int bi) __attribute__((always_inline)) {
    if constexpr (SPARSE) return kbeg + 64 * (int64_t)__builtin_amdgcn_readfirstlane(kept_s[bi >> 1]) + RB * (bi & 1);
    return bi < nba ? (int64_t)RB * bi : kbeg + (int64_t)RB * (bi - nba);
  };
  auto blk_nk = [&](int bi) __attribute__((always_inline)) {
    return (int)min((int64_t)RB, (bi < nba ? a_end : kend) - blk_k0(bi));
  };
  // 32-key blocks of K and V reach LDS through buffer loads that write LDS
  // directly, two blocks ahead (three buffers); keys past the window read as
  // zero, and their probabilities are masked.
  typedef __attribute__((address_space(3))) void lds_void;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int st2 = (int)p.st * 2;  // bytes between rows
  int doff[2];                    // this lane's byte offset within a tile, loads 2wv and 2wv+1
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int row = 4 * (2 * wv + x) + (lane >> 4);
    doff[x] = row * st2 + (((lane & 15) ^ fsw(row)) * 16);
  }
  auto issue = [&](int bi, auto buf_c) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value;
    const int64_t k0 = blk_k0(bi);
    const int nk = blk_nk(bi);
    // (a block with no key still issues its loads, which read zeros: every
    // block counts the same loads in the waits below)
    const int nbytes = nk > 0 ? (nk - 1) * st2 + BD * 2 : 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kb + k0 * p.st), (short)0, nbytes, fwd::kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vb + k0 * p.st), (short)0, nbytes, fwd::kBufWord3);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(ks_t(BUF) + (2 * wv + x) * 1024), 16, doff[x], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vs_t(BUF) + (2 * wv + x) * 1024), 16, doff[x], 0, 0, 0);
    }
  };
  auto block = [&](int bi, auto buf_c) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value;
    // this wave's loads of block bi are in LDS (those of block bi+1, four,
    // may still be in flight)
    if (bi + 1 < nblk)
      __builtin_amdgcn_s_waitcnt(fwd::wait_vm(4));
    else
      __builtin_amdgcn_s_waitcnt(fwd::wait_vm(0));
    __syncthreads();  // every wave's; and every wave is done with block bi-1, whose buffer block bi+2 takes
    if (bi + 2 < nblk) issue(bi + 2, std::integral_constant<int, (BUF + 2) % 3>{});
    const int nk = blk_nk(bi);
    if constexpr (SPARSE)
      if (nk <= 0) return;  // the same for the whole workgroup: no barrier is skipped by some waves only
    const unsigned char* kt = ks_t(BUF);
    const unsigned char* vt = vs_t(BUF);
    f32x16 sa = {}, pa = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sa = mfma32(row_frag(kt, 0, ks, lane), qr[ks], sa);  // S^T = K Q^T, queries on the lanes
      pa = mfma32(row_frag(vt, 0, ks, lane), gr[ks], pa);  // dP^T = V dO^T
    }
    uint32_t dd[8];
    // keys past the end of their range (only in a range's last block) get P = 0
    auto softmax_grad = [&](auto masked_c) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int m0 = out_row(i, hh), m1 = out_row(i + 1, hh);
        float p0 = __builtin_amdgcn_exp2f(fmaf(sa[i], p.scale_log2, -lse2));
        float p1 = __builtin_amdgcn_exp2f(fmaf(sa[i + 1], p.scale_log2, -lse2));
        if constexpr (decltype(masked_c)::value) {
          p0 = m0 < nk ? p0 : 0.f;
          p1 = m1 < nk ? p1 : 0.f;
        }
        dd[i >> 1] = pack_bf16(p0 * (pa[i] - del), p1 * (pa[i + 1] - del));
      }
    };
    if (nk < RB)
      softmax_grad(std::true_type{});
    else
      softmax_grad(std::false_type{});
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) dq[nb] = mfma32(col_frag(kt, ks, nb, lane), pack_b(dd, ks), dq[nb]);  // dQ^T += K^T dS^T
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  if (nblk > 0) issue(0, B0{});
  if (nblk > 1) issue(1, B1{});
  int bi = 0;
  for (; bi + 2 < nblk; bi += 3) {  // three blocks per iteration, so each one's buffer is known
    block(bi, B0{});
    block(bi + 1, B1{});
    block(bi + 2, B2{});
  }
  if (bi < nblk) block(bi, B0{});
  if (bi + 1 < nblk) block(bi + 1, B1{});
  __syncthreads();  // the epilogue reuses the K/V buffers
  float* dqr = p.dq + (bh * L + row0 + l32) * BD;
  // the chunk has a state (every chunk for w = 0; bidirectional, also a
  // future one while chunk c + max(w, 1) exists)
  // (anchored: the history is chunks a .. c - w)
  if (c - p.w >= p.anchors || (p.bidir && c + max(p.w, 1) <= p.N - 1)) {
    // S_c and the rows dout_i / D_i each as two bf16 parts, the three
    // products that matter (hi hi, hi lo, lo hi) on the matrix cores: with
    // one bf16 rounding of each operand the sum over features, which cancels
    // strongly, loses about 5e-3 relative, the same size as the state chunks'
    // whole query gradient error budget; split, the term is exact to float32
    // level.  The low part of S goes into the K/V staging buffers, free now.
    const int64_t slot = (int64_t)bh * p.N + c;
    stage_state_split(sm, slo_k, slo_v, p.S + slot * BD * BD, p.bidir ? p.S2 + slot * BD * BD : nullptr, tid);
    __syncthreads();
    const float rs = qok ? p.rsc[bh * L + row0 + l32] : 0.f;  // 1 / D_i
    const bf16_t* qt = qb + (row0 + l32) * p.st;                // phi' argument
    const float* zc = p.z + ((int64_t)bh * p.N + c) * BD;
    const float* zc2 = p.bidir ? p.z2 + ((int64_t)bh * p.N + c) * BD : nullptr;
    const float dD = qok ? p.zw[bh * L + row0 + l32] : 0.f;     // -delta_i / D_i
    // one 32-feature block at a time (16 more accumulators, not 64: the
    // kernel keeps two waves per SIMD)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x16 o1 = {};
      const unsigned char* slo = nb < 2 ? slo_k : slo_v;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 g = __builtin_bit_cast(u32x4, gr[ks]);
        u32x4 xh, xl;  // dout_i / D_i = xh + xl
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = bf16_lo(g[i]) * rs, x1 = bf16_hi(g[i]) * rs;
          xh[i] = pack_bf16(x0, x1);
          xl[i] = pack_bf16(x0 - bf16_lo(xh[i]), x1 - bf16_hi(xh[i]));
        }
        const bf16x8 sh = row_frag(sm, 32 * nb, ks, lane), sl = row_frag(slo, 32 * (nb & 1), ks, lane);
        o1 = mfma32(sh, __builtin_bit_cast(bf16x8, xh), o1);
        o1 = mfma32(sh, __builtin_bit_cast(bf16x8, xl), o1);
        o1 = mfma32(sl, __builtin_bit_cast(bf16x8, xh), o1);
      }
      if (qok) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int f = 32 * nb + 8 * rr + 4 * hh;
          f32x4 zz = *reinterpret_cast<const f32x4*>(zc + f);
          if (zc2 != nullptr) zz += *reinterpret_cast<const f32x4*>(zc2 + f);
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
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((BH * L + kPrepRowsPerBlock - 1) / kPrepRowsPerBlock)),
                     dim3(256), 0, s, p);
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
    const int lag_f = max(p.w, 1);  // bidirectional: the future part starts at chunk c + max(w, 1)
    if (p.bidir) {  // and dS_c, dz_c of every chunk into future slot c + max(w, 1)
      c.S2 = p.dS2;
      c.z2 = p.dz2;
      c.slot_offset2 = lag_f;
    }
    e = launch_chunk_state_bf16(c, BD, s);
    if (e != hipSuccess) return e;
    PrefixParams pr{p.dS, p.dz, (int)BH, p.N, p.w, BD, 1};
    e = launch_prefix(pr, s);
    if (e != hipSuccess) return e;
    if (p.bidir) {  // future slot j <- sum over slots max(w, 1) .. j
      PrefixParams pf{p.dS2, p.dz2, (int)BH, p.N, lag_f, BD, 0};
      e = launch_prefix(pf, s);
      if (e != hipSuccess) return e;
    }
  }
  const dim3 grid((unsigned)(BH * p.N * tiles128));
  if (p.kmask != nullptr) {
    hipLaunchKernelGGL(bwd_dkdv_pp_kernel<true>, grid, dim3(2 * TB), 0, s, p);
    hipLaunchKernelGGL(bwd_dq_kernel<true>, grid, dim3(TB), 0, s, p);
  } else {
    hipLaunchKernelGGL(bwd_dkdv_pp_kernel<false>, grid, dim3(2 * TB), 0, s, p);
    hipLaunchKernelGGL(bwd_dq_kernel<false>, grid, dim3(TB), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace rha
