// The per-chunk state contribution of "Transformers are RNNs" (one chunk's
// phi(K)^T V and sum of phi(k)) as a workgroup-level unit for bf16 inputs on
// gfx950: run by the state kernel, and by the extra workgroups of a split
// streaming forward pass (the fold of the chunk leaving the window, section
// 2.A of the Hybrid Forcing explainer, computed beside the attention).
//
// One workgroup per (head, chunk, 64-row slice of the feature axis e of U):
// 4 waves, each owning 32x32 output blocks of the slice.  Tokens stream
// through LDS in tiles of 64, stored as loaded (token-major rows, 16-byte
// granules XOR-swizzled); both operands are contracted over tokens, so both
// are read with the LDS transpose read ds_read_b64_tr_b16, which hands each
// lane 8 tokens of one feature column.  R tiles (four; six in the two-slice
// workgroups) are in flight from HBM while
// one is multiplied (the unit is bound by HBM, not by the products).  phi is evaluated
// in float32 and rounded to bf16 for the product; u is summed from the float32
// phi values in a fixed order.  With `accumulate` the result is added into
// the destination (the streaming fold), otherwise it is stored.  A "chunk" may
// also be a token range of a real chunk (the split streaming fold): tok_end
// cuts the last one short.
#pragma once

#include "rha_device.hpp"
#include "rha_fwd_common.hpp"
#include "rha_launch.hpp"

namespace rha {
namespace state {


constexpr int NW = 4;
constexpr int THREADS = NW * kWave;
constexpr int BT = 64;      // tokens per tile
constexpr int ESLICE = 64;  // rows e of U per workgroup

template <int D>
struct StateCfg {
  static constexpr int ES = D / ESLICE;                   // slices per chunk
  static constexpr int KBYTES = BT * ESLICE * 2;          // one phi(K) slice tile
  static constexpr int VBYTES = BT * D * 2;               // one V tile
  static constexpr int KG = BT * (ESLICE / 8) / THREADS;  // phi(K) granules per thread (every thread)
  static constexpr int KROWSTEP = THREADS / (ESLICE / 8);  // token rows between a thread's granules
  static constexpr int VUNITS = (BT / 4) * (D / 8);
  static constexpr int NBW = (ESLICE / 32) * (D / 32) / NW;  // output 32x32 blocks per wave
  static_assert(KG * THREADS == BT * (ESLICE / 8) && VUNITS <= THREADS, "even phi(K) split, one V unit per thread at most");
  static_assert(NBW >= 1 && (ESLICE / 32) * (D / 32) % NW == 0, "whole blocks per wave");
};

// Row-major tile of W features: granule g (8 features) of token row r sits at
// slot g ^ sw(r); the swizzle spreads the rows a transpose read covers over
// distinct banks (as for the attention kernels' V tiles).
template <int W> __device__ __forceinline__ int tsw(int r) { return fwd::vsw<W>(r); }

// One 16-byte granule: token row r, granule g.
template <int W>
__device__ __forceinline__ void store_granule(unsigned char* tile, int r, int g, const u32x4& x) {
  *reinterpret_cast<u32x4*>(tile + r * W * 2 + ((g ^ tsw<W>(r)) * 16)) = x;
}

// MFMA operand fragment over tokens 16ks .. 16ks+15 for feature columns
// cb*32 .. cb*32+31 of a W-wide tile: lane l gets column cb*32 + l%32 and 8
// tokens, in the same k-order for every operand read this way.
template <int W>
__device__ __forceinline__ bf16x8 read_frag_t(const unsigned char* tile, int ks, int cb, int lane) {
  const int hh = lane >> 5, vj = lane & 15;
  const int col = cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (vj & 3);
  const int ra = 16 * ks + 4 * hh + (vj >> 2), rb = ra + 8;
  const int ga = col >> 3, cbyte = (col & 7) * 2;
  const fwd::i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (fwd::lds_i16x4*)(tile + ra * W * 2 + ((ga ^ tsw<W>(ra)) * 16) + cbyte));
  const fwd::i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (fwd::lds_i16x4*)(tile + rb * W * 2 + ((ga ^ tsw<W>(rb)) * 16) + cbyte));
  const u32x2 w0 = __builtin_bit_cast(u32x2, x0), w1 = __builtin_bit_cast(u32x2, x1);
  return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
}

// One workgroup of SL * THREADS threads computes unit `logical` with the
// given LDS buffers.  SL = 1: the unit is (head, chunk, slice of e), slices of
// a chunk adjacent.  SL = StateCfg<D>::ES: the unit is (head, chunk) and the
// workgroup's thread group g (THREADS threads) takes slice g, every group
// doing exactly what a one-slice workgroup does (so the results are the same
// bits) except that V, the same for every slice, is loaded and staged once,
// by group 0.  Buffers: kt holds SL x 2 phi(K) slice tiles of
// StateCfg<D>::KBYTES (slice-major), vt0 / vt1 the two V tiles of
// StateCfg<D>::VBYTES, zred SL blocks of reduction rows
// [THREADS / (ESLICE / 8)][ESLICE].
// SCALED: the per-token factors vscale / zweight are applied (a separate
// instantiation, so the plain one keeps its registers).
template <int D, bool SCALED, int SL = 1, int R = 4>
__device__ __forceinline__ void chunk_state_unit(const ChunkStateParams& p, int logical, unsigned char* kt,
                                                 unsigned char* vt0, unsigned char* vt1, float* zred_all) {
  using Cfg = StateCfg<D>;
  static_assert(SL == 1 || SL == Cfg::ES, "one slice or every slice per workgroup");
  const int tid = threadIdx.x % THREADS;  // thread within the slice's group
  const int grp = SL == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / THREADS);  // wave-uniform
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  unsigned char* const ktg = kt + (size_t)grp * 2 * Cfg::KBYTES;
  auto kt_s = [&](int buf) __attribute__((always_inline)) { return ktg + buf * Cfg::KBYTES; };
  auto vt_s = [&](int buf) __attribute__((always_inline)) { return buf ? vt1 : vt0; };
  float (*zred)[ESLICE] = reinterpret_cast<float (*)[ESLICE]>(zred_all + (size_t)grp * (THREADS / (ESLICE / 8)) * ESLICE);

  const int es = SL == 1 ? logical % Cfg::ES : grp;
  const int jc = (SL == 1 ? logical / Cfg::ES : logical) % p.n_chunks;
  const int bh = (SL == 1 ? logical / Cfg::ES : logical) / p.n_chunks;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t t0 = (int64_t)(p.chunk0 + jc) * p.C;
  const int len = (int)min((int64_t)p.C, p.tok_end - t0);  // tokens of this chunk
  const bf16_t* kbase = (const bf16_t*)p.k + b * p.kv_sb + h * p.kv_sh + t0 * p.kv_st + es * ESLICE;
  const bf16_t* vbase = (const bf16_t*)p.v + b * p.kv_sb + h * p.kv_sh + t0 * p.kv_st;

  // V rows per thread: 4 (one-slice workgroups, the first VUNITS threads);
  // 2 in a two-slice workgroup, where every thread of both groups takes part
  constexpr int VR = SL == 1 ? 4 : 2;
  const int vt = SL == 1 ? tid : (int)threadIdx.x;
  const bool vact = SL == 1 ? tid < Cfg::VUNITS : vt < (BT / VR) * (D / 8);
  const int kfo = tid % (ESLICE / 8), krow0 = tid / (ESLICE / 8);  // phi(K): every thread, KG rows
  const int vfo = vt % (D / 8), vtq = vt / (D / 8);

  const int eb = wave / (NW * Cfg::NBW / (D / 32));
  const int nb0 = (wave * Cfg::NBW) % (D / 32);

  f32x16 acc[Cfg::NBW];
#pragma unroll
  for (int i = 0; i < Cfg::NBW; ++i) acc[i] = f32x16{};
  float zacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zacc[i] = 0.f;

  const int ntiles = (len + BT - 1) / BT;
  static_assert(R % 2 == 0, "R tiles in flight from HBM (register ring); LDS buffer = slot parity");
  u32x4 kw[R][Cfg::KG], vw[R][VR];

  // Buffer loads whose descriptors end at the chunk's last token: rows past
  // it (and the lanes without a unit) read zeros, so loads and stores need no
  // branches and the load waits stay exact.
  const int chunk_bytes = len * (int)p.kv_st * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, chunk_bytes, fwd::kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, chunk_bytes, fwd::kBufWord3);
  const int kofs0 = (krow0 * (int)p.kv_st + kfo * 8) * 2;
  const int vofs0 = vact ? (vtq * VR * (int)p.kv_st + vfo * 8) * 2 : chunk_bytes;
  const int row_bytes = (int)p.kv_st * 2;
  auto gload = [&](int j, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
    const int tile_off = j * BT * row_bytes;
#pragma unroll
    for (int r = 0; r < Cfg::KG; ++r)
      kw[sl][r] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, kofs0 + tile_off + r * Cfg::KROWSTEP * row_bytes, 0, 0));
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int vo = vact ? vofs0 + tile_off + r * row_bytes : chunk_bytes;
      vw[sl][r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vo, 0, 0));
    }
  };
  const int64_t sbase = (int64_t)bh * p.scale_bh + t0;  // per-token factors of this chunk
  auto lstore = [&](int j, int buf, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int r = 0; r < Cfg::KG; ++r) {
      const int row = krow0 + r * Cfg::KROWSTEP;
      const bool ok = j * BT + row < len;  // rows past the chunk: phi(0) would be 1
      float zw = 1.f;
      if constexpr (SCALED) zw = ok ? p.zweight[sbase + j * BT + row] : 0.f;
      u32x4 fw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = ok ? phi(bf16_lo(kw[sl][r][i])) : 0.f;
        const float c = ok ? phi(bf16_hi(kw[sl][r][i])) : 0.f;
        if constexpr (SCALED) {
          zacc[2 * i] += a * zw;
          zacc[2 * i + 1] += c * zw;
        } else {
          zacc[2 * i] += a;
          zacc[2 * i + 1] += c;
        }
        fw[i] = pack_bf16(a, c);
      }
      store_granule<ESLICE>(kt_s(buf), row, kfo, fw);
    }
    if (vact) {
#pragma unroll
      for (int r = 0; r < VR; ++r) {
        u32x4 x = vw[sl][r];
        if constexpr (SCALED) {
          const int tok = j * BT + vtq * VR + r;
          const float sc = tok < len ? p.vscale[sbase + tok] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = pack_bf16(bf16_lo(x[i]) * sc, bf16_hi(x[i]) * sc);
        }
        store_granule<D>(vt_s(buf), vtq * VR + r, vfo, x);
      }
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BT / 16; ++ks) {
      const bf16x8 a = read_frag_t<ESLICE>(kt_s(buf), ks, eb, lane);
#pragma unroll
      for (int i = 0; i < Cfg::NBW; ++i) acc[i] = mfma32(a, read_frag_t<D>(vt_s(buf), ks, nb0 + i, lane), acc[i]);
    }
  };
  using S0 = std::integral_constant<int, 0>;

  // tile j lives in register slot j % R and LDS buffer j % 2 (tiles past the
  // chunk load as zeros and store harmlessly: phi is masked by token index,
  // and the buffer they land in is not read again)
  static_for<0, R>([&](auto s_c) __attribute__((always_inline)) { gload(decltype(s_c)::value, s_c); });
  lstore(0, 0, S0{});
  __syncthreads();
  auto iter = [&](int j, auto slot_c) {  // slot_c = j % R
    constexpr int sl = decltype(slot_c)::value;
    using Next = std::integral_constant<int, (sl + 1) % R>;
    gload(j + R, slot_c);  // slot of tile j, already in LDS
    mma(sl & 1);
    lstore(j + 1, (sl + 1) & 1, Next{});
    __syncthreads();
  };
  int j = 0;
  for (; j + R - 1 < ntiles; j += R)
    static_for<0, R>([&](auto s_c) __attribute__((always_inline)) { iter(j + decltype(s_c)::value, s_c); });
  static_for<0, R - 1>([&](auto s_c) __attribute__((always_inline)) {
    if (j + decltype(s_c)::value < ntiles) iter(j + decltype(s_c)::value, s_c);
  });

  // U: acc[i] reg 4r+q <-> e = es*64 + eb*32 + 8r + 4hh + q, n = (nb0+i)*32 + l32
  const int slot1 = jc + p.slot_offset, slot2 = jc + p.slot_offset2;
  const bool put1 = p.n_slots <= 0 || (slot1 >= 0 && slot1 < p.n_slots);
  const bool put2 = p.S2 != nullptr && slot2 >= 0 && slot2 < p.n_slots;
  auto store_u = [&](float* Sbase, int slot) {
    float* Sdst = Sbase + (int64_t)bh * p.s_bh + (int64_t)slot * D * D;
#pragma unroll
    for (int i = 0; i < Cfg::NBW; ++i) {
      const int n = (nb0 + i) * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = es * ESLICE + eb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        float* dst = Sdst + (int64_t)e * D + n;
        const float val = acc[i][r];
        *dst = p.accumulate ? *dst + val : val;
      }
    }
  };
  if (put1) store_u(p.S, slot1);
  if (put2) store_u(p.S2, slot2);

  // u: fixed-order reduction of the per-thread partial sums
#pragma unroll
  for (int i = 0; i < 8; ++i) zred[krow0][kfo * 8 + i] = zacc[i];
  __syncthreads();
  if (tid < ESLICE) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < THREADS / (ESLICE / 8); ++r) s += zred[r][tid];
    if (put1) {
      float* zd = p.z + (int64_t)bh * p.z_bh + (int64_t)slot1 * D + es * ESLICE + tid;
      *zd = p.accumulate ? *zd + s : s;
    }
    if (put2) {
      float* zd = p.z2 + (int64_t)bh * p.z_bh + (int64_t)slot2 * D + es * ESLICE + tid;
      *zd = p.accumulate ? *zd + s : s;
    }
  }
}

}  // namespace state
}  // namespace rha
