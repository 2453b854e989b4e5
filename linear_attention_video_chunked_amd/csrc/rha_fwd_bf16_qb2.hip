// Fused hybrid-attention forward, bf16, head dimension 128: 64 query rows
// per wave, one wave per SIMD.
//
// Computes ("Long-Horizon Streaming Video Generation via Hybrid Attention with
// Decoupled Distillation", explainer section 2.A: FlashAttention-style window
// blocks plus the folded linear state, one shared normaliser)
//   out_i = (sum_{j in window} exp(s_ij) v_j + phi(q_i)^T S_c)
//         / (sum_{j in window} exp(s_ij)     + phi(q_i)^T z_c)
//
// Design (gfx950):
// * Each wave owns two 32-row query blocks, so every K or V fragment read
//   from LDS feeds two 32x32x16 products.  Scores are computed transposed
//   (S^T = K Q^T, one query per lane) and the output as O^T = V^T P^T, so the
//   probabilities of a lane feed the product without any exchange.
// * Registers: O^T accumulators (128) in AGPRs, Q fragments, score
//   accumulators and probabilities in VGPRs; one wave per SIMD.
// * Software pipeline over 32-key blocks; step s computes QK^T of block s+1,
//   the softmax of block s and P V of block s-1.  Every step is hand-ordered:
//   8 rounds of 4 groups, each group one matrix product followed by a short
//   slice of independent VALU work, closed by a scheduling fence.
// * The softmax keeps a stale reference maximum: exponentials are taken
//   against the current reference without a per-block maximum, and the block
//   is accepted while its row sum stays below 2^64 (which bounds every term).
//   A block that fails (first block without linear state, or a score that
//   grew by 2^64) is redone against its true maximum; if the reference of a
//   query moved after something was accumulated, the whole tile is computed
//   again with the final references, which nothing exceeds by the bound.
// * K/V tiles of 64 keys are staged one period ahead through registers with
//   buffer loads (zero past the window end) into XOR-swizzled LDS; V is read
//   transposed with ds_read_b64_tr_b16; tiles are visited in an XCD-aware
//   order, longest windows first.
// * A short tail of a chunk (C mod 256 rows, at most 32) would leave three of
//   its tile's four waves without rows; its workgroup instead splits the
//   tail's key window four ways between its waves (tail_pass).
#include <type_traits>

#include "rha_device.hpp"
#include "rha_frag.hpp"
#include "rha_fwd_common.hpp"
#include "rha_state_unit.hpp"
#include "rha_launch.hpp"
#include "rha_small.hpp"

namespace rha {
namespace {

using namespace fwd;

// Empty asm that claims to modify x: the value is produced before this point
// and cannot be moved past it (keeps hand-ordered work in its slot).
template <typename T> __device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }
template <typename T> __device__ __forceinline__ void pin_acc(T& x) { asm volatile("" : "+a"(x)); }

// S^T += K Q^T block product in the VGPR-accumulator form of the
// instruction (the softmax VALU reads these accumulators; in AGPRs every read
// would cost a copy).  Written as asm because the compiler picks the AGPR
// form for every product of a kernel that keeps accumulators in AGPRs.  No
// vector-ALU instruction writes these operands shortly before: K fragments
// come from LDS reads (ordered by the LDS counter waits), Q fragments are
// loaded once, and the accumulators are written by products (or masked by
// the softmax) a whole pipeline step earlier; the results are first read by
// VALU code one step (32 further products) later, far past the result
// latency, and the accumulation chain has three other products between
// dependent ones.  So no wait states are inserted.
__device__ __forceinline__ void mfma_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

constexpr int Q2_QB = 2;  // 32-row query blocks per wave
// waves per workgroup: 4 (256 query rows); 2 (128 rows, less padding of
// 1560-row chunks) measured 5% slower on the Wan 1.3B shape
constexpr int Q2_NW = 4;
// Probabilities up to 2^kQ2Slack are accepted against a stale reference
// (far inside the bf16 and f32 ranges).
constexpr float kQ2Slack = 64.0f;
// Key tiles the state-seeded split of a split pass gives up to the others:
// seeding (the linear term, 64 products per wave plus the state loads)
// measured about 3 us, two 64-key tiles of the pipeline.
constexpr int kQ2SeedTiles = 2;

// LDS tile buffers (head dimension 128): K and V, double buffered.  At
// namespace scope so that the rare second pass, a separate function, shares
// them with the kernel.
constexpr int Q2_D = 128;
constexpr int Q2_TILE = BN * Q2_D * 2;
__shared__ __attribute__((aligned(1024))) unsigned char q2_kb0[Q2_TILE];
__shared__ __attribute__((aligned(1024))) unsigned char q2_kb1[Q2_TILE];
__shared__ __attribute__((aligned(1024))) unsigned char q2_vb0[Q2_TILE];
__shared__ __attribute__((aligned(1024))) unsigned char q2_vb1[Q2_TILE];
// key tiles a pass visits, in order, then one past the end: pruned passes
// list kept window tiles; anchored passes list first keys (q2_act) and key
// counts (q2_actv) of the anchor and window tiles
__shared__ int q2_act[kSparseMaxKeyTiles + 1];
__shared__ int q2_actv[kSparseMaxKeyTiles + 1];
__shared__ int q2_act_n;

// Launch order.  Workgroup b runs on XCD b % 8; each XCD takes a contiguous
// range of logical tiles (xcd_remap), so a chunk's tiles share an L2.  With
// short tails (unsplit passes), each XCD runs the full tiles of its range
// first and the tails (logical tiles t*tpc - 1, one per chunk) last: short
// jobs at the end of a queue fill the gaps the long ones leave (a model of
// the per-XCD dispatch: 6% off the Wan-1.3B makespan).
__device__ __forceinline__ int launch_order(int bid, int total, int tpc, bool tails_last) {
  if (!tails_last || tpc < 2) return xcd_remap(bid, total);
  const int per = total >> 3, rem = total & 7, x = bid & 7, local = bid >> 3;
  const int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  const int n = x < rem ? per + 1 : per;
  const int ntail = (base + n) / tpc - base / tpc;  // tails in [base, base + n)
  const int nfull = n - ntail;
  if (local < nfull) {  // the local-th full tile of the range
    const int g = base - base / tpc + local;
    return (g / (tpc - 1)) * tpc + g % (tpc - 1);
  }
  return (base / tpc + local - nfull) * tpc + tpc - 1;
}

// One pass over a tile, output included.  FIRST: references start at 0 (with
// linear state) or -inf and blocks are checked against the bound; returns
// nonzero where a reference moved after accumulation.  Otherwise references
// start at mio and no block is checked.  mio receives the final references.
// VIS: which key tiles a pass visits -- 0 the window's (dense), 1 the kept
// ones of a pruned window, 2 the anchor chunks' and the window's.
template <int D, int NW, bool FIRST, bool PARTIAL, int VIS>
__device__ __forceinline__ int tile_pass(const FwdParams& p, float (&mio)[Q2_QB]) {
  static_assert(D == Q2_D, "tile buffers are sized for head dimension 128");
  constexpr bool SPARSE = VIS == 1, ANCH = VIS == 2;
  static_assert(!(PARTIAL && ANCH), "anchored passes are not split");
  constexpr int THREADS = NW * 64, QB = Q2_QB, BM = NW * 32 * Q2_QB;
  constexpr int DS = D / 16, DB = D / 32, GR = D / 8;
  constexpr int TILE = BN * D * 2;
  constexpr int LPT = BN * GR / THREADS;
  static_assert(LPT * THREADS == BN * GR, "tile must split evenly over the threads");
  static_assert(TILE >= D * D, "half of the state staging must fit one V buffer");
  static_assert(TILE >= 32 * QB * D * 2, "one wave's output rows must fit one tile buffer");
  static_assert(NW == 2 || NW == 4, "the epilogue stages one wave per tile buffer; loads split evenly");

  static_assert(TILE == Q2_TILE, "tile buffer size");
  unsigned char* const kb0 = q2_kb0;
  unsigned char* const kb1 = q2_kb1;
  unsigned char* const vb0 = q2_vb0;
  unsigned char* const vb1 = q2_vb1;

  const int tid = threadIdx.x;
  // the wave index is the same in every lane: kept scalar, so the tile loads'
  // LDS addresses are formed without vector instructions
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- which tile
  const int logical0 = launch_order(blockIdx.x, p.total_tiles, p.tiles_per_chunk, !PARTIAL && p.tail_rows > 0);
  const int split = PARTIAL ? logical0 % p.n_splits : 0;  // splits of a tile adjacent (one XCD)
  const int logical = PARTIAL ? logical0 / p.n_splits : logical0;
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
  bool has_state, has_past = true, has_future = false;
  const float* Sp;
  const float* zp;
  const float* Sp2 = nullptr;  // future state (bidirectional)
  const float* zp2 = nullptr;
  if (!p.stream_mode) {
    if (p.w > 0) {
      kbeg = (int64_t)max(0, c - p.w + 1) * p.C;
      kend = (int64_t)(p.bidir ? min(p.n_qchunks, c + p.w) : c + 1) * p.C;
    } else {
      kbeg = kend = 0;
    }
    // history: chunks anchors .. c-w (w = 0: own chunk included)
    has_past = p.anchors > 0 ? (c - p.w >= p.anchors) : ((p.w == 0) || (c >= p.w));
    has_future = p.bidir && c + max(p.w, 1) <= p.n_qchunks - 1;
    has_state = has_past || has_future;
    Sp = p.S + ((int64_t)bh * p.n_qchunks + c) * D * D;
    zp = p.z + ((int64_t)bh * p.n_qchunks + c) * D;
    if (p.bidir) {
      Sp2 = p.S2 + ((int64_t)bh * p.n_qchunks + c) * D * D;
      zp2 = p.z2 + ((int64_t)bh * p.n_qchunks + c) * D;
    }
  } else {
    kbeg = 0;
    kend = p.n_keys;
    has_state = p.has_state != 0;
    if (PARTIAL) {  // this split's share of the key tiles; the first split takes the state
      // (and kQ2SeedTiles fewer key tiles: seeding the accumulators with the
      // linear term costs about that much, so the splits end together)
      const int tiles_all = (p.n_keys + BN - 1) / BN;
      const int n = p.n_splits;
      const int e0 = max(1, tiles_all / n - (has_state && tiles_all >= 4 * n ? kQ2SeedTiles : 0));
      const int t_lo = split == 0 ? 0 : e0 + (int)((int64_t)(split - 1) * (tiles_all - e0) / (n - 1));
      const int t_hi = split == 0 ? e0 : e0 + (int)((int64_t)split * (tiles_all - e0) / (n - 1));
      kbeg = (int64_t)t_lo * BN;
      kend = min((int64_t)t_hi * BN, (int64_t)p.n_keys);
      has_state = has_state && split == 0;
    }
    Sp = p.S + (int64_t)bh * D * D;
    zp = p.z + (int64_t)bh * D;
  }
  const int T = (int)((kend - kbeg + BN - 1) / BN);  // LDS tiles in the window

  // Pruned pass: the kept key tiles of this query tile, listed in order by
  // wave 0 (ballot + prefix count over the mask row), followed by T (one tile
  // past the window, which loads as zeros).  The pipeline then visits Tp tiles;
  // act(t) is the window tile that visit t loads.
  int Tp = T;
  if constexpr (SPARSE) {
    // (a split streaming pass lists the kept tiles of its own share: its
    // first tile is tile kbeg / BN of the step's window)
    const unsigned char* mrow = p.kmask + (((int64_t)bh * p.n_qchunks + c) * p.mask_qtiles + tile) * p.nkt +
                                (p.stream_mode ? kbeg / BN : 0);
    if (wave == 0) {
      int base = 0;
      for (int j0 = 0; j0 < T; j0 += 64) {
        const int j = j0 + lane;
        const bool keep = j < T && mrow[j] != 0;
        const uint64_t bal = __ballot(keep);
        if (keep) q2_act[base + __popcll(bal & ((1ull << lane) - 1ull))] = j;
        base += __popcll(bal);
      }
      if (lane == 0) {
        q2_act[base] = T;
        q2_act_n = base;
      }
    }
    __syncthreads();
    Tp = q2_act_n;
  }
  // Anchored pass: the anchor keys [0, a_end) (anchors not in the query's
  // future) and the window [kbeg, kend), merged when they touch, each cut
  // into 64-key tiles from its start; visit t loads the tile at key
  // q2_act[t] holding q2_actv[t] keys.
  if constexpr (ANCH) {
    const int64_t a_end = (int64_t)min(p.anchors, c + 1) * p.C;
    int64_t s0e = a_end, s1b = kbeg, s1e = kend;
    if (s1e <= s1b) s1b = s1e = 0;                                  // no window (w = 0)
    if (s1e > s1b && s1b <= s0e) {                                  // contiguous union
      s0e = max(s0e, s1e);
      s1b = s1e = 0;
    }
    const int TA = (int)((s0e + BN - 1) / BN), TW = (int)((s1e - s1b + BN - 1) / BN);
    Tp = TA + TW;
    kend = max(s0e, s1e);  // the descriptor covers every visited key
    for (int t = tid; t <= Tp; t += THREADS) {
      int64_t st;
      int64_t n;
      if (t < TA) {
        st = (int64_t)t * BN;
        n = s0e - st;
      } else if (t < Tp) {
        st = s1b + (int64_t)(t - TA) * BN;
        n = s1e - st;
      } else {
        st = kend;  // past the end: loads as zeros
        n = 0;
      }
      q2_act[t] = (int)st;
      q2_actv[t] = (int)min((int64_t)BN, n);
    }
    __syncthreads();
  }
  // The listed values are the same for every lane; reading them as wave-uniform
  // keeps the tile descriptors built from them in scalar registers (a
  // descriptor the compiler cannot prove uniform becomes a loop over lanes
  // around every tile load).
  auto act = [&](int t) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(q2_act[t]);
    else return t;
  };
  // first key of visit t
  auto act_key = [&](int t) __attribute__((always_inline)) -> int64_t {
    if constexpr (ANCH) return __builtin_amdgcn_readfirstlane(q2_act[t]);
    else return kbeg + (int64_t)act(t) * BN;
  };

  // ---- tile loads: direct HBM -> LDS (buffer loads with the LDS flag).  One
  // such load moves 64 lanes x 16 bytes into 1 KiB of consecutive LDS (lane L
  // at byte 16L): 4 rows of a tile.  Wave w issues loads i = 0..LPW-1 of a
  // tile, rows 4(LPW*w+i) .. +3; lane L fills row 4(LPW*w+i) + L/16, slot L%16,
  // with the global granule that the swizzle puts there (g = slot ^ sw(row)).
  // The descriptor of a tile starts at the tile's first key and ends at the
  // window end (its size is clamped at 0 for tiles past the window), so rows
  // past the end read as zero; the tile's offset lives in the descriptor's
  // base (scalar arithmetic), and each lane's offset within the tile is a
  // fixed register.
  constexpr int LPW = BN / 4 / NW;  // 4-row loads per wave and tile
  static_assert(LPW * 4 * NW == BN && LPW % 4 == 0 && GR == 16, "whole 4-row loads per wave");
  const int lrow = lane >> 4, lslot = lane & 15;
  int kdma[LPW], vdma[LPW];  // byte offsets within a tile of this lane's granule in load i
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = 4 * (LPW * wave + i) + lrow;
    kdma[i] = (row * (int)p.kv_st + (lslot ^ ksw<D>(row)) * 8) * 2;
    vdma[i] = (row * (int)p.kv_st + (lslot ^ vsw<D>(row)) * 8) * 2;
  }
  const int win_bytes = (int)(kend * p.kv_st * 2);
  typedef __attribute__((address_space(3))) void lds_void;
  // The descriptor's fields are read as wave-uniform: in the kernel they are
  // scalar already, and in the out-of-line second pass (whose parameter block
  // arrives in vector registers) this keeps each tile load a single load
  // instead of a loop over lanes.
  auto tile_rsrc = [&](const bf16_t* base, int64_t key) __attribute__((always_inline)) {
    const int tile_off = (int)(key * p.kv_st * 2);
    const uint64_t a = (uint64_t)((const unsigned char*)base + tile_off);
    const uint64_t ua = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc((void*)ua, (short)0,
                                             __builtin_amdgcn_readfirstlane(max(win_bytes - tile_off, 0)), kBufWord3);
  };
  auto dma_k = [&](unsigned char* dst, int64_t key, int i) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tile_rsrc(kbase, key), (lds_void*)(dst + (LPW * wave + i) * 1024), 16,
                                             kdma[i], 0, 0, 0);
  };
  auto dma_v = [&](unsigned char* dst, int64_t key, int i) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tile_rsrc(vbase, key), (lds_void*)(dst + (LPW * wave + i) * 1024), 16,
                                             vdma[i], 0, 0, 0);
  };

  // ---- The pass's first loads, all in flight together (one memory round
  // trip): the first K tile, the linear state and its normaliser (the state
  // of chunk c is always addressable, so the past state is loaded
  // unconditionally and dropped below when the chunk has no history), then Q.
  if (Tp > 0) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) dma_k(kb0, act_key(0), i);
  }
  constexpr int SUNITS = (D / 8) * (D / 4);
  constexpr int UPT = SUNITS / THREADS;  // 8-row x 4-column units of S per thread
  static_assert(UPT * THREADS == SUNITS && D / 4 <= THREADS, "state units split evenly over the threads");
  f32x4 srows[UPT][8];
  f32x4 zq = {0.f, 0.f, 0.f, 0.f};  // z[4 tid .. 4 tid + 3] (threads below D/4)
  if (has_state) {
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu) {
      const int u = tid + uu * THREADS, eg = u / (D / 4), ng = u % (D / 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) srows[uu][i] = *reinterpret_cast<const f32x4*>(Sp + (int64_t)(eg * 8 + i) * D + ng * 4);
    }
    if (tid < D / 4) zq = *reinterpret_cast<const f32x4*>(zp + tid * 4);
  }

  // ---- Q fragments of both query blocks (rows past the chunk re-read the last valid row)
  bf16x8 qf[QB][DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = min(wave * 32 * QB + qb * 32 + l32, nrows - 1);
    const bf16_t* qr = qbase + (int64_t)row * p.q_st + hh * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[qb][s] = __builtin_bit_cast(bf16x8, ld16(qr + s * 16));
  }
  // Mark the fragments as produced here (the load wait lands on this empty
  // statement), so the loop below is not made to wait for them again.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(qf[qb][s]));

  f32x16 o[QB][DB];
  float lsum[QB], mrun[QB];
  // Reference maximum (log2 units; an integer, or -inf before the first
  // block): 0 where the linear term seeds the accumulators.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mrun[qb] = FIRST ? (has_state ? 0.f : -INFINITY) : mio[qb];

  // ---- accumulators at the start of a pass: the linear term at the
  // reference, O^T = 2^-m S^T phi(Q)^T and l = 2^-m phi(Q).z (m is an integer,
  // so scaling phi(Q) by 2^-m before rounding it to bf16 is exact)
  auto init_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      lsum[qb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < DB; ++nb) o[qb][nb] = f32x16{};
    }
    if (!has_state) return;
    if (!has_past) {
#pragma unroll
      for (int uu = 0; uu < UPT; ++uu)
#pragma unroll
        for (int i = 0; i < 8; ++i) srows[uu][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      zq = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (has_future) {  // bidirectional: the past and future states summed in float32 before rounding
#pragma unroll
      for (int uu = 0; uu < UPT; ++uu) {
        const int u = tid + uu * THREADS, eg = u / (D / 4), ng = u % (D / 4);
        f32x4 r2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r2[i] = *reinterpret_cast<const f32x4*>(Sp2 + (int64_t)(eg * 8 + i) * D + ng * 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) srows[uu][i] += r2[i];
      }
      if (tid < D / 4) zq += *reinterpret_cast<const f32x4*>(zp2 + tid * 4);
    }
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu) {
      const int u = tid + uu * THREADS, eg = u / (D / 4), ng = u % (D / 4);
      unsigned char* dst = eg < DS ? vb0 + (size_t)eg * D * 16 : vb1 + (size_t)(eg - DS) * D * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16(srows[uu][2 * i][j], srows[uu][2 * i + 1][j]);
        *reinterpret_cast<u32x4*>(dst + (size_t)(ng * 4 + j) * 16) = w;
      }
    }
    // the normaliser in float32 in the second K buffer (free until the pipeline starts)
    if (tid < D / 4) *reinterpret_cast<f32x4*>(kb1 + tid * 16) = zq;
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float sc = ldexpf(1.0f, -(int)mrun[qb]);
      float lz = 0.f;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const u32x4 qw = __builtin_bit_cast(u32x4, qf[qb][s]);
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = phi(bf16_lo(qw[i]));
          f[2 * i + 1] = phi(bf16_hi(qw[i]));
        }
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(kb1 + (s * 16 + hh * 8) * 4);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(kb1 + (s * 16 + hh * 8 + 4) * 4);
        lz += f[0] * z0[0] + f[1] * z0[1] + f[2] * z0[2] + f[3] * z0[3] + f[4] * z1[0] + f[5] * z1[1] +
              f[6] * z1[2] + f[7] * z1[3];
        const u32x4 pw = {pack_bf16(f[0] * sc, f[1] * sc), pack_bf16(f[2] * sc, f[3] * sc),
                          pack_bf16(f[4] * sc, f[5] * sc), pack_bf16(f[6] * sc, f[7] * sc)};
        const int eg = s * 2 + hh;
        const unsigned char* src = eg < DS ? vb0 + (size_t)eg * D * 16 : vb1 + (size_t)(eg - DS) * D * 16;
#pragma unroll
        for (int nb = 0; nb < DB; ++nb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + (nb * 32 + l32) * 16));
          o[qb][nb] = mfma32(a, __builtin_bit_cast(bf16x8, pw), o[qb][nb]);
        }
      }
      lsum[qb] = lz * sc;  // this lane's half of the features; the halves are summed at the end
    }
    __syncthreads();
  };

  // ---- pipeline machinery
  const int kswz = ksw<D>(l32);
  // V fragment layout of the transposed read: in each 16-lane group, source
  // lane 4e + r supplies row 16ks + 8t + 4hh + e, columns nb*32 + 16*(group&1)
  // + 4r; lane j of the group then holds column nb*32 + 16*(group&1) + j.
  const int vj = lane & 15;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (vj & 3);
  const int vrow0 = 4 * hh + (vj >> 2);
  // keys of block blk inside the window (<= 0 for the second block of a last
  // tile that holds at most 32 keys)
  auto block_valid = [&](int blk) __attribute__((always_inline)) {
    if constexpr (ANCH) {
      return min(32, __builtin_amdgcn_readfirstlane(q2_actv[blk >> 1]) - 32 * (blk & 1));
    } else {
      const int real = 2 * act(blk >> 1) + (blk & 1);  // block of the window
      return (int)min((int64_t)32, kend - (kbeg + (int64_t)real * 32));
    }
  };
  // Tile buffers by tile index t + AHEAD.  PAR is the parity of t when known
  // at compile time (0 or 1; -1 if not); then every LDS address folds into a
  // constant offset from a per-lane register.
  auto kbuf = [&](auto par_c, int t, auto ahead_c) __attribute__((always_inline)) -> unsigned char* {
    constexpr int par = decltype(par_c)::value, ahead = decltype(ahead_c)::value;
    if constexpr (par < 0) return ((t + ahead) & 1) ? kb1 : kb0;
    else return ((par + ahead) & 1) ? kb1 : kb0;
  };
  auto vbuf = [&](auto par_c, int t, auto ahead_c) __attribute__((always_inline)) -> unsigned char* {
    constexpr int par = decltype(par_c)::value, ahead = decltype(ahead_c)::value;
    if constexpr (par < 0) return ((t + ahead) & 1) ? vb1 : vb0;
    else return ((par + ahead + 2) & 1) ? vb1 : vb0;
  };
  using A0 = std::integral_constant<int, 0>;
  using A1 = std::integral_constant<int, 1>;
  using Am1 = std::integral_constant<int, -1>;

  f32x16 sacc[2][QB];
  bf16x2 pk[2][QB][8];
  bf16x8 kf[3], vf[3];  // fragment ring
  // Per-lane LDS byte offsets of the fragments within a tile; everything else
  // (tile buffer, 32-key half, 16-key step, the second 8 rows of a V read) is
  // a constant added to them.  K fragment s: row l32, granule (2s + hh) ^
  // ksw(l32).  V fragment (ks, nb): rows 16ks + vrow0 (+8), column nb*32 +
  // vcol; the swizzle vsw(row) depends on vrow0 only.
  int kofs[DS], vofs[DB];
#pragma unroll
  for (int sidx = 0; sidx < DS; ++sidx) kofs[sidx] = l32 * D * 2 + ((2 * sidx + hh) ^ kswz) * 16;
#pragma unroll
  for (int nb = 0; nb < DB; ++nb) {
    const int col = nb * 32 + vcol;
    vofs[nb] = vrow0 * D * 2 + (((col >> 3) ^ vsw<D>(vrow0)) * 16) + (col & 7) * 2;
  }
  auto read_k = [&](const unsigned char* kt, int qh, int sidx) __attribute__((always_inline)) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kt + kofs[sidx] + 32 * qh * D * 2));
  };
  auto read_v = [&](const unsigned char* vt, int vh, int r) __attribute__((always_inline)) -> bf16x8 {
    const int ks = r >> 2, nb = r & 3;
    const unsigned char* pa = vt + vofs[nb] + (32 * vh + 16 * ks) * D * 2;
    const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pa);
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * D * 2));
    const u32x2 w0 = __builtin_bit_cast(u32x2, x0), w1 = __builtin_bit_cast(u32x2, x1);
    return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
  };

  // Softmax of one 32-key block for both query blocks, 16 slices per block
  // (slice u of block x runs in group 2u + x of the step).  Per block x,
  // elements 2j and 2j+1 (acc reg 4r+i holds key 8r + 4hh + i):
  //   slice 2j:   argument fma of the pair; rounding and summing of pair j-1
  //   slice 2j+1: exponentials of the pair
  // so no slice waits on its own results; pair 7 is finished after the rounds.
  float sm_f[QB][2], sm_e[QB][2], sm_ps[QB][2], sm_lold[QB];
  bool sm_bad[QB];
  int dirty = 0;
  const float ps_max = __builtin_amdgcn_exp2f(kQ2Slack);
  auto sm_slice = [&](auto u_c, auto x_c, const f32x16 (&acc)[QB], bf16x2 (&pkc)[QB][8]) __attribute__((always_inline)) {
    constexpr int u = decltype(u_c)::value, x = decltype(x_c)::value, j = u >> 1;
    if constexpr ((u & 1) == 0) {
      sm_f[x][0] = fmaf(acc[x][2 * j], p.scale_log2, -mrun[x]);
      sm_f[x][1] = fmaf(acc[x][2 * j + 1], p.scale_log2, -mrun[x]);
      pin(sm_f[x][0]);
      pin(sm_f[x][1]);
      if constexpr (j >= 1) {
        bf16x2 pr;
        pr[0] = (__bf16)sm_e[x][0];
        pr[1] = (__bf16)sm_e[x][1];
        pkc[x][j - 1] = pr;
        pin(pkc[x][j - 1]);
        if constexpr (j == 1) {
          sm_ps[x][0] = sm_e[x][0];
          sm_ps[x][1] = sm_e[x][1];
        } else {
          sm_ps[x][0] += sm_e[x][0];
          sm_ps[x][1] += sm_e[x][1];
        }
        pin(sm_ps[x][0]);
        pin(sm_ps[x][1]);
      }
    } else {
      sm_e[x][0] = __builtin_amdgcn_exp2f(sm_f[x][0]);
      sm_e[x][1] = __builtin_amdgcn_exp2f(sm_f[x][1]);
      pin(sm_e[x][0]);
      pin(sm_e[x][1]);
    }
  };
  // Pair 7 and the block's row sum; CHECK: test the bound.
  auto sm_finish = [&](auto x_c, auto check_c, bf16x2 (&pkc)[QB][8]) __attribute__((always_inline)) {
    constexpr int x = decltype(x_c)::value;
    bf16x2 pr;
    pr[0] = (__bf16)sm_e[x][0];
    pr[1] = (__bf16)sm_e[x][1];
    pkc[x][7] = pr;
    const float ps = (sm_ps[x][0] + sm_e[x][0]) + (sm_ps[x][1] + sm_e[x][1]);
    if constexpr (decltype(check_c)::value) sm_bad[x] = __any(!(ps <= ps_max));
    sm_lold[x] = lsum[x];
    lsum[x] += ps;
  };
  // The rare path: redo block x against its true maximum (merged over the two
  // lanes that hold a query's keys), rounded up to an integer.  Before the
  // first accepted block nothing has been accumulated; after it, the
  // accumulators no longer match the new reference and the tile is marked
  // for a second pass.
  auto sm_redo = [&](auto x_c, const f32x16 (&acc)[QB], bf16x2 (&pkc)[QB][8]) __attribute__((always_inline)) {
    constexpr int x = decltype(x_c)::value;
    const f32x16& a = acc[x];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, a[i]);
    const float mold = mrun[x];
    const float mnew = fmaxf(mold, ceilf(half_max(mx) * p.scale_log2));
    dirty |= (int)(mold != -INFINITY && mnew != mold);
    mrun[x] = mnew;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(a[2 * i], p.scale_log2, -mnew));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(a[2 * i + 1], p.scale_log2, -mnew));
      pkc[x][i][0] = (__bf16)e0;
      pkc[x][i][1] = (__bf16)e1;
      ps += e0 + e1;
    }
    lsum[x] = mold == -INFINITY ? ps : fmaf(sm_lold[x], __builtin_amdgcn_exp2f(mold - mnew), ps);
  };
  // keys at or past `valid` get score -inf (acc reg i holds key
  // 8(i/4) + 4hh + i%4; compared as constant >= valid - 4hh, so no per-key
  // lane values are kept live)
  auto sm_mask = [&](f32x16 (&acc)[QB], int valid) __attribute__((always_inline)) {
    const int vrel = valid - 4 * hh;
#pragma unroll
    for (int x = 0; x < QB; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) >= vrel) acc[x][i] = -INFINITY;
  };
  // Tile loads of a period's first step, one per round: K of visit t+1 and
  // V of visit t (their buffers were last read in period t-1); tk, tv are the
  // first keys of those visits.
  auto stage_op = [&](auto j_c, auto par_c, int t, int64_t tk, int64_t tv) __attribute__((always_inline)) {
    constexpr int j = decltype(j_c)::value;
    if constexpr (j < LPW) dma_k(kbuf(par_c, t, A1{}), tk, j);
    else dma_v(vbuf(par_c, t, A0{}), tv, j - LPW);
  };

  // One step.  F: flags; BASE: ring slot of round 0; CHECK: test the softmax
  // bound (first pass).  PRE_K / PRE_V: the period's second step needs K / V
  // fragments, prefetched in rounds 6 and 7.
  enum : int { kQK = 1, kSM = 2, kPV = 4, kMASK = 8, kSTAGE = 16, kPRE_K = 32, kPRE_V = 64 };
  auto step = [&](auto f_c, auto base_c, auto par_c, auto check_c, int t, const unsigned char* kt, int qh,
                  f32x16 (&acc_next)[QB], f32x16 (&acc_cur)[QB], bf16x2 (&pk_cur)[QB][8], int valid,
                  const unsigned char* vt, int vh, const bf16x2 (&pk_prev)[QB][8], int64_t tk, int64_t tv)
                  __attribute__((always_inline)) {
    constexpr int F = decltype(f_c)::value, base = decltype(base_c)::value;
    constexpr bool QK = F & kQK, SM = F & kSM, PV = F & kPV, CHECK = decltype(check_c)::value;
    if constexpr (SM && (F & kMASK)) {
      if (valid < 32) sm_mask(acc_cur, valid);
    }
    static_for<0, 8>([&](auto r_c) __attribute__((always_inline)) {
      constexpr int r = decltype(r_c)::value;
      constexpr int slot = (base + r) % 3, pre = (base + r + 2) % 3;
      constexpr int ks = r >> 2, nb = r & 3;
      // group 0: LDS reads two rounds ahead, QK^T for query block 0
      if constexpr (r + 2 < 8) {
        if constexpr (QK) kf[pre] = read_k(kt, qh, r + 2);
        if constexpr (PV) vf[pre] = read_v(vt, vh, r + 2);
      } else {
        if constexpr ((F & kPRE_K) != 0) kf[pre] = read_k(kt, qh + 1, r - 6);
        if constexpr ((F & kPRE_V) != 0) vf[pre] = read_v(vt, vh + 1, r - 6);
      }
      if constexpr (QK) {
        if constexpr (r == 0) mfma_qk_first(acc_next[0], kf[slot], qf[0][r]);
        else mfma_qk(acc_next[0], kf[slot], qf[0][r]);
      }
      if constexpr (SM) sm_slice(std::integral_constant<int, 2 * r>{}, A0{}, acc_cur, pk_cur);
      __builtin_amdgcn_sched_barrier(0);
      // group 1: QK^T for query block 1
      if constexpr (QK) {
        if constexpr (r == 0) mfma_qk_first(acc_next[1], kf[slot], qf[1][r]);
        else mfma_qk(acc_next[1], kf[slot], qf[1][r]);
      }
      if constexpr (SM) sm_slice(std::integral_constant<int, 2 * r>{}, A1{}, acc_cur, pk_cur);
      __builtin_amdgcn_sched_barrier(0);
      // group 2: P V for query block 0 (+ staged-tile work)
      if constexpr (PV) {
        const u32x4 w4 = {__builtin_bit_cast(uint32_t, pk_prev[0][4 * ks]), __builtin_bit_cast(uint32_t, pk_prev[0][4 * ks + 1]),
                          __builtin_bit_cast(uint32_t, pk_prev[0][4 * ks + 2]), __builtin_bit_cast(uint32_t, pk_prev[0][4 * ks + 3])};
        o[0][nb] = mfma32(vf[slot], __builtin_bit_cast(bf16x8, w4), o[0][nb]);
        pin_acc(o[0][nb]);
      }
      if constexpr ((F & kSTAGE) != 0) {
        static_for<0, LPW / 4>([&](auto o_c) __attribute__((always_inline)) {
          stage_op(std::integral_constant<int, r * (LPW / 4) + decltype(o_c)::value>{}, par_c, t, tk, tv);
        });
      }
      if constexpr (SM) sm_slice(std::integral_constant<int, 2 * r + 1>{}, A0{}, acc_cur, pk_cur);
      __builtin_amdgcn_sched_barrier(0);
      // group 3: P V for query block 1
      if constexpr (PV) {
        const u32x4 w4 = {__builtin_bit_cast(uint32_t, pk_prev[1][4 * ks]), __builtin_bit_cast(uint32_t, pk_prev[1][4 * ks + 1]),
                          __builtin_bit_cast(uint32_t, pk_prev[1][4 * ks + 2]), __builtin_bit_cast(uint32_t, pk_prev[1][4 * ks + 3])};
        o[1][nb] = mfma32(vf[slot], __builtin_bit_cast(bf16x8, w4), o[1][nb]);
        pin_acc(o[1][nb]);
      }
      if constexpr (SM) sm_slice(std::integral_constant<int, 2 * r + 1>{}, A1{}, acc_cur, pk_cur);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (SM) {
      sm_finish(A0{}, check_c, pk_cur);
      sm_finish(A1{}, check_c, pk_cur);
      if constexpr (CHECK) {
        if (__builtin_expect(sm_bad[0] | sm_bad[1], 0)) {
          if (sm_bad[0]) sm_redo(A0{}, acc_cur, pk_cur);
          if (sm_bad[1]) sm_redo(A1{}, acc_cur, pk_cur);
        }
      }
    }
  };
  // Period t: steps A and B with flags FA, FB (prefetch flags derived here).
  auto period = [&](int t, auto par_c, auto check_c, auto fa_c, auto fb_c, int valid_a, int valid_b) __attribute__((always_inline)) {
    constexpr int FA0 = decltype(fa_c)::value, FB = decltype(fb_c)::value;
    constexpr int FA = FA0 | ((FB & kQK) ? kPRE_K : 0) | ((FB & kPV) ? kPRE_V : 0);
    const unsigned char* kt = kbuf(par_c, t, A0{});
    const unsigned char* vprev = vbuf(par_c, t, Am1{});
    int64_t tk = 0, tv = 0;  // first keys of the visits staged in this period
    if constexpr ((FA0 & kSTAGE) != 0) {
      tk = act_key(t + 1);
      tv = act_key(t);
    }
    if constexpr ((FA & kQK) != 0) {
      kf[0] = read_k(kt, 0, 0);
      kf[1] = read_k(kt, 0, 1);
    }
    if constexpr ((FA & kPV) != 0) {
      vf[0] = read_v(vprev, 0, 0);
      vf[1] = read_v(vprev, 0, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    step(std::integral_constant<int, FA>{}, A0{}, par_c, check_c, t, kt, 0, sacc[0], sacc[1], pk[1], valid_a, vprev, 0, pk[0],
         tk, tv);
    step(std::integral_constant<int, FB>{}, std::integral_constant<int, 2>{}, par_c, check_c, t, kt, 1, sacc[1], sacc[0], pk[0],
         valid_b, vprev, 1, pk[1], tk, tv);
  };
  using C0 = std::integral_constant<int, kQK | kSTAGE>;
  using C1 = std::integral_constant<int, kQK | kSM | kMASK>;
  using CA = std::integral_constant<int, kQK | kSM | kPV | kSTAGE>;
  using CB = std::integral_constant<int, kQK | kSM | kPV>;
  using CAm = std::integral_constant<int, kQK | kSM | kPV | kSTAGE | kMASK>;
  using CBm = std::integral_constant<int, kQK | kSM | kPV | kMASK>;
  using CTa = std::integral_constant<int, kSM | kPV | kMASK>;
  using CTb = std::integral_constant<int, kPV>;

  // The whole window: period t (0 <= t <= T) covers K tile t and V tile t-1.
  // Its first step also moves the staged tiles: LDS stores of K tile t+1 and
  // V tile t from registers, buffer loads of K tile t+2 and V tile t+1
  // (tiles past the window read as zeros and are never used).
  auto pipeline = [&](auto check_c) __attribute__((always_inline)) {
    // prologue: K tile 0 (its loads issued at the start of the pass) in LDS
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __syncthreads();
    period(0, A0{}, check_c, C0{}, C1{}, 32, block_valid(0));
    __syncthreads();
    // steady state: every block of K tile t and V tile t-1 is full; two
    // periods per iteration so the buffer parity is known
    // (anchored passes: the anchor segment's last tile may be partial too,
    // so every period tests its blocks)
    using SA = std::conditional_t<ANCH, CAm, CA>;
    using SB = std::conditional_t<ANCH, CBm, CB>;
    auto va = [&](int t) __attribute__((always_inline)) { return ANCH ? block_valid(2 * t - 1) : 32; };
    auto vb = [&](int t) __attribute__((always_inline)) { return ANCH ? block_valid(2 * t) : 32; };
    int t = 1;
    for (; t + 2 < Tp; t += 2) {
      period(t, A1{}, check_c, SA{}, SB{}, va(t), vb(t));
      __syncthreads();
      period(t + 1, A0{}, check_c, SA{}, SB{}, va(t + 1), vb(t + 1));
      __syncthreads();
    }
    if (t + 1 < Tp) {
      period(t, A1{}, check_c, SA{}, SB{}, va(t), vb(t));
      __syncthreads();
    }
    if (Tp > 1) {  // period Tp-1: the last K tile (may be partial)
      period(Tp - 1, Am1{}, check_c, SA{}, CBm{}, va(Tp - 1), block_valid(2 * Tp - 2));
      __syncthreads();
    }
    // period Tp: softmax of the last block, P V of the last V tile
    period(Tp, Am1{}, check_c, CTa{}, CTb{}, block_valid(2 * Tp - 1), 32);
  };

  init_acc();
  if (Tp > 0) pipeline(std::integral_constant<bool, FIRST>{});

  // ---- epilogue: normalise, stage bf16 rows in LDS (per wave), write
  // coalesced.  A split pass writes its rows, normalised by its own
  // denominator, to its partial-result slot (row stride D), and beside them
  // per row {denominator, reference}; the merge weighs the slots.
  __syncthreads();
  unsigned char* stage = wave == 0 ? kb0 : wave == 1 ? kb1 : wave == 2 ? vb0 : vb1;
  bf16_t* obase;
  int64_t ostride;
  float* plm = nullptr;
  if constexpr (PARTIAL) {
    const int64_t pidx = ((int64_t)bh * p.tiles_per_chunk + tile) * p.n_splits + split;
    const int64_t n_part = (int64_t)p.B * p.H * p.tiles_per_chunk * p.n_splits;
    obase = reinterpret_cast<bf16_t*>(p.part) + pidx * BM * D;
    ostride = D;
    plm = reinterpret_cast<float*>(reinterpret_cast<bf16_t*>(p.part) + n_part * BM * D) + pidx * BM * 2;
  } else {
    obase = (bf16_t*)p.out + b * p.q_sb + h * p.q_sh + qtok0 * p.q_st;
    ostride = p.q_st;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = half_sum(lsum[qb]);
    // (a pruned pass can leave a row with no weight at all: output 0)
    const float inv = SPARSE || PARTIAL ? (ltot > 0.f ? 1.0f / ltot : 0.f) : 1.0f / ltot;
    const int r = qb * 32 + l32;  // row within the wave's 64
#pragma unroll
    for (int nb = 0; nb < DB; ++nb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int col = nb * 32 + 8 * rr + 4 * hh;
        const int g = col >> 3;
        u32x2 pr = {pack_bf16(o[qb][nb][4 * rr] * inv, o[qb][nb][4 * rr + 1] * inv),
                    pack_bf16(o[qb][nb][4 * rr + 2] * inv, o[qb][nb][4 * rr + 3] * inv)};
        *reinterpret_cast<u32x2*>(stage + r * D * 2 + ((g ^ ksw<D>(r)) * 16) + (col & 7) * 2) = pr;
      }
    const int myrow = wave * 32 * QB + r;
    if (hh == 0 && myrow < nrows) {
      if constexpr (PARTIAL) {
        plm[myrow * 2] = ltot;
        plm[myrow * 2 + 1] = mrun[qb];
      } else if (p.lse != nullptr) {
        const int64_t L = (int64_t)p.n_qchunks * p.C;
        p.lse[(int64_t)bh * L + qtok0 + myrow] = (mrun[qb] + __log2f(ltot)) * kLn2;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's staging writes are complete
  __builtin_amdgcn_wave_barrier();
  for (int idx = lane; idx < 32 * QB * GR; idx += 64) {
    const int r = idx / GR, g = idx % GR;
    const int row = wave * 32 * QB + r;
    if (row < nrows)
      st16(obase + (int64_t)row * ostride + g * 8, *reinterpret_cast<const u32x4*>(stage + r * D * 2 + ((g ^ ksw<D>(r)) * 16)));
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mio[qb] = mrun[qb];
  return dirty;
}

// ---- Short chunk tails (causal or bidirectional window, seq mode).
// Rows C - tail_rows .. C - 1 of chunk c (at most 32), the chunk's last tile
// in the launch order (so it runs next to the chunk's other tiles, on the same
// XCD, while their keys are in L2).
// Wave i takes the i-th quarter of the window's 32-key blocks with its own
// running maximum m_i and sum l_i (plain online softmax, rescaled when the
// maximum grows); the linear term enters every wave at reference 0, wave i
// taking output features 32i .. 32i+31 of phi(Q) S and wave 0 the
// denominator term phi(q).z.  The four partial results meet in LDS:
//   out = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
// Products as in the tiles: S^T = K Q^T (one query per lane; K rows straight
// from memory as the first operand), O^T += V^T P^T with V staged in the
// wave's own LDS buffer for the transposed read; blocks go in pairs, the next
// pair's rows in flight in registers.
// A pruned pass (SPARSE) visits only the 32-key blocks of kept 64-key tiles
// (mask row: query tile C / 256 of the chunk); an anchored pass (ANCH) also
// visits the anchor chunks' keys.  In stream mode the keys are
// the cache rows and the state is the head's; a split pass (PARTIAL) covers
// its split's share of the key tiles and writes the unnormalised partial
// result in the split layout, as the tiles do.
constexpr int kTailMaxRows = 32;

template <bool SPARSE, bool PARTIAL, bool ANCH>
__device__ __noinline__ void tail_pass(const FwdParams pin) {
  using namespace frag;
  // The parameters are the same in every lane; copies through readfirstlane
  // let the compiler keep them (and the block loops) scalar in this
  // out-of-line function.
  auto rfl = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto rfl64 = [](int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x), hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  auto uni = [&](const void* ptr) { return (void*)rfl64((int64_t)ptr); };
  struct {
    const void *q, *k, *v;
    void* out;
    float* lse;
    const float *S, *z, *S2, *z2;
    const unsigned char* kmask;
    float* part;
    int64_t q_sb, q_sh, q_st, kv_sb, kv_sh, kv_st;
    int B, H, C, w, n_qchunks, tiles_per_chunk, total_tiles, bidir, tail_rows, mask_qtiles, nkt, anchors;
    int stream_mode, n_keys, has_state, n_splits;
    float scale_log2;
  } p;
  p.q = uni(pin.q);
  p.k = uni(pin.k);
  p.v = uni(pin.v);
  p.out = uni(pin.out);
  p.lse = (float*)uni(pin.lse);
  p.S = (const float*)uni(pin.S);
  p.z = (const float*)uni(pin.z);
  p.S2 = (const float*)uni(pin.S2);
  p.z2 = (const float*)uni(pin.z2);
  p.kmask = (const unsigned char*)uni(pin.kmask);
  p.part = (float*)uni(pin.part);
  p.B = rfl(pin.B);
  p.stream_mode = rfl(pin.stream_mode);
  p.n_keys = rfl(pin.n_keys);
  p.has_state = rfl(pin.has_state);
  p.n_splits = rfl(pin.n_splits);
  p.q_sb = rfl64(pin.q_sb);
  p.q_sh = rfl64(pin.q_sh);
  p.q_st = rfl64(pin.q_st);
  p.kv_sb = rfl64(pin.kv_sb);
  p.kv_sh = rfl64(pin.kv_sh);
  p.kv_st = rfl64(pin.kv_st);
  p.H = rfl(pin.H);
  p.C = rfl(pin.C);
  p.w = rfl(pin.w);
  p.n_qchunks = rfl(pin.n_qchunks);
  p.tiles_per_chunk = rfl(pin.tiles_per_chunk);
  p.total_tiles = rfl(pin.total_tiles);
  p.bidir = rfl(pin.bidir);
  p.tail_rows = rfl(pin.tail_rows);
  p.mask_qtiles = rfl(pin.mask_qtiles);
  p.nkt = rfl(pin.nkt);
  p.anchors = rfl(pin.anchors);
  p.scale_log2 = __int_as_float(rfl(__float_as_int(pin.scale_log2)));
  static_assert(Q2_NW == 4 && Q2_TILE == 2 * ROWT, "four waves, each with a buffer for a 32-key block of K and V");
  static_assert(Q2_TILE == BD * 32 * 4, "one wave's partial output (128 features x 32 rows, float32) fits its buffer");
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block loops stay scalar
  // which tail, as in tile_pass
  const int logical0 = launch_order(blockIdx.x, p.total_tiles, p.tiles_per_chunk, !PARTIAL);
  const int split = PARTIAL ? logical0 % p.n_splits : 0;
  const int rest = (PARTIAL ? logical0 / p.n_splits : logical0) / p.tiles_per_chunk;
  const int c = p.n_qchunks - 1 - rest % p.n_qchunks;
  const int bh = rest / p.n_qchunks;
  const int b = bh / p.H, h = bh % p.H;
  const int nr = p.tail_rows;  // 1 .. kTailMaxRows (checked by the launcher)
  const int r0 = p.C - nr;
  const int64_t qtok0 = (int64_t)c * p.C + r0;
  const bf16_t* kbase = (const bf16_t*)p.k + b * p.kv_sb + h * p.kv_sh;
  const bf16_t* vbase = (const bf16_t*)p.v + b * p.kv_sb + h * p.kv_sh;

  int64_t kbeg = 0, kend = 0;
  bool has_past, has_future = false;
  int64_t slot;  // state slot
  if (!p.stream_mode) {
    if (p.w > 0) {
      kbeg = (int64_t)max(0, c - p.w + 1) * p.C;
      kend = (int64_t)(p.bidir ? min(p.n_qchunks, c + p.w) : c + 1) * p.C;
    }
    has_past = ANCH ? (c - p.w >= p.anchors) : ((p.w == 0) || (c >= p.w));
    has_future = p.bidir && c + max(p.w, 1) <= p.n_qchunks - 1;
    slot = (int64_t)bh * p.n_qchunks + c;
  } else {
    kend = p.n_keys;
    has_past = p.has_state != 0;
    if (PARTIAL) {  // this split's share of the 64-key tiles; the first split takes the state
      const int tiles_all = (p.n_keys + BN - 1) / BN;
      const int t_lo = (int)((int64_t)split * tiles_all / p.n_splits);
      const int t_hi = (int)((int64_t)(split + 1) * tiles_all / p.n_splits);
      kbeg = (int64_t)t_lo * BN;
      kend = min((int64_t)t_hi * BN, (int64_t)p.n_keys);
      has_past = has_past && split == 0;
    }
    slot = bh;
  }

  // Q rows of the tail, second operand, one query per lane (lanes past the
  // tail repeat its last row; their results are not written)
  bf16x8 qf[8];
  {
    const bf16_t* qrow = (const bf16_t*)p.q + b * p.q_sb + h * p.q_sh + (qtok0 + min(l32, nr - 1)) * p.q_st;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qrow + 16 * ks + 8 * hh));
  }
  unsigned char* const vbuf = wave == 0 ? q2_kb0 : wave == 1 ? q2_kb1 : wave == 2 ? q2_vb0 : q2_vb1;
  f32x16 o[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) o[nb] = f32x16{};
  float m = -INFINITY, l = 0.f;

  if (has_past || has_future) {
    // Wave i: output features v = 32 i + lane % 32 of phi(Q) S at reference 0.
    // The first operand holds S[16 ks + 8 (lane / 32) + 0..7][v], read straight
    // from memory (32 lanes read 32 consecutive floats of a row of S).
    const float* Sp = p.S + slot * BD * BD + 32 * wave + l32;
    const float* Sp2 = p.bidir ? p.S2 + slot * BD * BD + 32 * wave + l32 : nullptr;
    // every load in flight at once: the state slot is always addressable, so
    // the past state is loaded unconditionally and dropped when absent
    float col[8][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) col[ks][e] = Sp[(16 * ks + 8 * hh + e) * BD];
    if (!has_past) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) col[ks][e] = 0.f;
    }
    if (has_future) {
      float c2[8][8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) c2[ks][e] = Sp2[(16 * ks + 8 * hh + e) * BD];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) col[ks][e] += c2[ks][e];
    }
    f32x16 t = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 a = {pack_bf16(col[ks][0], col[ks][1]), pack_bf16(col[ks][2], col[ks][3]),
                       pack_bf16(col[ks][4], col[ks][5]), pack_bf16(col[ks][6], col[ks][7])};
      t = mfma32(__builtin_bit_cast(bf16x8, a), phi8(qf[ks]), t);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      if (nb == wave) o[nb] = t;
    if (wave == 0) {  // phi(q).z, summed over both halves of the features
      const float* zp = p.z + slot * BD;
      const float* zp2 = p.bidir ? p.z2 + slot * BD : nullptr;
      f32x4 zz[8][2];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        zz[ks][0] = *reinterpret_cast<const f32x4*>(zp + 16 * ks + 8 * hh);
        zz[ks][1] = *reinterpret_cast<const f32x4*>(zp + 16 * ks + 8 * hh + 4);
      }
      if (!has_past) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) zz[ks][0] = zz[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (has_future) {
        f32x4 z2[8][2];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          z2[ks][0] = *reinterpret_cast<const f32x4*>(zp2 + 16 * ks + 8 * hh);
          z2[ks][1] = *reinterpret_cast<const f32x4*>(zp2 + 16 * ks + 8 * hh + 4);
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          zz[ks][0] += z2[ks][0];
          zz[ks][1] += z2[ks][1];
        }
      }
      float acc = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 x = __builtin_bit_cast(u32x4, qf[ks]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qv = (e & 1) ? bf16_hi(x[e >> 1]) : bf16_lo(x[e >> 1]);
          acc = fmaf(phi(qv), e < 4 ? zz[ks][0][e] : zz[ks][1][e - 4], acc);
        }
      }
      const float tot = half_sum(acc);  // the lane swap needs every lane active
      l = hh == 0 ? tot : 0.f;
    }
    m = 0.f;
  }

  // this wave's quarter of the window's 32-key blocks
  // Visited keys: [0, r0e) (anchored passes: the anchor chunks not in the
  // query's future, merged with the window when they touch) and the window
  // [r1b, r1e), each cut into 32-key blocks from its start; block j < nA
  // lies in the first range.
  int64_t r0e = 0, r1b = kbeg, r1e = kend;
  if constexpr (ANCH) {
    r0e = (int64_t)min(p.anchors, c + 1) * p.C;
    if (r1e <= r1b) r1b = r1e = 0;  // no window (w = 0)
    if (r1e > r1b && r1b <= r0e) {  // contiguous union
      r0e = max(r0e, r1e);
      r1b = r1e = 0;
    }
    kend = max(r0e, r1e);  // the descriptors cover every visited key
  }
  const int nA = (int)((r0e + RB - 1) / RB);
  const int nblk = nA + (int)((r1e - r1b + RB - 1) / RB);
  const int j0 = wave * nblk / Q2_NW, j1 = (wave + 1) * nblk / Q2_NW;
  auto blk_start = [&](int j) { return j < nA ? (int64_t)RB * j : r1b + (int64_t)RB * (j - nA); };
  auto blk_end = [&](int j) { return j < nA ? r0e : r1e; };
  const unsigned char* mrow =
      SPARSE ? p.kmask + (((int64_t)bh * p.n_qchunks + c) * p.mask_qtiles + p.mask_qtiles - 1) * p.nkt +
                   (p.stream_mode ? kbeg / 64 : 0)
             : nullptr;
  // first visited block at or after j (j1 if none); the mask byte is the same
  // in every lane, and readfirstlane keeps the search (and the block loop
  // after it) in scalar control flow: the transposed reads and lane swaps of
  // the loop body need every lane of the wave active
  auto next_kept = [&](int j) {
    if constexpr (SPARSE)
      while (j < j1 && __builtin_amdgcn_readfirstlane((int)mrow[j >> 1]) == 0) ++j;
    return j;
  };
  // Blocks are taken in pairs (an odd count ends with a padding block past
  // the window, fully masked).  Per pair: V rows go to the wave's LDS buffer
  // (8 KB per block) and the next pair's V is loaded; S^T = K Q^T for both
  // blocks as two interleaved product chains (K rows straight from memory
  // as the first operand); the next pair's K is loaded; one online-softmax
  // step over both blocks; then O^T += V^T P^T for both.  Buffer loads whose
  // descriptors end at the window end read zeros past it (and for padding).
  const int row_bytes = (int)p.kv_st * 2;
  const int win_bytes = (int)(kend * p.kv_st * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, win_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, win_bytes, kBufWord3);
  auto blk_off = [&](int j) { return j < j1 ? (int)(blk_start(j) * p.kv_st * 2) : win_bytes; };
  const int vofs = (lane >> 4) * row_bytes + (lane & 15) * 16;  // V: 16 lanes per 256-byte row
  const int kofs = l32 * row_bytes + hh * 16;                   // K: row lane % 32, features 8 (lane / 32) + 16 ks
  u32x4 kr[2][8], vr[2][8];
  auto load_k = [&](int ja_, int jb_) __attribute__((always_inline)) {
    const int oa = blk_off(ja_) + kofs, ob = blk_off(jb_) + kofs;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kr[0][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, oa + 32 * ks, 0, 0));
      kr[1][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, ob + 32 * ks, 0, 0));
    }
  };
  auto load_v = [&](int ja_, int jb_) __attribute__((always_inline)) {
    const int oa = blk_off(ja_) + vofs, ob = blk_off(jb_) + vofs;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vr[0][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, oa + 4 * i * row_bytes, 0, 0));
      vr[1][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, ob + 4 * i * row_bytes, 0, 0));
    }
  };
  auto nk_of = [&](int j) { return j < j1 ? (int)min((int64_t)RB, blk_end(j) - blk_start(j)) : 0; };
  unsigned char* const vt[2] = {vbuf, vbuf + ROWT};
  int ja = next_kept(j0);
  int jb = ja < j1 ? next_kept(ja + 1) : j1;
  load_v(ja, jb);
  load_k(ja, jb);
  while (ja < j1) {
    const int na = jb < j1 ? next_kept(jb + 1) : j1;
    const int nb_ = na < j1 ? next_kept(na + 1) : j1;
    // the wave's LDS operations run in order: these writes land after the
    // previous pair's reads
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int i = 0; i < 8; ++i) put_granule(vt[sl], (lane >> 4) + 4 * i, lane & 15, vr[sl][i]);
    load_v(na, nb_);
    f32x16 sa[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) sa[sl] = mfma32(__builtin_bit_cast(bf16x8, kr[sl][ks]), qf[ks], sa[sl]);
    load_k(na, nb_);
    const int nk[2] = {nk_of(ja), nk_of(jb)};
    float bm = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (nk[sl] == RB) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sa[sl][i] *= p.scale_log2;
          bm = fmaxf(bm, sa[sl][i]);
        }
      } else {  // the window's last, partial block, or padding
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sa[sl][i] = out_row(i, hh) < nk[sl] ? sa[sl][i] * p.scale_log2 : -INFINITY;
          bm = fmaxf(bm, sa[sl][i]);
        }
      }
    }
    const float mn = fmaxf(m, half_max(bm));
    if (__any(mn > m)) {
      const float sc = exp2f(m - mn);
      l *= sc;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) o[nb] *= sc;
      m = mn;
    }
    uint32_t pp[2][8];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sa[sl][i] - m), p1 = __builtin_amdgcn_exp2f(sa[sl][i + 1] - m);
        l += p0 + p1;
        pp[sl][i >> 1] = pack_bf16(p0, p1);
      }
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) o[nb] = mfma32(col_frag(vt[sl], ks, nb, lane), pack_b(pp[sl], ks), o[nb]);  // O^T += V^T P^T
    ja = na;
    jb = nb_;
  }

  // ---- merge: partial O^T [feature][row] in the wave's buffer, m and l per row
  float* const ow = reinterpret_cast<float*>(vbuf);
  float* const sm = reinterpret_cast<float*>(q2_act);   // [wave][32]
  float* const sl = reinterpret_cast<float*>(q2_actv);  // [wave][half][32]
  __syncthreads();  // every wave is done with its V blocks
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) ow[(32 * nb + out_row(i, hh)) * 32 + l32] = o[nb][i];
  if (hh == 0) sm[wave * 32 + l32] = m;
  sl[(wave * 2 + hh) * 32 + l32] = l;
  __syncthreads();
  const int q = tid & 31, f0 = (tid >> 5) * 16;
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < Q2_NW; ++i) M = fmaxf(M, sm[i * 32 + q]);
  float sc[Q2_NW], den = 0.f;
#pragma unroll
  for (int i = 0; i < Q2_NW; ++i) {
    const float mi = sm[i * 32 + q];
    sc[i] = mi == -INFINITY ? 0.f : exp2f(mi - M);
    den = fmaf(sc[i], sl[(i * 2) * 32 + q] + sl[(i * 2 + 1) * 32 + q], den);
  }
  const float* o0 = reinterpret_cast<const float*>(q2_kb0);
  const float* o1 = reinterpret_cast<const float*>(q2_kb1);
  const float* o2 = reinterpret_cast<const float*>(q2_vb0);
  const float* o3 = reinterpret_cast<const float*>(q2_vb1);
  if (PARTIAL && q < nr) {
    // split layout: bf16 rows normalised by the split's own denominator,
    // then {denominator, M}; the tail is the chunk's last tile, rows 0 ..
    // nr-1 of it
    constexpr int BM = Q2_NW * 32 * Q2_QB;
    const int64_t pidx = ((int64_t)bh * p.tiles_per_chunk + p.tiles_per_chunk - 1) * p.n_splits + split;
    const int64_t n_part = (int64_t)p.B * p.H * p.tiles_per_chunk * p.n_splits;
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int f = 0; f < 16; f += 2) {
      float v2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int idx = (f0 + f + e) * 32 + q;
        v2[e] = (sc[0] * o0[idx] + sc[1] * o1[idx] + sc[2] * o2[idx] + sc[3] * o3[idx]) * inv;
      }
      pk[f >> 1] = pack_bf16(v2[0], v2[1]);
    }
    bf16_t* po = reinterpret_cast<bf16_t*>(p.part) + (pidx * BM + q) * BD + f0;
    st16(po, u32x4{pk[0], pk[1], pk[2], pk[3]});
    st16(po + 8, u32x4{pk[4], pk[5], pk[6], pk[7]});
    if (f0 == 0) {
      float* plm = reinterpret_cast<float*>(reinterpret_cast<bf16_t*>(p.part) + n_part * BM * BD) + (pidx * BM + q) * 2;
      plm[0] = den;
      plm[1] = M;
    }
  }
  if (!PARTIAL && q < nr) {
    const float inv = den > 0.f ? 1.0f / den : 0.f;  // no weight at all (everything pruned, no state): 0
    uint32_t pk[8];
#pragma unroll
    for (int f = 0; f < 16; f += 2) {
      float v2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int idx = (f0 + f + e) * 32 + q;
        v2[e] = (sc[0] * o0[idx] + sc[1] * o1[idx] + sc[2] * o2[idx] + sc[3] * o3[idx]) * inv;
      }
      pk[f >> 1] = pack_bf16(v2[0], v2[1]);
    }
    bf16_t* dst = (bf16_t*)p.out + b * p.q_sb + h * p.q_sh + (qtok0 + q) * p.q_st + f0;
    st16(dst, u32x4{pk[0], pk[1], pk[2], pk[3]});
    st16(dst + 8, u32x4{pk[4], pk[5], pk[6], pk[7]});
    if (p.lse != nullptr && f0 == 0)
      p.lse[(int64_t)bh * p.n_qchunks * p.C + qtok0 + q] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
  }
}

// The rare second pass, kept out of line so that its registers do not add to
// the first pass's.
template <int D, int NW, bool PARTIAL, int VIS>
__device__ __noinline__ void tile_second_pass(const FwdParams p, float m0, float m1) {
  float m[Q2_QB] = {m0, m1};
  tile_pass<D, NW, false, PARTIAL, VIS>(p, m);
}

// A split pass (PARTIAL) may carry the units of the streaming fold (partial
// states of the chunk leaving the window, `fold`; fold.k set): they run where
// the attention leaves compute units idle -- after the short tails (which end
// long before the full tiles), tail workgroup i taking units i, i + n_tails,
// ..., or, in a pass without tails, in extra workgroups after its
// p.total_tiles tiles.
template <int D, int NW>
__device__ __forceinline__ void fold_unit(const ChunkStateParams& fold, int u) {
  static_assert(NW * 64 == state::THREADS && state::StateCfg<D>::KBYTES * 2 <= Q2_TILE &&
                    state::StateCfg<D>::VBYTES <= Q2_TILE &&
                    sizeof(float) * (state::THREADS / (state::ESLICE / 8)) * state::ESLICE <= Q2_TILE,
                "the fold unit's buffers fit the tile buffers");
  state::chunk_state_unit<D, false>(fold, u, q2_kb0, q2_vb0, q2_vb1, reinterpret_cast<float*>(q2_kb1));
}

template <int D, int NW, bool PARTIAL, int VIS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_qb2_kernel(const FwdParams p, const ChunkStateParams fold) {
  if constexpr (PARTIAL) {
    if ((int)blockIdx.x >= p.total_tiles) {
      fold_unit<D, NW>(fold, (int)blockIdx.x - p.total_tiles);
      return;
    }
  }
  {
    const int logical0 = launch_order(blockIdx.x, p.total_tiles, p.tiles_per_chunk, !PARTIAL && p.tail_rows > 0);
    const int logical = logical0 / (PARTIAL ? p.n_splits : 1);
    if (p.tail_rows > 0 && logical % p.tiles_per_chunk == p.tiles_per_chunk - 1) {
      // a chunk's short tail (the parameter block by value: a pointer to it
      // measured slower, the callee then saves most of its registers)
      tail_pass<VIS == 1, PARTIAL, VIS == 2>(p);
      if constexpr (PARTIAL) {
        if (fold.k != nullptr) {
          const int n_tails = p.total_tiles / p.tiles_per_chunk;
          const int units = fold.B * fold.H * fold.n_chunks * state::StateCfg<D>::ES;
          for (int u = (logical / p.tiles_per_chunk) * p.n_splits + logical0 % p.n_splits; u < units; u += n_tails) {
            __syncthreads();  // the tile buffers are free
            fold_unit<D, NW>(fold, u);
          }
        }
      }
      return;
    }
  }
  float m[Q2_QB];
  const int dirty = tile_pass<D, NW, true, PARTIAL, VIS>(p, m);
  // Every wave reaches this barrier.  Where some query's reference moved after
  // accumulation, the whole tile is computed again with the final references
  // (which no score exceeds by the bound); its output replaces the first.
  if (__syncthreads_or(dirty)) tile_second_pass<D, NW, PARTIAL, VIS>(p, m[0], m[1]);
}

// Merge of a split pass: per query row, the splits' normalised rows are
// weighted by their denominators brought to the largest reference and summed
// in split order; one thread per 8 output columns.
// Workgroups from fwd_blocks on run the state merge sc instead (the fold of a
// streaming step, merged in the same launch).
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const FwdParams p, const StateCombineParams sc,
                                                          int fwd_blocks) {
  constexpr int BM = Q2_NW * 32 * Q2_QB;
  if ((int)blockIdx.x >= fwd_blocks) {
    state_combine_unit(sc, (int64_t)(blockIdx.x - fwd_blocks) * blockDim.x + threadIdx.x);
    return;
  }
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.H * p.C * (D / 8);
  if (idx >= total) return;
  const int col = (int)(idx % (D / 8)) * 8;
  const int64_t r = idx / (D / 8);
  const int row = (int)(r % p.C);
  const int bh = (int)(r / p.C);
  const int b = bh / p.H, h = bh % p.H;
  const int tile = row / BM, trow = row % BM;
  const int64_t n_part = (int64_t)p.B * p.H * p.tiles_per_chunk * p.n_splits;
  const int64_t pidx0 = ((int64_t)bh * p.tiles_per_chunk + tile) * p.n_splits;
  const bf16_t* pn = reinterpret_cast<const bf16_t*>(p.part);
  const float* plm = reinterpret_cast<const float*>(pn + n_part * BM * D);
  // every split's {denominator, reference} and row slice requested at once
  // (at most kMaxSplits splits)
  f32x2 lmv[kMaxSplits];
  u32x4 xs[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < p.n_splits) {
      lmv[sp] = *reinterpret_cast<const f32x2*>(plm + ((pidx0 + sp) * BM + trow) * 2);
      xs[sp] = ld16(pn + ((pidx0 + sp) * BM + trow) * D + col);
    }
  float mmax = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < p.n_splits) mmax = fmaxf(mmax, lmv[sp][1]);
  // split sp holds its rows normalised by its denominator l_sp at reference
  // m_sp: its weight is l_sp 2^(m_sp - mmax)
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    if (sp >= p.n_splits) break;
    const float wgt = lmv[sp][1] == -INFINITY ? 0.f : lmv[sp][0] * __builtin_amdgcn_exp2f(lmv[sp][1] - mmax);
    den += wgt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      num[2 * i] = fmaf(wgt, bf16_lo(xs[sp][i]), num[2 * i]);
      num[2 * i + 1] = fmaf(wgt, bf16_hi(xs[sp][i]), num[2 * i + 1]);
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;  // (pruned: a row with no weight at all gets 0)
  bf16_t* dst = (bf16_t*)p.out + b * p.q_sb + h * p.q_sh + (int64_t)row * p.q_st + col;
  st16(dst, u32x4{pack_bf16(num[0] * inv, num[1] * inv), pack_bf16(num[2] * inv, num[3] * inv),
                  pack_bf16(num[4] * inv, num[5] * inv), pack_bf16(num[6] * inv, num[7] * inv)});
  if (p.lse != nullptr && col == 0) p.lse[(int64_t)bh * p.C + row] = den > 0.f ? (mmax + __log2f(den)) * kLn2 : -INFINITY;
}

template <int NW>
hipError_t launch_nw(FwdParams& p, hipStream_t s, const ChunkStateParams& fold = ChunkStateParams{},
                     int fold_blocks = 0) {
  constexpr int BM = NW * 32 * Q2_QB;
  static_assert(BM == kQb2RowsPerTile, "partial-result tile size");
  const int splits = p.n_splits > 1 ? p.n_splits : 1;
  // short tails: dense seq-mode passes whose chunks end in 1 .. 32 rows past
  // the last full tile (also chunks of at most 32 rows: no tile at all)
  const int rem = p.C % BM;
  const bool tails = rem > 0 && rem <= kTailMaxRows;
  p.tail_rows = tails ? rem : 0;
  p.mask_qtiles = (p.C + BM - 1) / BM;
  p.tiles_per_chunk = p.mask_qtiles;
  p.total_tiles = p.B * p.H * p.n_qchunks * p.tiles_per_chunk * splits;
  const int64_t grid = p.total_tiles;
  if (grid == 0) return hipSuccess;
  if (splits > 1 && p.kmask != nullptr)
    hipLaunchKernelGGL((fwd_bf16_qb2_kernel<128, NW, true, 1>), dim3((unsigned)(grid + fold_blocks)), dim3(NW * 64), 0,
                       s, p, fold);
  else if (splits > 1)
    hipLaunchKernelGGL((fwd_bf16_qb2_kernel<128, NW, true, 0>), dim3((unsigned)(grid + fold_blocks)), dim3(NW * 64), 0,
                       s, p, fold);
  else if (p.kmask != nullptr)
    hipLaunchKernelGGL((fwd_bf16_qb2_kernel<128, NW, false, 1>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p, fold);
  else if (p.anchors > 0)
    hipLaunchKernelGGL((fwd_bf16_qb2_kernel<128, NW, false, 2>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p, fold);
  else
    hipLaunchKernelGGL((fwd_bf16_qb2_kernel<128, NW, false, 0>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p, fold);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_qb2(FwdParams& p, hipStream_t s) {
  return launch_nw<Q2_NW>(p, s);
}

hipError_t launch_fwd_bf16_qb2_fold(FwdParams& p, const ChunkStateParams& fold, hipStream_t s) {
  if (p.n_splits < 2 || fold.k == nullptr) return hipErrorInvalidValue;  // the fold rides on a split pass only
  // extra workgroups only for passes without short tails (the tails take the units)
  const int rem = p.C % kQb2RowsPerTile;
  const bool tails = rem > 0 && rem <= kTailMaxRows;
  const int fold_blocks = tails ? 0 : fold.B * fold.H * fold.n_chunks * state::StateCfg<128>::ES;
  return launch_nw<Q2_NW>(p, s, fold, fold_blocks);
}

size_t fwd_split_bytes(int B, int H, int C, int d, int n_splits) {
  const int64_t tiles = (C + kQb2RowsPerTile - 1) / kQb2RowsPerTile;
  const int64_t n_part = (int64_t)B * H * tiles * n_splits;
  // bf16 rows, then {denominator, reference} in float32 per row
  return (size_t)(n_part * kQb2RowsPerTile * (2 * (int64_t)d + 2 * (int64_t)sizeof(float)));
}

hipError_t launch_fwd_state_combine(const FwdParams& p, const StateCombineParams& sc, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.H * p.C * (128 / 8);
  const int64_t fwd_blocks = (total + 255) / 256;
  const int64_t state_units = sc.G > 0 ? (int64_t)sc.BH * ((int64_t)sc.d * sc.d + sc.d) / 4 : 0;
  const int64_t blocks = fwd_blocks + (state_units + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_combine_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, p, sc, (int)fwd_blocks);
  return hipGetLastError();
}

hipError_t launch_fwd_combine(const FwdParams& p, hipStream_t s) {
  return launch_fwd_state_combine(p, StateCombineParams{}, s);
}

}  // namespace rha
