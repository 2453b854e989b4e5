// Kernel parameter blocks and launchers (host side), shared by the C ABI
// (rha_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rha {

// One fused hybrid-attention pass over query tiles.  Two key sources:
//   seq mode    (stream_mode == 0): keys are the query sequence itself; query
//               chunk c reads keys [max(0,c-w+1)*C, (c+1)*C) and state slot
//               S[bh, c] (present when w == 0 or c >= w).
//   stream mode (stream_mode == 1): one query chunk (n_qchunks == 1); keys are
//               rows [0, n_keys) of a contiguous cache [bh][w*C][d]; state
//               S[bh] present when has_state != 0.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const float* S;
  const float* z;
  int64_t q_sb, q_sh, q_st;   // q and out strides (elements)
  int64_t kv_sb, kv_sh, kv_st;  // k and v strides (elements)
  int B, H, C, w;
  int n_qchunks;      // query chunks per (b, h)
  int tiles_per_chunk;  // set by the launcher
  int total_tiles;      // set by the launcher
  int stream_mode;
  int n_keys;         // stream mode
  int has_state;      // stream mode
  float scale_log2;   // log2(e) / sqrt(d)
  // Split of the key range (stream mode, head_dim 128 bf16 only): with
  // n_splits > 1 every query tile is processed by n_splits workgroups, each
  // over its share of the key tiles (the first one also takes the state, and
  // so a little less of them), and the partial results go to `part` instead
  // of out:
  //   ((bf16*)part)[(pidx * BM + row) * d + col]      row normalised by its
  //                                                 own denominator (bf16)
  //   then float32 {denominator, reference} at index (pidx * BM + row) * 2
  //   from byte n_part * BM * d * 2 on
  // with pidx = (bh * tiles_per_chunk + tile) * n_splits + split and n_part the
  // number of pidx values.  launch_fwd_combine merges them into out and lse.
  int n_splits;
  float* part;
  // Pruned key tiles (seq mode, head_dim 128 bf16 only): with kmask set,
  // query tile i of chunk c of head bh visits only key tile j of its window
  // (keys kbeg + 64 j ..) where kmask[((bh * n_qchunks + c) * mask_qtiles
  // + i) * nkt + j] != 0, mask_qtiles = ceil(C / 256) (set by the launcher).
  const unsigned char* kmask;
  int nkt;
  int mask_qtiles;
  // Rows of a short chunk tail (set by the launcher): with tail_rows > 0 the
  // last tile of every chunk (tile tiles_per_chunk - 1, rows C - tail_rows ..
  // C - 1) runs the tail pass instead of a full tile.
  int tail_rows;
  // Bidirectional (seq mode, head_dim 128 bf16 only): the window of chunk c is
  // chunks max(0, c-w+1) .. min(N-1, c+w-1), and the linear term adds the
  // future state S2[bh, c], z2[bh, c] (chunks from c + max(w, 1) on) to the
  // past state S, z.
  int bidir;
  const float* S2;
  const float* z2;
  // Anchor chunks (seq mode, head_dim 128 bf16 only): chunks 0 .. anchors-1
  // are in the softmax window of every later (or the same) query chunk, and
  // the state slots exclude them.
  int anchors;
};

// Most key tiles per window of a pruned pass (the kept-tile list lives in LDS).
constexpr int kSparseMaxKeyTiles = 2048;
// most workgroups a streaming step splits one query tile's key window over
constexpr int kMaxSplits = 8;
// the pruned backward pass's key-gradient kernel lists at most this many
// 32-row query blocks per workgroup (beyond it, it visits every block)
constexpr int kMaxListedQBlocks = 2048;

// Copy one chunk [B,H,C,d] (strided) into cache slot `slot` of [B,H,w,C,d].
struct CopyParams {
  const void* src;
  void* dst;
  const void* src2;  // optional second chunk (same shape and strides) into dst2
  void* dst2;
  int64_t sb, sh, st;
  int B, H, C, d, w, slot;
  int elem_bytes;
};

// S[bh] += sum over g of part[bh][g] (g = 0 .. G-1 in order), likewise z:
// part holds B*H*G slots of d*d floats, then B*H*G slots of d floats.
struct StateCombineParams {
  float* S;
  float* z;
  const float* part;
  int BH, G, d;
};

// Per-chunk state contribution phi(K_c)^T V_c, sum_t phi(k_t) for a list of
// chunks, written to (or, with accumulate, added into) float32 state slots.
//   chunk index j in [0, n_chunks) of head bh reads tokens
//   [ (chunk0 + j) * C, +C ) of k, v, cut at token tok_end (tokens at or
//   past it count as absent); it writes slot (j + slot_offset) of S[bh] (slot
//   stride d*d, head stride s_bh) and z[bh] (slot stride d, head stride z_bh).
struct ChunkStateParams {
  const void* k;
  const void* v;
  float* S;
  float* z;
  int64_t kv_sb, kv_sh, kv_st;
  int64_t s_bh, z_bh;
  int B, H, C;
  int chunk0;
  int n_chunks;
  int slot_offset;
  int accumulate;
  int64_t tok_end;  // (chunk0 + n_chunks) * C for whole chunks
  // Optional second destination (S2, z2: same strides as S, z), written at
  // slot j + slot_offset2.  With n_slots > 0, a destination slot outside
  // [0, n_slots) is skipped (chunks whose contribution one side does not use).
  float* S2;
  float* z2;
  int slot_offset2;
  int n_slots;
  // Optional cache copy run by extra workgroups of the same launch (copy.src
  // set): copy_blocks_per_bh workgroups of 256 threads per (tensor, head).
  CopyParams copy;
  int copy_blocks_per_bh;
  // Optional per-token factors (the backward pass's state gradient): v rows
  // are multiplied by vscale[bh * scale_bh + token] before rounding, and z
  // sums phi(k_t) * zweight[bh * scale_bh + token] (token: index in the head).
  const float* vscale;
  const float* zweight;
  int64_t scale_bh;
};

// In-place inclusive prefix over the state slots of every head:
//   slot c < w        -> 0
//   slot c >= w       -> sum of the per-chunk contributions stored in slots w..c
// With reverse, the same with slot c read as slot N-1-c (a suffix sum).
struct PrefixParams {
  float* S;
  float* z;
  int BH, N, w, d;
  int reverse;
};

// Backward pass of the causal hybrid (head_dim 128, bf16 inputs): gradients
// of sum(dout * out) with respect to q, k, v, in float32 [B,H,L,d]
// (contiguous).  delta, rsc, zw: float32 [B,H,L] scratch (dout . out,
// exp(-lse), -delta * exp(-lse)); dS, dz: float32 [B,H,N,d,d] / [B,H,N,d]
// scratch for the state gradients.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const float* S;
  const float* z;
  float* dq;
  float* dk;
  float* dv;
  float* delta;
  float* rsc;
  float* zw;
  float* lse2;  // lse * log2(e) per row
  // bidirectional hybrid (bidir != 0): S, z hold the past states and S2, z2
  // the future ones; dS, dz receive the past part of the state gradients
  // (suffix sums with lag w) and dS2, dz2 the future part (prefix sums with
  // lag max(w, 1)); the window is symmetric
  const float* S2;
  const float* z2;
  float* dS2;
  float* dz2;
  int bidir;
  // anchor chunks (causal only): chunks 0 .. anchors-1 are softmax keys of
  // every chunk not before them and are in no state
  int anchors;
  // pruned window (causal, no anchors): kmask[B, H, N, mask_qtiles, nkt] as
  // for the pruned forward pass; NULL for none
  const unsigned char* kmask;
  int mask_qtiles, nkt;
  float* dS;
  float* dz;
  int64_t sb, sh, st;  // element strides of q, k, v, out, dout
  int B, H, C, N, w;
  float scale_log2;  // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
};
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s);

// The forward launchers fill in tiles_per_chunk and total_tiles (they depend
// on the kernel's tile height) before launching.
hipError_t launch_fwd_bf16(FwdParams& p, int d, hipStream_t s);
// head_dim 128 with 64 query rows per wave (the default for d = 128)
hipError_t launch_fwd_bf16_qb2(FwdParams& p, hipStream_t s);
// The same as a split pass (p.n_splits > 1, stream mode) whose extra
// workgroups compute the state contributions `fold` (bf16, head_dim 128,
// accumulate == 0, no cache copy, no per-token factors): the streaming fold,
// beside the attention on the compute units it leaves idle.
hipError_t launch_fwd_bf16_qb2_fold(FwdParams& p, const ChunkStateParams& fold, hipStream_t s);
// head_dim 128, window of 0 chunks (sequence mode, causal, no mask or anchors)
hipError_t launch_fwd_linear_bf16(const FwdParams& p, hipStream_t s);
// Query rows per workgroup of the d = 128 bf16 kernel (the partial-result tile).
constexpr int kQb2RowsPerTile = 256;
// Bytes of partial results for a split stream pass (see FwdParams::part).
size_t fwd_split_bytes(int B, int H, int C, int d, int n_splits);
// Merge the partial results of a split pass into out (and lse).
hipError_t launch_fwd_combine(const FwdParams& p, hipStream_t s);
// The same merge with a state merge (sc.G > 0) run by extra workgroups.
hipError_t launch_fwd_state_combine(const FwdParams& p, const StateCombineParams& sc, hipStream_t s);
hipError_t launch_fwd_f32(FwdParams& p, int d, hipStream_t s);
hipError_t launch_chunk_state_bf16(const ChunkStateParams& p, int d, hipStream_t s);
hipError_t launch_chunk_state_f32(const ChunkStateParams& p, int d, hipStream_t s);
hipError_t launch_prefix(const PrefixParams& p, hipStream_t s);
hipError_t launch_copy_chunk(const CopyParams& p, hipStream_t s);
hipError_t launch_state_combine(const StateCombineParams& p, hipStream_t s);

}  // namespace rha
