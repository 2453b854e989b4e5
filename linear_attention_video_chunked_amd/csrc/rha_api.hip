// C ABI of librha (declared in include/rha.h): argument validation, then
// kernel launches on the caller's stream.  Every check runs before anything
// is enqueued, so a call that fails has no side effect.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "rha.h"
#include "rha_launch.hpp"

namespace {

thread_local std::string g_last_error;

rha_status fail(rha_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

rha_status ok() {
  g_last_error.clear();
  return RHA_OK;
}

rha_status hip_fail(hipError_t e, const char* what) {
  return fail(RHA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}


int elem_bytes(const rha_problem* p) { return p->dtype == RHA_BF16 ? 2 : 4; }

// Checks shared by all calls.  `stream` selects the streaming rules
// (n_chunks ignored, window >= 1).
rha_status check_problem(const rha_problem* p, bool stream) {
  if (p == nullptr) return fail(RHA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 0 || p->heads < 0)
    return fail(RHA_ERR_INVALID_ARG, "batch (%d) and heads (%d) must be >= 0", p->batch, p->heads);
  if (p->dtype != RHA_F32 && p->dtype != RHA_BF16)
    return fail(RHA_ERR_INVALID_ARG, "dtype %d is not RHA_F32 or RHA_BF16", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(RHA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  if (p->chunk_len < 1) return fail(RHA_ERR_INVALID_ARG, "chunk_len %d must be >= 1", p->chunk_len);
  if (!stream && p->n_chunks < 0) return fail(RHA_ERR_INVALID_ARG, "n_chunks %d must be >= 0", p->n_chunks);
  if (p->window < 0) return fail(RHA_ERR_INVALID_ARG, "window %d must be >= 0", p->window);
  if (stream && p->window < 1) return fail(RHA_ERR_INVALID_ARG, "streaming needs window >= 1 (got %d)", p->window);
  if (p->anchor_chunks < 0) return fail(RHA_ERR_INVALID_ARG, "anchor_chunks %d must be >= 0", p->anchor_chunks);
  if (p->anchor_chunks > 0 && !stream) {
    if (p->dtype != RHA_BF16 || p->head_dim != 128)
      return fail(RHA_ERR_UNSUPPORTED, "anchor chunks need dtype RHA_BF16 and head_dim 128");
    // the anchor and window tiles of a query chunk are listed in LDS
    const int64_t a = p->anchor_chunks < p->n_chunks ? p->anchor_chunks : p->n_chunks;
    const int64_t wl = p->window < p->n_chunks ? p->window : p->n_chunks;
    const int64_t tiles = (a * p->chunk_len + 63) / 64 + (wl * p->chunk_len + 63) / 64;
    if (tiles > RHA_SPARSE_MAX_KTILES)
      return fail(RHA_ERR_UNSUPPORTED, "anchors and window span %lld key tiles (at most %d)", (long long)tiles,
                  RHA_SPARSE_MAX_KTILES);
  }
  if (p->stride_t < p->head_dim)
    return fail(RHA_ERR_INVALID_ARG, "stride_t %lld < head_dim %d", (long long)p->stride_t, p->head_dim);
  if (p->stride_h < 0 || p->stride_b < 0) return fail(RHA_ERR_INVALID_ARG, "strides must be >= 0");
  const int64_t eb = elem_bytes(p);
  if ((p->stride_t * eb) % 16 || (p->stride_h * eb) % 16 || (p->stride_b * eb) % 16)
    return fail(RHA_ERR_INVALID_ARG, "strides must be multiples of 16 bytes");
  // index arithmetic in the kernels keeps token and tile counts in 32 bits
  const int64_t nc = stream ? 1 : p->n_chunks;
  const int64_t L = nc * (int64_t)p->chunk_len;
  const int64_t bhn = (int64_t)p->batch * p->heads * nc;
  // (streaming: the window slots and the anchor slots of the cache)
  const int64_t win_keys = ((int64_t)(p->window < 1 ? 1 : p->window) + (stream ? p->anchor_chunks : 0)) * p->chunk_len;
  if (L > INT32_MAX / 2 || bhn * p->chunk_len > INT32_MAX || (int64_t)p->batch * p->heads > INT32_MAX / 2 ||
      (stream && win_keys > INT32_MAX / 2))
    return fail(RHA_ERR_INVALID_ARG, "problem too large for 32-bit tile indexing");
  // the forward kernels address one head's keys with 32-bit byte offsets
  // (buffer loads), reaching up to two 64-key tiles past the last key
  const int64_t head_keys = stream ? win_keys : L;
  if ((head_keys + 128) * p->stride_t * eb > INT32_MAX)
    return fail(RHA_ERR_INVALID_ARG, "one head's keys span more than 2 GiB (stride_t %lld)", (long long)p->stride_t);
  return RHA_OK;
}

bool empty(const rha_problem* p, bool stream) {
  return p->batch == 0 || p->heads == 0 || (!stream && p->n_chunks == 0);
}

rha_status need(const void* ptr, const char* name, bool data = true, int elem_align = 16) {
  if (ptr == nullptr) return fail(RHA_ERR_INVALID_ARG, "%s is NULL", name);
  if (data && (reinterpret_cast<uintptr_t>(ptr) % elem_align) != 0)
    return fail(RHA_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, elem_align);
  return RHA_OK;
}

#define RHA_TRY(expr)             \
  do {                            \
    rha_status _s = (expr);       \
    if (_s != RHA_OK) return _s;  \
  } while (0)

rha::ChunkStateParams state_params(const rha_problem* p, const void* k, const void* v, float* S, float* z) {
  rha::ChunkStateParams c{};
  c.k = k;
  c.v = v;
  c.S = S;
  c.z = z;
  c.kv_sb = p->stride_b;
  c.kv_sh = p->stride_h;
  c.kv_st = p->stride_t;
  c.B = p->batch;
  c.H = p->heads;
  c.C = p->chunk_len;
  return c;
}

hipError_t launch_chunk_state(const rha_problem* p, const rha::ChunkStateParams& c, hipStream_t s) {
  return p->dtype == RHA_BF16 ? rha::launch_chunk_state_bf16(c, p->head_dim, s)
                              : rha::launch_chunk_state_f32(c, p->head_dim, s);
}

hipError_t launch_fwd(const rha_problem* p, rha::FwdParams& f, hipStream_t s) {
  return p->dtype == RHA_BF16 ? rha::launch_fwd_bf16(f, p->head_dim, s) : rha::launch_fwd_f32(f, p->head_dim, s);
}

// Split of a stream step's key window: enough workgroups per query tile to
// give every compute unit one, at most 8, and at least 4 key tiles each.
int stream_splits(const rha_problem* p, int64_t n_keys) {
  if (p->dtype != RHA_BF16 || p->head_dim != 128) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 1;
  const int64_t tiles = (int64_t)p->batch * p->heads * ((p->chunk_len + rha::kQb2RowsPerTile - 1) / rha::kQb2RowsPerTile);
  int64_t splits = cus / (tiles > 0 ? tiles : 1);
  const int64_t key_tiles = (n_keys + 63) / 64;
  if (splits > key_tiles / 4) splits = key_tiles / 4;
  if (splits > rha::kMaxSplits) splits = rha::kMaxSplits;
  return splits < 2 ? 1 : (int)splits;
}

// Split of the streaming fold (bf16): the folded chunk's tokens in groups of
// whole 64-token tiles, enough groups for about one workgroup per compute
// unit (per `share` compute units).  Returns the number of groups (1: no
// split) and their length.
int fold_groups(const rha_problem* p, int* group_len, int share = 1) {
  *group_len = p->chunk_len;
  if (p->dtype != RHA_BF16) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 1;
  const int64_t units = (int64_t)p->batch * p->heads * (p->head_dim / 64);  // workgroups per group
  const int64_t ntiles = (p->chunk_len + 63) / 64;
  const int64_t wgs = (cus + share - 1) / share;
  int64_t g = (wgs + units - 1) / units;
  if (g > ntiles) g = ntiles;
  if (g < 2) return 1;
  const int64_t per = (ntiles + g - 1) / g;
  g = (ntiles + per - 1) / per;
  if (g < 2) return 1;
  *group_len = (int)(per * 64);
  return (int)g;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t fold_bytes(const rha_problem* p, int groups) {
  const int64_t d = p->head_dim;
  return (size_t)((int64_t)p->batch * p->heads * groups * (d * d + d) * (int64_t)sizeof(float));
}

}  // namespace

extern "C" {

rha_status rha_state_scan(const rha_problem* p, const void* k, const void* v, float* S, float* z, void* stream) {
  RHA_TRY(check_problem(p, false));
  if (empty(p, false)) return ok();
  RHA_TRY(need(k, "k"));
  RHA_TRY(need(v, "v"));
  RHA_TRY(need(S, "S"));
  RHA_TRY(need(z, "z"));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int N = p->n_chunks, w = p->window, d = p->head_dim;
  const int a = p->anchor_chunks < N ? p->anchor_chunks : N;  // anchors never enter the state
  const int nproc = N - w - a;  // chunks a .. N-1-w are folded into some later chunk's state
  if (nproc > 0) {
    rha::ChunkStateParams c = state_params(p, k, v, S, z);
    c.chunk0 = a;
    c.n_chunks = nproc;
    c.slot_offset = a + w;  // chunk j -> slot j + w
    c.accumulate = 0;
    c.s_bh = (int64_t)N * d * d;
    c.z_bh = (int64_t)N * d;
    c.tok_end = (int64_t)(N - w) * p->chunk_len;
    hipError_t e = launch_chunk_state(p, c, s);
    if (e != hipSuccess) return hip_fail(e, "chunk state launch");
  }
  rha::PrefixParams pp{S, z, p->batch * p->heads, N, a + w, d};
  hipError_t e = rha::launch_prefix(pp, s);
  if (e != hipSuccess) return hip_fail(e, "prefix launch");
  return ok();
}

rha_status rha_hybrid_fwd(const rha_problem* p, const void* q, const void* k, const void* v, const float* S,
                          const float* z, void* out, float* lse, void* stream) {
  RHA_TRY(check_problem(p, false));
  if (empty(p, false)) return ok();
  RHA_TRY(need(q, "q"));
  RHA_TRY(need(k, "k"));
  RHA_TRY(need(v, "v"));
  RHA_TRY(need(S, "S"));
  RHA_TRY(need(z, "z"));
  RHA_TRY(need(out, "out"));
  if (lse != nullptr) RHA_TRY(need(lse, "lse", true, 4));
  rha::FwdParams f{};
  f.q = q;
  f.k = k;
  f.v = v;
  f.out = out;
  f.lse = lse;
  f.S = S;
  f.z = z;
  f.q_sb = f.kv_sb = p->stride_b;
  f.q_sh = f.kv_sh = p->stride_h;
  f.q_st = f.kv_st = p->stride_t;
  f.B = p->batch;
  f.H = p->heads;
  f.C = p->chunk_len;
  f.w = p->window;
  f.n_qchunks = p->n_chunks;
  f.stream_mode = 0;
  f.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  f.anchors = p->anchor_chunks;
  hipError_t e = launch_fwd(p, f, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

rha_status rha_state_scan_bidir(const rha_problem* p, const void* k, const void* v, float* S_past, float* z_past,
                                float* S_future, float* z_future, void* stream) {
  RHA_TRY(check_problem(p, false));
  if (p->anchor_chunks > 0) return fail(RHA_ERR_UNSUPPORTED, "anchor chunks are not supported by this call");
  if (p->dtype != RHA_BF16 || p->head_dim != 128)
    return fail(RHA_ERR_UNSUPPORTED, "bidirectional problems need dtype RHA_BF16 and head_dim 128");
  if (empty(p, false)) return ok();
  RHA_TRY(need(k, "k"));
  RHA_TRY(need(v, "v"));
  RHA_TRY(need(S_past, "S_past"));
  RHA_TRY(need(z_past, "z_past"));
  RHA_TRY(need(S_future, "S_future"));
  RHA_TRY(need(z_future, "z_future"));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int N = p->n_chunks, w = p->window, d = p->head_dim;
  const int lag_f = w > 0 ? w : 1;  // the future part starts at chunk c + max(w, 1)
  if (w < N) {
    // every chunk's contribution, into past slot j + w and future slot j - lag_f
    rha::ChunkStateParams c = state_params(p, k, v, S_past, z_past);
    c.chunk0 = 0;
    c.n_chunks = N;
    c.slot_offset = w;
    c.accumulate = 0;
    c.s_bh = (int64_t)N * d * d;
    c.z_bh = (int64_t)N * d;
    c.tok_end = (int64_t)N * p->chunk_len;
    c.S2 = S_future;
    c.z2 = z_future;
    c.slot_offset2 = -lag_f;
    c.n_slots = N;
    hipError_t e = launch_chunk_state(p, c, s);
    if (e != hipSuccess) return hip_fail(e, "chunk state launch");
  }
  rha::PrefixParams pp{S_past, z_past, p->batch * p->heads, N, w, d, 0};
  hipError_t e = rha::launch_prefix(pp, s);
  if (e != hipSuccess) return hip_fail(e, "prefix launch");
  rha::PrefixParams ps{S_future, z_future, p->batch * p->heads, N, lag_f, d, 1};
  e = rha::launch_prefix(ps, s);
  if (e != hipSuccess) return hip_fail(e, "suffix launch");
  return ok();
}

rha_status rha_hybrid_fwd_bidir(const rha_problem* p, const void* q, const void* k, const void* v,
                                const float* S_past, const float* z_past, const float* S_future,
                                const float* z_future, void* out, float* lse, void* stream) {
  RHA_TRY(check_problem(p, false));
  if (p->anchor_chunks > 0) return fail(RHA_ERR_UNSUPPORTED, "anchor chunks are not supported by this call");
  if (p->dtype != RHA_BF16 || p->head_dim != 128)
    return fail(RHA_ERR_UNSUPPORTED, "bidirectional problems need dtype RHA_BF16 and head_dim 128");
  if (empty(p, false)) return ok();
  RHA_TRY(need(q, "q"));
  RHA_TRY(need(k, "k"));
  RHA_TRY(need(v, "v"));
  RHA_TRY(need(S_past, "S_past"));
  RHA_TRY(need(z_past, "z_past"));
  RHA_TRY(need(S_future, "S_future"));
  RHA_TRY(need(z_future, "z_future"));
  RHA_TRY(need(out, "out"));
  if (lse != nullptr) RHA_TRY(need(lse, "lse", true, 4));
  rha::FwdParams f{};
  f.q = q;
  f.k = k;
  f.v = v;
  f.out = out;
  f.lse = lse;
  f.S = S_past;
  f.z = z_past;
  f.q_sb = f.kv_sb = p->stride_b;
  f.q_sh = f.kv_sh = p->stride_h;
  f.q_st = f.kv_st = p->stride_t;
  f.B = p->batch;
  f.H = p->heads;
  f.C = p->chunk_len;
  f.w = p->window;
  f.n_qchunks = p->n_chunks;
  f.stream_mode = 0;
  f.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  f.bidir = 1;
  f.S2 = S_future;
  f.z2 = z_future;
  hipError_t e = launch_fwd(p, f, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

namespace {

// Bytes of the backward pass's workspace: per row delta, 1/D, -delta/D and
// lse log2(e); the per-chunk state gradients (twice for the bidirectional
// hybrid: past and future parts).
size_t bwd_workspace_bytes(const rha_problem* p, bool bidir) {
  const int64_t BH = (int64_t)p->batch * p->heads, L = (int64_t)p->n_chunks * p->chunk_len, d = p->head_dim;
  const size_t states = align256((size_t)(BH * p->n_chunks * (d * d + d) * 4));
  return align256((size_t)(4 * BH * L * 4)) + (bidir ? 2 : 1) * states;
}

rha_status hybrid_bwd(const rha_problem* p, const void* q, const void* k, const void* v, const float* S,
                      const float* z, const float* S2, const float* z2, const void* out, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                      void* stream, bool bidir, const uint8_t* block_mask = nullptr, int64_t nkt = 0) {
  RHA_TRY(check_problem(p, false));
  if (p->dtype != RHA_BF16 || p->head_dim != 128)
    return fail(RHA_ERR_UNSUPPORTED, "the backward pass needs dtype RHA_BF16 and head_dim 128");
  if (bidir && p->anchor_chunks > 0)
    return fail(RHA_ERR_UNSUPPORTED, "the bidirectional backward pass takes no anchor chunks");
  if (empty(p, false)) return ok();
  if (nkt > 0) RHA_TRY(need(block_mask, "block_mask", true, 1));
  RHA_TRY(need(q, "q"));
  RHA_TRY(need(k, "k"));
  RHA_TRY(need(v, "v"));
  RHA_TRY(need(S, bidir ? "S_past" : "S"));
  RHA_TRY(need(z, bidir ? "z_past" : "z"));
  if (bidir) {
    RHA_TRY(need(S2, "S_future"));
    RHA_TRY(need(z2, "z_future"));
  }
  RHA_TRY(need(out, "out"));
  RHA_TRY(need(lse, "lse", true, 4));
  RHA_TRY(need(dout, "dout"));
  RHA_TRY(need(dq, "dq"));
  RHA_TRY(need(dk, "dk"));
  RHA_TRY(need(dv, "dv"));
  RHA_TRY(need(workspace, "workspace"));
  const size_t need_bytes = bwd_workspace_bytes(p, bidir);
  if (workspace_bytes < need_bytes)
    return fail(RHA_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need_bytes);
  const int64_t BH = (int64_t)p->batch * p->heads, L = (int64_t)p->n_chunks * p->chunk_len;
  float* ws = static_cast<float*>(workspace);
  rha::BwdParams b{};
  b.q = q;
  b.k = k;
  b.v = v;
  b.out = out;
  b.dout = dout;
  b.lse = lse;
  b.S = S;
  b.z = z;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.delta = ws;
  b.rsc = ws + BH * L;
  b.zw = ws + 2 * BH * L;
  b.lse2 = ws + 3 * BH * L;
  const size_t states = align256((size_t)(BH * p->n_chunks * (128 * 128 + 128) * 4));
  char* st = static_cast<char*>(workspace) + align256((size_t)(4 * BH * L * 4));
  b.dS = reinterpret_cast<float*>(st);
  b.dz = b.dS + BH * p->n_chunks * 128 * 128;
  if (bidir) {
    b.bidir = 1;
    b.S2 = S2;
    b.z2 = z2;
    b.dS2 = reinterpret_cast<float*>(st + states);
    b.dz2 = b.dS2 + BH * p->n_chunks * 128 * 128;
  }
  b.sb = p->stride_b;
  b.sh = p->stride_h;
  b.st = p->stride_t;
  b.B = p->batch;
  b.H = p->heads;
  b.C = p->chunk_len;
  b.N = p->n_chunks;
  b.w = p->window;
  b.anchors = p->anchor_chunks;
  if (nkt > 0) {
    b.kmask = block_mask;
    b.mask_qtiles = (p->chunk_len + RHA_SPARSE_QTILE - 1) / RHA_SPARSE_QTILE;
    b.nkt = (int)nkt;
  }
  b.scale = (float)(1.0 / std::sqrt((double)p->head_dim));
  b.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  hipError_t e = rha::launch_bwd_bf16(b, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

}  // namespace

size_t rha_hybrid_bwd_workspace_size(const rha_problem* p) {
  if (p == nullptr || check_problem(p, false) != RHA_OK) return 0;
  return bwd_workspace_bytes(p, false);
}

rha_status rha_hybrid_bwd(const rha_problem* p, const void* q, const void* k, const void* v, const float* S,
                          const float* z, const void* out, const float* lse, const void* dout, float* dq, float* dk,
                          float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return hybrid_bwd(p, q, k, v, S, z, nullptr, nullptr, out, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                    stream, false);
}

rha_status rha_hybrid_bwd_sparse(const rha_problem* p, const void* q, const void* k, const void* v, const float* S,
                                 const float* z, const uint8_t* block_mask, const void* out, const float* lse,
                                 const void* dout, float* dq, float* dk, float* dv, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  RHA_TRY(check_problem(p, false));
  if (p->anchor_chunks > 0) return fail(RHA_ERR_UNSUPPORTED, "anchor chunks are not supported by this call");
  int64_t nkt = 0;  // window 0: nothing to prune, the plain backward pass
  if (p->window > 0) {
    const int64_t wl = p->window < p->n_chunks ? p->window : p->n_chunks;
    nkt = (wl * p->chunk_len + RHA_SPARSE_KTILE - 1) / RHA_SPARSE_KTILE;
    if (nkt > RHA_SPARSE_MAX_KTILES)
      return fail(RHA_ERR_UNSUPPORTED, "window of %lld key blocks exceeds %d", (long long)nkt, RHA_SPARSE_MAX_KTILES);
  }
  return hybrid_bwd(p, q, k, v, S, z, nullptr, nullptr, out, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                    stream, false, block_mask, nkt);
}

size_t rha_hybrid_bwd_bidir_workspace_size(const rha_problem* p) {
  if (p == nullptr || check_problem(p, false) != RHA_OK) return 0;
  return bwd_workspace_bytes(p, true);
}

rha_status rha_hybrid_bwd_bidir(const rha_problem* p, const void* q, const void* k, const void* v,
                                const float* S_past, const float* z_past, const float* S_future,
                                const float* z_future, const void* out, const float* lse, const void* dout, float* dq,
                                float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return hybrid_bwd(p, q, k, v, S_past, z_past, S_future, z_future, out, lse, dout, dq, dk, dv, workspace,
                    workspace_bytes, stream, true);
}

static_assert(RHA_SPARSE_QTILE == rha::kQb2RowsPerTile && RHA_SPARSE_KTILE == 64 &&
                  RHA_SPARSE_MAX_KTILES == rha::kSparseMaxKeyTiles,
              "block sizes of the pruned window are the d = 128 kernel's tiles");

rha_status rha_hybrid_fwd_sparse(const rha_problem* p, const void* q, const void* k, const void* v, const float* S,
                                 const float* z, const uint8_t* block_mask, void* out, float* lse, void* stream) {
  RHA_TRY(check_problem(p, false));
  if (p->anchor_chunks > 0) return fail(RHA_ERR_UNSUPPORTED, "anchor chunks are not supported by this call");
  if (p->dtype != RHA_BF16 || p->head_dim != 128)
    return fail(RHA_ERR_UNSUPPORTED, "pruned windows need dtype RHA_BF16 and head_dim 128");
  if (p->window == 0) return rha_hybrid_fwd(p, q, k, v, S, z, out, lse, stream);
  const int64_t wl = p->window < p->n_chunks ? p->window : p->n_chunks;
  const int64_t nkt = (wl * p->chunk_len + RHA_SPARSE_KTILE - 1) / RHA_SPARSE_KTILE;
  if (nkt > RHA_SPARSE_MAX_KTILES)
    return fail(RHA_ERR_UNSUPPORTED, "window of %lld key blocks exceeds %d", (long long)nkt, RHA_SPARSE_MAX_KTILES);
  if (empty(p, false)) return ok();
  RHA_TRY(need(q, "q"));
  RHA_TRY(need(k, "k"));
  RHA_TRY(need(v, "v"));
  RHA_TRY(need(S, "S"));
  RHA_TRY(need(z, "z"));
  RHA_TRY(need(block_mask, "block_mask", true, 1));
  RHA_TRY(need(out, "out"));
  if (lse != nullptr) RHA_TRY(need(lse, "lse", true, 4));
  rha::FwdParams f{};
  f.q = q;
  f.k = k;
  f.v = v;
  f.out = out;
  f.lse = lse;
  f.S = S;
  f.z = z;
  f.q_sb = f.kv_sb = p->stride_b;
  f.q_sh = f.kv_sh = p->stride_h;
  f.q_st = f.kv_st = p->stride_t;
  f.B = p->batch;
  f.H = p->heads;
  f.C = p->chunk_len;
  f.w = p->window;
  f.n_qchunks = p->n_chunks;
  f.stream_mode = 0;
  f.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  f.kmask = block_mask;
  f.nkt = (int)nkt;
  hipError_t e = launch_fwd(p, f, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

size_t rha_stream_workspace_size(const rha_problem* p) {
  if (p == nullptr || check_problem(p, true) != RHA_OK || empty(p, true)) return 0;
  // the split window's partial results, then the split fold's partial states
  const int splits = stream_splits(p, ((int64_t)p->window + p->anchor_chunks) * p->chunk_len);
  int glen = 0;
  const int groups = fold_groups(p, &glen);
  size_t bytes = splits < 2 ? 0 : align256(rha::fwd_split_bytes(p->batch, p->heads, p->chunk_len, p->head_dim, splits));
  if (groups > 1) bytes += align256(fold_bytes(p, groups));
  return bytes;
}

namespace {

// The streaming step; block_mask (pruned steps, bf16 d = 128 without anchors)
// is [B, H, ceil(C/256), ceil(w*C/64)] over the window's keys in slot order.
rha_status stream_step(const rha_problem* p, const void* q_new, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, float* S, float* z, rha_stream_cursor* cursor, int32_t commit,
                       const uint8_t* block_mask, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
  RHA_TRY(check_problem(p, true));
  if (cursor == nullptr) return fail(RHA_ERR_CURSOR, "cursor is NULL");
  if (cursor->t < 0) return fail(RHA_ERR_CURSOR, "cursor->t = %lld < 0", (long long)cursor->t);
  if (empty(p, true)) {
    if (commit) cursor->t += 1;
    return ok();
  }
  RHA_TRY(need(q_new, "q_new"));
  RHA_TRY(need(k_new, "k_new"));
  RHA_TRY(need(v_new, "v_new"));
  RHA_TRY(need(k_cache, "k_cache"));
  RHA_TRY(need(v_cache, "v_cache"));
  RHA_TRY(need(S, "S"));
  RHA_TRY(need(z, "z"));
  RHA_TRY(need(out, "out"));
  if (lse != nullptr) RHA_TRY(need(lse, "lse", true, 4));
  if (workspace != nullptr) RHA_TRY(need(workspace, "workspace"));

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t t = cursor->t;
  const int w = p->window, C = p->chunk_len, d = p->head_dim;
  const int a = p->anchor_chunks;  // anchor (sink) chunks: cache slots w .. w+a-1
  const int slot = (int)(t % w);
  const int64_t BH = (int64_t)p->batch * p->heads;
  const int64_t slots = (int64_t)w + a;  // cache slots per head
  hipError_t e;

  // The plan.  The window's key range is split over several workgroups per
  // query tile when a workspace allows (partial results, then a merge), and
  // the fold of a committed chunk is split into token groups (partial states,
  // then added in order).  Workspace: split-window partials first, then the
  // fold's partial states, each 256-byte aligned.
  // Keys: the window slots in use, then the anchor slots of the anchors that
  // have left the window (chunk j < a sits in slot w + j) -- one contiguous
  // row range of the cache, since anchors leave only once the window is full.
  // The chunk leaving the window at a commit is folded unless it is an anchor.
  const int64_t in_window = t + 1 < w ? t + 1 : w;
  const int64_t left = t - w + 1;  // chunks 0 .. left-1 have left the window
  const int64_t n_anc = left > 0 ? (left < a ? left : a) : 0;
  const int n_keys = (int)((in_window + n_anc) * C);
  const bool fold = commit && left >= 0 && left >= a;
  const int splits = workspace != nullptr ? stream_splits(p, n_keys) : 1;
  const size_t fwd_part = splits > 1 ? align256(rha::fwd_split_bytes(p->batch, p->heads, C, d, splits)) : 0;
  const bool split_fwd = splits > 1 && workspace_bytes >= fwd_part;
  // beside a split attention the fold takes the compute units the attention
  // leaves idle (about one in four), else about all of them
  int glen = C;
  const int groups = (workspace != nullptr && fold) ? fold_groups(p, &glen, split_fwd ? 4 : 1) : 1;
  const size_t fold_part = groups > 1 ? align256(fold_bytes(p, groups)) : 0;
  const bool split_fold = groups > 1 && workspace_bytes >= (split_fwd ? fwd_part : 0) + fold_part;
  float* fold_ws = split_fold ? reinterpret_cast<float*>(static_cast<char*>(workspace) + (split_fwd ? fwd_part : 0))
                              : nullptr;

  // 1. the new chunk's keys and values into its cache slot (t % w).  A split
  // fold's partial states (the chunk leaving the window) are computed by extra
  // workgroups of the split attention launch (step 2), on the compute units
  // the attention leaves idle; without a split attention, by this launch.
  const bool fold_in_fwd = split_fold && split_fwd && p->dtype == RHA_BF16 && d == 128;
  rha::CopyParams cp{};
  cp.sb = p->stride_b;
  cp.sh = p->stride_h;
  cp.st = p->stride_t;
  cp.B = p->batch;
  cp.H = p->heads;
  cp.C = C;
  cp.d = d;
  cp.w = (int)slots;
  cp.slot = slot;
  cp.elem_bytes = elem_bytes(p);
  cp.src = k_new;
  cp.dst = k_cache;
  cp.src2 = v_new;
  cp.dst2 = v_cache;
  rha::ChunkStateParams fold_c{};
  if (split_fold) {
    // the chunk leaving the window (t-w+1) sits in slot (t+1) % w, which the
    // copy does not touch -- except for w = 1, where it is the new chunk
    // itself, read from k_new / v_new
    rha::ChunkStateParams c{};
    if (w > 1) {
      const int64_t slot_off = (int64_t)((t + 1) % w) * C * d * elem_bytes(p);
      c.k = static_cast<const char*>(k_cache) + slot_off;
      c.v = static_cast<const char*>(v_cache) + slot_off;
      c.kv_sb = (int64_t)p->heads * slots * C * d;
      c.kv_sh = slots * C * d;
      c.kv_st = d;
    } else {
      c.k = k_new;
      c.v = v_new;
      c.kv_sb = p->stride_b;
      c.kv_sh = p->stride_h;
      c.kv_st = p->stride_t;
    }
    c.B = p->batch;
    c.H = p->heads;
    c.S = fold_ws;
    c.z = fold_ws + BH * groups * d * d;
    c.C = glen;
    c.chunk0 = 0;
    c.n_chunks = groups;
    c.slot_offset = 0;
    c.accumulate = 0;
    c.s_bh = (int64_t)groups * d * d;
    c.z_bh = (int64_t)groups * d;
    c.tok_end = C;
    fold_c = c;
    if (!fold_in_fwd) {
      c.copy = cp;
      c.copy_blocks_per_bh = (int)(((int64_t)C * (d * cp.elem_bytes / 16) + 255) / 256);
      e = launch_chunk_state(p, c, s);
      if (e != hipSuccess) return hip_fail(e, "cache copy and fold launch");
    }
  }
  if (!split_fold || fold_in_fwd) {
    e = rha::launch_copy_chunk(cp, s);
    if (e != hipSuccess) return hip_fail(e, "cache copy launch");
  }
  if (t < a) {  // an anchor chunk: also into its own slot, which it keeps for good
    rha::CopyParams ca = cp;
    ca.slot = (int)(w + t);
    e = rha::launch_copy_chunk(ca, s);
    if (e != hipSuccess) return hip_fail(e, "anchor copy launch");
  }

  // 2. attention of the new chunk: cached window (chunks max(0,t-w+1)..t) + state
  rha::FwdParams f{};
  f.q = q_new;
  f.k = k_cache;
  f.v = v_cache;
  f.out = out;
  f.lse = lse;
  f.S = S;
  f.z = z;
  f.q_sb = p->stride_b;
  f.q_sh = p->stride_h;
  f.q_st = p->stride_t;
  f.kv_sb = (int64_t)p->heads * slots * C * d;
  f.kv_sh = slots * C * d;
  f.kv_st = d;
  f.B = p->batch;
  f.H = p->heads;
  f.C = C;
  f.w = w;
  f.n_qchunks = 1;
  f.stream_mode = 1;
  f.n_keys = n_keys;
  f.has_state = left > a ? 1 : 0;  // chunks a .. t-w are in the state
  f.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  f.n_splits = split_fwd ? splits : 1;
  f.part = split_fwd ? static_cast<float*>(workspace) : nullptr;
  if (block_mask != nullptr) {
    f.kmask = block_mask;
    f.nkt = (int)(((int64_t)w * C + RHA_SPARSE_KTILE - 1) / RHA_SPARSE_KTILE);
  }
  e = fold_in_fwd ? rha::launch_fwd_bf16_qb2_fold(f, fold_c, s) : launch_fwd(p, f, s);
  if (e != hipSuccess) return hip_fail(e, "forward launch");

  // 3. merges (after the pass has read S, z), then the unsplit fold
  rha::StateCombineParams sc{};
  if (split_fold) sc = rha::StateCombineParams{S, z, fold_ws, (int)BH, groups, d};
  if (split_fwd) {
    e = rha::launch_fwd_state_combine(f, sc, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  } else if (split_fold) {
    e = rha::launch_state_combine(sc, s);
    if (e != hipSuccess) return hip_fail(e, "fold merge launch");
  }
  if (commit) {
    if (fold && !split_fold) {
      const int out_slot = (int)((t + 1) % w);
      rha::ChunkStateParams c{};
      c.k = k_cache;
      c.v = v_cache;
      c.S = S;
      c.z = z;
      c.kv_sb = f.kv_sb;
      c.kv_sh = f.kv_sh;
      c.kv_st = d;
      c.B = p->batch;
      c.H = p->heads;
      c.C = C;
      c.chunk0 = out_slot;
      c.n_chunks = 1;
      c.slot_offset = 0;
      c.accumulate = 1;
      c.s_bh = (int64_t)d * d;
      c.z_bh = d;
      c.tok_end = (int64_t)(out_slot + 1) * C;
      e = launch_chunk_state(p, c, s);
      if (e != hipSuccess) return hip_fail(e, "fold launch");
    }
    cursor->t = t + 1;
  }
  return ok();
}

}  // namespace

rha_status rha_stream_step(const rha_problem* p, const void* q_new, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, float* S, float* z, rha_stream_cursor* cursor,
                           int32_t commit, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return stream_step(p, q_new, k_new, v_new, k_cache, v_cache, S, z, cursor, commit, nullptr, out, lse, workspace,
                     workspace_bytes, stream);
}

rha_status rha_stream_step_sparse(const rha_problem* p, const void* q_new, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, float* S, float* z, rha_stream_cursor* cursor,
                                  int32_t commit, const uint8_t* block_mask, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  RHA_TRY(check_problem(p, true));
  if (p->anchor_chunks > 0) return fail(RHA_ERR_UNSUPPORTED, "anchor chunks are not supported by this call");
  if (p->dtype != RHA_BF16 || p->head_dim != 128)
    return fail(RHA_ERR_UNSUPPORTED, "pruned windows need dtype RHA_BF16 and head_dim 128");
  const int64_t nkt = ((int64_t)p->window * p->chunk_len + RHA_SPARSE_KTILE - 1) / RHA_SPARSE_KTILE;
  if (nkt > RHA_SPARSE_MAX_KTILES)
    return fail(RHA_ERR_UNSUPPORTED, "window of %lld key blocks exceeds %d", (long long)nkt, RHA_SPARSE_MAX_KTILES);
  if (!empty(p, true)) RHA_TRY(need(block_mask, "block_mask", true, 1));
  return stream_step(p, q_new, k_new, v_new, k_cache, v_cache, S, z, cursor, commit, block_mask, out, lse, workspace,
                     workspace_bytes, stream);
}

// ---- the step without allocation: its workspace in a file-scope device
// array (one copy per GPU), whose device address is looked up once per device
// with that device current.  In host code `scratch` only names the symbol;
// kernels and copies get the looked-up address.
static __device__ __align__(256) unsigned char scratch[RHA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

rha_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RHA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(RHA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RHA_OK;
}
}  // namespace

rha_status rha_stream_step_noalloc(const rha_problem* p, const void* q_new, const void* k_new, const void* v_new,
                                   void* k_cache, void* v_cache, float* S, float* z, rha_stream_cursor* cursor,
                                   int32_t commit, void* out, float* lse, void* stream) {
  RHA_TRY(check_problem(p, true));
  const size_t need = rha_stream_workspace_size(p);
  if (need > RHA_NOALLOC_SCRATCH_BYTES)
    return fail(RHA_ERR_UNSUPPORTED, "this step needs %zu bytes of scratch, the no-allocation step holds %zu",
                need, (size_t)RHA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && !empty(p, true)) RHA_TRY(scratch_address(&ws));
  return rha_stream_step(p, q_new, k_new, v_new, k_cache, v_cache, S, z, cursor, commit, out, lse, ws, need, stream);
}

const char* rha_status_string(rha_status st) {
  switch (st) {
    case RHA_OK: return "RHA_OK";
    case RHA_ERR_INVALID_ARG: return "RHA_ERR_INVALID_ARG";
    case RHA_ERR_UNSUPPORTED: return "RHA_ERR_UNSUPPORTED";
    case RHA_ERR_CURSOR: return "RHA_ERR_CURSOR";
    case RHA_ERR_HIP: return "RHA_ERR_HIP";
  }
  return "RHA_ERR_UNKNOWN";
}

const char* rha_last_error(void) { return g_last_error.c_str(); }

int32_t rha_version(void) { return 100; }  // 0.1.0

}  // extern "C"
