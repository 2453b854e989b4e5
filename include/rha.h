/*
 * librha: chunk-wise recurrent hybrid attention for video diffusion
 * transformers, for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Sources: "ReHyAt: Recurrent Hybrid Attention for Video
 * Diffusion Transformers" (abstract: softmax attention combined with linear
 * attention, evaluated chunk by chunk as a recurrence with constant memory);
 * "Long-Horizon Streaming Video Generation via Hybrid Attention with
 * Decoupled Distillation" (explainer page, section 2.A "Hybrid Attention":
 * softmax attention over a sliding window of recent frames computed in
 * FlashAttention-style blocks; frames leaving the window are folded online
 * into a fixed-size linear-attention state); "Transformers are RNNs" (listed
 * by the ReHyAt page among its foundations) for phi(x) = elu(x) + 1.
 *
 * Per (batch b, head h) with q, k, v in R^{L x d}, chunk length C (one latent
 * frame), N = L / C chunks, window w chunks counting the query's own chunk:
 *
 *   query i in chunk c = floor(i / C)
 *   window  W(i) = keys of chunks max(0, c-w+1) .. c      (empty if w == 0)
 *   history H(i) = keys of chunks 0 .. c-w                (empty if c < w)
 *   S_c = sum_{j in H} phi(k_j) v_j^T   (d x d),   z_c = sum_{j in H} phi(k_j)
 *   out_i = ( sum_{j in W} exp(q_i.k_j/sqrt d) v_j + phi(q_i)^T S_c )
 *         / ( sum_{j in W} exp(q_i.k_j/sqrt d)     + phi(q_i)^T z_c )
 *
 * Readings where the pages are silent: attention is chunk-causal (no chunk
 * after the query's own is visible; no token mask inside the window); w >= N
 * gives block-causal softmax attention; w == 0 is linear attention whose
 * state already holds the own chunk; phi acts on the raw q and k.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no device memory, keeps no pointer after a call returns and has
 *    no global mutable state except a thread-local error message.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; results are ready when the stream is.
 *  - Every argument is validated before anything is enqueued: a call that
 *    returns an error has had no side effect.  rha_last_error() then gives a
 *    human-readable reason.  NaN/Inf in the data are not detected; they
 *    propagate into the outputs.
 *  - Element layout of q, k, v and out: element (b, h, t, f) of a tensor with
 *    base pointer P is at P[b*stride_b + h*stride_h + t*stride_t + f] (feature
 *    stride 1).  For bf16 every base pointer and every stride*2 must be a
 *    multiple of 16 bytes; for f32 every base pointer and stride*4 likewise.
 *  - State tensors are always contiguous float32.
 */
#ifndef RHA_H
#define RHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RHA_OK = 0,
  RHA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad stride or alignment */
  RHA_ERR_UNSUPPORTED = 2, /* valid but not implemented (head_dim, dtype) */
  RHA_ERR_CURSOR = 3,      /* streaming cursor out of range */
  RHA_ERR_HIP = 4          /* HIP runtime error: no device, launch failure */
} rha_status;

typedef enum {
  RHA_F32 = 0, /* IEEE float32 storage; all arithmetic in float32 */
  RHA_BF16 = 1 /* bfloat16 storage; bf16 matrix-core products, float32 accumulation */
} rha_dtype;

typedef struct {
  int32_t batch;     /* B >= 0 */
  int32_t heads;     /* H >= 0 */
  int32_t head_dim;  /* d: 64 or 128 */
  int32_t chunk_len; /* C >= 1 tokens per chunk */
  int32_t n_chunks;  /* N >= 0 chunks per sequence, L = N*C (ignored by rha_stream_step) */
  int32_t window;    /* w >= 0 softmax window in chunks, the query's own chunk included */
  int32_t dtype;     /* rha_dtype of q, k, v, out and the KV cache */
  int32_t anchor_chunks; /* a >= 0 anchor (sink) chunks, see below; 0 = none */
  int64_t stride_b;  /* element strides of q, k, v and out (see above) */
  int64_t stride_h;
  int64_t stride_t;  /* >= head_dim */
} rha_problem;

/*
 * Anchor (sink) chunks.  Hybrid Forcing explainer section 1 (the attention-
 * sink workaround keeps the first frame attended).  With anchor_chunks = a
 * > 0, chunks 0 .. a-1 are in the softmax window of every query chunk c they
 * do not lie in the future of (chunks 0 .. min(a, c+1)-1), in addition to
 * chunks max(0, c-w+1) .. c, and the state excludes them: it sums chunks
 * a .. c-w.  rha_state_scan, rha_hybrid_fwd, rha_stream_step and
 * rha_hybrid_bwd honour it for RHA_BF16 with head_dim 128 (RHA_ERR_UNSUPPORTED
 * otherwise, and for the pruned and bidirectional calls, which need a = 0);
 * the anchor and window keys of a chunk may span at most 2048 tiles of 64
 * keys.
 */

/*
 * rha_state_scan -- the folded history each query chunk reads.
 *
 * ReHyAt abstract (chunk-wise recurrent form); Hybrid Forcing explainer
 * section 2.A (frames leaving the window are accumulated into the state).
 * For every (b, h) and chunk c in [0, N):
 *   S[b,h,c] = sum over chunks a <= j <= c - w of phi(K_j)^T V_j      (d x d)
 *   z[b,h,c] = sum over chunks a <= j <= c - w of sum_t phi(k_t)       (d)
 * and zero where c < w + a (a = anchor_chunks, usually 0).  Per chunk the contribution is one bf16 (f32 for
 * RHA_F32) matrix-core product with float32 accumulation; the prefix over
 * chunks is summed in float32 in chunk order, so results are bitwise
 * reproducible.
 *
 *   k, v : [B, H, L, d] with the problem's strides, dtype p->dtype (read)
 *   S    : [B, H, N, d, d] float32 contiguous (written)
 *   z    : [B, H, N, d]    float32 contiguous (written)
 *
 * rha_hybrid_fwd must be given the S, z produced with the same window.
 */
rha_status rha_state_scan(const rha_problem* p, const void* k, const void* v, float* S, float* z,
                          void* stream);

/*
 * rha_hybrid_fwd -- the hybrid attention output for a whole sequence.
 *
 * Hybrid Forcing explainer section 2.A (window attention in FlashAttention
 * blocks plus the linear state) with the shared normaliser written at the top
 * of this header.  One fused pass per query tile: the linear term
 * phi(Q)^T S_c, phi(Q).z_c seeds the running numerator and denominator at
 * reference maximum 0, then the window keys are streamed with an online
 * maximum.
 *
 *   q, k, v : [B, H, L, d] with the problem's strides, dtype p->dtype (read)
 *   S, z    : the output of rha_state_scan for the same problem (read)
 *   out     : [B, H, L, d] with the problem's strides, dtype p->dtype (written)
 *   lse     : NULL, or [B, H, L] float32 contiguous: ln of the denominator
 *
 * out must not overlap q, k, v, S or z.
 */
rha_status rha_hybrid_fwd(const rha_problem* p, const void* q, const void* k, const void* v,
                          const float* S, const float* z, void* out, float* lse, void* stream);

/*
 * rha_hybrid_fwd_sparse -- rha_hybrid_fwd with pruned blocks of the window.
 *
 * Hybrid Forcing explainer section 2.A (block-sparse sliding-window
 * attention: the window's attention is evaluated block by block and blocks
 * judged unimportant are pruned).  The page gives no importance criterion, so
 * the kept blocks are an input.  Blocks:
 *   query block i of chunk c : rows c*C + RHA_SPARSE_QTILE*i ..  (clipped to the chunk)
 *   key block j of its window: keys kbeg + RHA_SPARSE_KTILE*j .. (clipped to the window)
 * with kbeg = max(0, c-w+1)*C the window's first key.  A pruned block adds
 * nothing to the numerator or the denominator; the linear state is untouched.
 * A query left with no weight at all (every block pruned and c < w) gets
 * out = 0 and lse = -inf.
 *
 *   block_mask : uint8 [B, H, N, nqt, nkt] contiguous device memory (read);
 *                nonzero keeps the block.  nqt = ceil(C / RHA_SPARSE_QTILE),
 *                nkt = ceil(min(w, N) * C / RHA_SPARSE_KTILE); entries past a
 *                shorter window (chunks c < w-1) are ignored.
 *   other arguments as for rha_hybrid_fwd.
 * With every entry nonzero the result equals rha_hybrid_fwd's bitwise.
 *
 * Errors: RHA_ERR_UNSUPPORTED unless dtype is RHA_BF16 and head_dim is 128,
 * or when nkt exceeds RHA_SPARSE_MAX_KTILES.  With window 0 there is no
 * window to prune and the call is rha_hybrid_fwd (block_mask may be NULL).
 */
#define RHA_SPARSE_QTILE 256
#define RHA_SPARSE_KTILE 64
#define RHA_SPARSE_MAX_KTILES 2048
rha_status rha_hybrid_fwd_sparse(const rha_problem* p, const void* q, const void* k, const void* v,
                                 const float* S, const float* z, const uint8_t* block_mask, void* out,
                                 float* lse, void* stream);

/*
 * rha_hybrid_bwd -- gradients of rha_hybrid_fwd (the causal hybrid, with or
 * without anchor chunks; no pruning) for training or distilling through it.
 *
 * ReHyAt (abstract) and the Hybrid Forcing explainer (section 2.B) train
 * models that use the hybrid, so the gradients of its output with respect to
 * q, k and v are needed: with L = sum(dout * out), the exact derivatives of
 * the definition at the top of this header (through the softmax window, the
 * shared normaliser and the linear state, whose gradient flows back to every
 * earlier chunk that was folded in).  With p->anchor_chunks = a > 0, the
 * anchored definition (see rha_problem): anchor chunks are softmax keys of
 * every chunk not before them, so their gradients gather from all later
 * chunks, and they receive no state gradient.  Matrix products use bf16
 * operands and float32 accumulation.
 *
 *   q, k, v, S, z : as given to rha_hybrid_fwd, with the same anchor_chunks (read)
 *   out, lse      : rha_hybrid_fwd's output and lse for them (read; lse required)
 *   dout          : [B, H, L, d], the problem's strides and dtype (read)
 *   dq, dk, dv    : [B, H, L, d] float32 contiguous (written)
 *   workspace     : device scratch of rha_hybrid_bwd_workspace_size(p) bytes,
 *                   16-byte aligned, no initialisation needed
 *
 * Errors: RHA_ERR_UNSUPPORTED unless dtype is RHA_BF16 and head_dim is 128;
 * RHA_ERR_INVALID_ARG if the workspace is too small.
 */
size_t rha_hybrid_bwd_workspace_size(const rha_problem* p);
rha_status rha_hybrid_bwd(const rha_problem* p, const void* q, const void* k, const void* v,
                          const float* S, const float* z, const void* out, const float* lse,
                          const void* dout, float* dq, float* dk, float* dv, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * rha_hybrid_bwd_sparse -- gradients of rha_hybrid_fwd_sparse (the causal
 * hybrid with pruned blocks of the window).
 *
 * Hybrid Forcing explainer, sections 2.A (the block-sparse window) and 2.B
 * (the model is trained through it): with L = sum(dout * out), the exact
 * derivatives of the pruned definition, in which a pruned (query block, key
 * block) pair has weight zero; its pairs therefore carry no gradient, and the
 * linear state is as in rha_hybrid_bwd.  A query row left with no weight at
 * all (lse = -inf, out = 0) gets dq = 0 and sends no gradient to any key.
 * With every mask entry nonzero the result equals rha_hybrid_bwd's bitwise.
 *
 *   q, k, v, S, z, block_mask : as given to rha_hybrid_fwd_sparse (read)
 *   out, lse                  : its output and lse (read; lse required)
 *   dout, dq, dk, dv          : as for rha_hybrid_bwd
 *   workspace                 : device scratch of rha_hybrid_bwd_workspace_size(p)
 *                               bytes, 16-byte aligned, no initialisation needed
 *
 * Errors: as rha_hybrid_fwd_sparse (RHA_ERR_UNSUPPORTED unless dtype is
 * RHA_BF16, head_dim is 128, anchor_chunks is 0 and the window spans at most
 * RHA_SPARSE_MAX_KTILES key blocks); RHA_ERR_INVALID_ARG if the workspace is
 * too small.  With window 0 the call is rha_hybrid_bwd (block_mask may be NULL).
 */
rha_status rha_hybrid_bwd_sparse(const rha_problem* p, const void* q, const void* k, const void* v,
                                 const float* S, const float* z, const uint8_t* block_mask,
                                 const void* out, const float* lse, const void* dout, float* dq,
                                 float* dk, float* dv, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * rha_hybrid_bwd_bidir -- gradients of rha_hybrid_fwd_bidir, for training or
 * distilling the bidirectional models that the hybrid serves (ReHyAt,
 * abstract: the hybrid replaces the attention of video diffusion
 * transformers, which attend over the whole clip in both directions).
 *
 * With L = sum(dout * out) for out = rha_hybrid_fwd_bidir's output (the
 * definition below, at rha_state_scan_bidir): the exact derivatives through
 * the symmetric softmax window, the shared normaliser and both states.  The
 * state used by chunk c is S_past[c] + S_future[c], so its gradient reaches
 * the keys of chunk j through the past state when j <= c - w (w == 0:
 * j <= c) and through the future state when j >= c + max(w, 1).  Matrix
 * products use bf16 operands and float32 accumulation.
 *
 *   q, k, v                       : as given to rha_hybrid_fwd_bidir (read)
 *   S_past, z_past, S_future, z_future : rha_state_scan_bidir's states (read)
 *   out, lse                      : rha_hybrid_fwd_bidir's output and lse (read; lse required)
 *   dout                          : [B, H, L, d], the problem's strides and dtype (read)
 *   dq, dk, dv                    : [B, H, L, d] float32 contiguous (written)
 *   workspace                     : device scratch of rha_hybrid_bwd_bidir_workspace_size(p)
 *                                   bytes, 16-byte aligned, no initialisation needed
 *
 * Errors: RHA_ERR_UNSUPPORTED unless dtype is RHA_BF16, head_dim is 128 and
 * anchor_chunks is 0; RHA_ERR_INVALID_ARG if the workspace is too small.
 */
size_t rha_hybrid_bwd_bidir_workspace_size(const rha_problem* p);
rha_status rha_hybrid_bwd_bidir(const rha_problem* p, const void* q, const void* k, const void* v,
                                const float* S_past, const float* z_past, const float* S_future,
                                const float* z_future, const void* out, const float* lse,
                                const void* dout, float* dq, float* dk, float* dv, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Bidirectional hybrid -- rha_state_scan_bidir and rha_hybrid_fwd_bidir.
 *
 * ReHyAt (abstract): the hybrid takes the place of the softmax attention of
 * video diffusion transformers, which attend over the whole clip in both
 * directions.  Here the softmax window of chunk c is symmetric,
 *   chunks max(0, c-w+1) .. min(N-1, c+w-1)      (none if w == 0),
 * and every chunk outside it, before or after, is in the linear term with the
 * shared normaliser: S = S_past[c] + S_future[c], z = z_past[c] + z_future[c],
 *   S_past[c]   = sum over chunks j <= c - w          (w == 0: j <= c)
 *   S_future[c] = sum over chunks j >= c + max(w, 1)
 * of phi(K_j)^T V_j (z: of sum phi(k)).  A window covering every chunk is
 * dense unmasked softmax attention; w == 0 is non-causal linear attention.
 *
 *   S_past, S_future : [B, H, N, d, d] float32 contiguous
 *   z_past, z_future : [B, H, N, d]    float32 contiguous
 *   other arguments as for rha_state_scan / rha_hybrid_fwd (the scan writes
 *   the four state tensors, the forward pass reads them).
 *
 * Errors: RHA_ERR_UNSUPPORTED unless dtype is RHA_BF16 and head_dim is 128.
 */
rha_status rha_state_scan_bidir(const rha_problem* p, const void* k, const void* v, float* S_past,
                                float* z_past, float* S_future, float* z_future, void* stream);
rha_status rha_hybrid_fwd_bidir(const rha_problem* p, const void* q, const void* k, const void* v,
                                const float* S_past, const float* z_past, const float* S_future,
                                const float* z_future, void* out, float* lse, void* stream);

/*
 * Streaming cursor: the number of chunks committed so far, which is the
 * index of the chunk the next call processes.  Start at 0 with S, z zeroed.
 */
typedef struct {
  int64_t t;
} rha_stream_cursor;

/*
 * rha_stream_step -- one new chunk of an autoregressive (streaming) generator.
 *
 * Hybrid Forcing explainer section 1 (a sliding-window KV cache of recent
 * frames) and section 2.A (frames evicted from the window are folded online
 * into the linear state; the local window can then shrink, e.g. from 21 to 9
 * frames).  With t = cursor->t, window w >= 1 and a = p->anchor_chunks >= 0
 * anchor (attention-sink) chunks -- the explainer's section 1 describes
 * streaming generators that keep the first frames in attention for good:
 *   1. the new chunk's k, v are copied into cache slot t % w, and for t < a
 *      also into anchor slot w + t, which it keeps;
 *   2. the new chunk's queries attend, with exact softmax, to the cached
 *      chunks max(0, t-w+1) .. t and the anchor chunks 0 .. a-1 that have
 *      left the window, plus the state S, z (chunks a .. t-w), with the shared
 *      normaliser (rha_hybrid_fwd's anchored definition, chunk t);
 *   3. if commit != 0 and t >= w-1: chunk t-w+1 (slot (t+1) % w) leaves the
 *      window; unless it is an anchor (t-w+1 < a), phi(K)^T V and sum phi(k)
 *      of that slot are added into S, z; then cursor->t is incremented.
 * With commit == 0 nothing but the cache slot of chunk t changes, so the same
 * chunk can be re-run (e.g. once per denoising step) before committing it.
 * Outputs equal those of rha_hybrid_fwd over the concatenated sequence up to
 * float rounding (the key window is visited in another order).  Without a
 * workspace, S, z after each commit equal rha_state_scan's entry for chunk
 * t+1 bitwise; with one, up to float rounding (the fold sums token groups).
 * p->anchor_chunks applies to the stream from its first chunk on (a is part
 * of the stream's configuration, like w).
 * Either way a step is deterministic.
 *
 *   p->n_chunks is ignored; p's strides describe q_new, k_new, v_new, out
 *   q_new, k_new, v_new : [B, H, C, d] (read)
 *   k_cache, v_cache    : [B, H, w + a, C, d] contiguous, dtype p->dtype (read/written)
 *   S : [B, H, d, d] float32, z : [B, H, d] float32 (read; written on commit)
 *   out : [B, H, C, d] (written);  lse : NULL or [B, H, C] float32
 *   cursor : host memory, read and (on commit) updated at enqueue time
 *   workspace, workspace_bytes : NULL/0 or device scratch, see below
 *
 * Errors: RHA_ERR_CURSOR if cursor is NULL or cursor->t < 0.
 */
rha_status rha_stream_step(const rha_problem* p, const void* q_new, const void* k_new,
                           const void* v_new, void* k_cache, void* v_cache, float* S, float* z,
                           rha_stream_cursor* cursor, int32_t commit, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * rha_stream_workspace_size -- bytes of device workspace with which
 * rha_stream_step spreads one step over more of the GPU.
 *
 * One chunk has few query tiles, so the step splits the key window across
 * several workgroups per tile and merges their partial results (numerators,
 * denominators and reference maxima, in float32) in a second small kernel.
 * Likewise the fold of a committed chunk splits the chunk's tokens into
 * groups whose partial states are then added to S, z in group order.  The
 * size depends on p (batch, heads, chunk_len, head_dim, window, dtype) and on
 * the number of compute units of the current device; it is 0 when p would
 * not be split (enough tiles and heads already, or float32 problems).
 * Pass workspace = NULL, or workspace_bytes below this size, to run without
 * the split; results agree to rounding either way.  The workspace must be
 * 16-byte aligned device memory owned by the caller, not used by anything else
 * while the step runs; its contents need no initialisation.
 */
size_t rha_stream_workspace_size(const rha_problem* p);

/*
 * rha_stream_step_sparse -- rha_stream_step with pruned blocks of the window.
 *
 * Hybrid Forcing explainer, section 1 (the streaming generator's KV cache)
 * and section 2.A (its window attention is block-sparse: blocks judged
 * unimportant are pruned; the page gives no criterion, so the kept blocks are
 * an input, one mask per step).  The blocks follow the cache's own layout,
 * the order in which the step reads the window:
 *   query block i : rows RHA_SPARSE_QTILE*i .. of the new chunk (clipped)
 *   key block j   : keys RHA_SPARSE_KTILE*j .. of the window's chunks taken in
 *                   cache-slot order (chunk c sits in slot c % w; before the
 *                   ring is full the slots in use are 0 .. t)
 * so a key block may span two chunks.  A pruned block adds nothing to the
 * numerator or the denominator; the fold and the state are those of
 * rha_stream_step.  A query left with no weight at all (every block pruned
 * and no state yet) gets out = 0 and lse = -inf.  Until the ring turns
 * (t < w) slot order is the sequence order, and the step equals
 * rha_hybrid_fwd_sparse over the concatenated sequence, chunk t, with this
 * step's mask; with every entry nonzero it equals rha_stream_step.
 *
 *   block_mask : uint8 [B, H, ceil(C / RHA_SPARSE_QTILE), ceil(w * C / RHA_SPARSE_KTILE)]
 *                contiguous device memory (read); nonzero keeps the block;
 *                entries past the keys in use (t < w-1) are ignored.
 *   other arguments as for rha_stream_step, the workspace included (each
 *   split of the key window visits the kept blocks of its share).
 *
 * Errors: as rha_stream_step; RHA_ERR_UNSUPPORTED unless dtype is RHA_BF16,
 * head_dim is 128 and anchor_chunks is 0, or when the window spans more than
 * RHA_SPARSE_MAX_KTILES key blocks.
 */
rha_status rha_stream_step_sparse(const rha_problem* p, const void* q_new, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache, float* S,
                                  float* z, rha_stream_cursor* cursor, int32_t commit,
                                  const uint8_t* block_mask, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of device scratch that rha_stream_step_noalloc holds per GPU. */
#define RHA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

/*
 * rha_stream_step_noalloc -- rha_stream_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.
 *
 * The same step, arguments and results as rha_stream_step with its workspace
 * (the split key window and the split fold), but the workspace is the
 * library's own: a file-scope device array of RHA_NOALLOC_SCRATCH_BYTES (48
 * MiB) that every GPU the library runs on holds until the process ends.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Its address is looked up once per device, on the first call
 * with that device current.
 *
 * The scratch keeps the last call's contents; nothing in it needs clearing
 * (every byte a step reads it first writes).  Calls that overlap on one GPU
 * -- on two streams at once, or from two threads -- share that GPU's scratch
 * and race: serialise them (one stream, or one call in flight per GPU).
 *
 * Errors: as rha_stream_step; RHA_ERR_UNSUPPORTED if the step needs more
 * scratch than RHA_NOALLOC_SCRATCH_BYTES (rha_stream_workspace_size(p) tells
 * how much: about 41 MB for 12 heads of 1560-token chunks with a 9-chunk
 * window; the split gives each compute unit at most one workgroup, which on
 * a 256-CU MI355X bounds any problem's need near 43 MB), RHA_ERR_HIP if the
 * scratch's address cannot be obtained.
 */
rha_status rha_stream_step_noalloc(const rha_problem* p, const void* q_new, const void* k_new,
                                   const void* v_new, void* k_cache, void* v_cache, float* S, float* z,
                                   rha_stream_cursor* cursor, int32_t commit, void* out, float* lse,
                                   void* stream);

/* Static name of a status code. */
const char* rha_status_string(rha_status s);

/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char* rha_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int32_t rha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RHA_H */
