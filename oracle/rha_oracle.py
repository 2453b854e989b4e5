"""Plain, slow, float64 oracle of chunk-wise recurrent hybrid attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the library
path may import or call this module.

Sources (page title, then the part of the page):

* "ReHyAt: Recurrent Hybrid Attention for Video Diffusion Transformers",
  abstract: attention that mixes exact softmax attention with linear
  attention, evaluated chunk by chunk as a recurrence with a memory footprint
  that does not grow with the sequence.
* "Long-Horizon Streaming Video Generation via Hybrid Attention with Decoupled
  Distillation" (explainer page), section 2.A "Hybrid Attention": recent
  frames inside a sliding window get softmax attention, organised in blocks as
  in FlashAttention; the key/value content of frames that leave the window is
  accumulated online into a fixed-size linear-attention state.  Section 1
  "Background and problem": the sliding window keeps only recent frames in a
  KV cache of an autoregressive (streaming) generator.
* "Transformers are RNNs: Fast Autoregressive Transformers with Linear
  Attention" (listed among the works ReHyAt builds on): the feature map
  phi(x) = elu(x) + 1 and the recurrent form S = sum phi(k) v^T,
  z = sum phi(k).

The pages print no equation for the hybrid.  This oracle uses the shared
normaliser form: for query i in chunk c = floor(i / C) with window w chunks
(the query's own chunk included),

    W(i) = { j : max(0, c - w + 1) <= floor(j / C) <= c }   softmax window
    H(i) = { j : floor(j / C) <= c - w }                      folded history
    a_ij = exp(q_i . k_j / sqrt(d))   for j in W(i)
         = phi(q_i) . phi(k_j)         for j in H(i)
         = 0                           otherwise
    out_i = sum_j a_ij v_j / sum_j a_ij

Splitting the sums over H(i) gives S_c = sum_{H} phi(k_j) v_j^T and
z_c = sum_{H} phi(k_j), the state the recurrence carries.  Readings taken where
the pages are silent: chunk-causal (no future chunk is visible, no token mask
inside the window); w counts the query's own chunk; w = 0 means the own chunk
is already folded into the state (pure linear attention); phi acts on the raw
q and k, feature size d; softmax scale 1/sqrt(d) with the natural exponential.

Every function here is pinned by tests against something other than itself
(brute force, torch's SDPA in the w >= N limit, a token-by-token linear RNN
in the w = 0 limit, hand-derived closed forms, and algebraic invariants).

Arrays are numpy float64.  Per-head functions take [L, d] arrays; the
``*_batched`` helpers loop over [B, H, L, d].
"""
from __future__ import annotations

import math

import numpy as np

# exp of a score is taken literally (no max subtraction); scores this large
# would overflow float64, so the oracle refuses them rather than return inf.
_MAX_ABS_SCORE = 700.0


def phi(x):
    """Feature map elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (always > 0)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def window_range(c: int, w: int):
    """Chunks [lo, hi] of the softmax window of query chunk c (empty if w == 0)."""
    if w <= 0:
        return c + 1, c  # empty
    return max(0, c - w + 1), c


def _scores(q, k):
    d = q.shape[-1]
    s = (q @ k.T) / math.sqrt(d)
    if s.size and np.abs(s).max() >= _MAX_ABS_SCORE:
        raise OverflowError("score magnitude too large for the literal exponential")
    return s


def brute_masked(q, k, v, C: int, w: int, return_den: bool = False):
    """The definition written out as one L x L weight matrix (tiny inputs only).

    a_ij as in the module docstring, out = (A V) / (A 1).
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L = q.shape[0]
    cid = np.arange(L) // C
    cq, ck = cid[:, None], cid[None, :]
    in_window = (ck <= cq) & (ck >= cq - w + 1) if w > 0 else np.zeros((L, L), bool)
    in_history = ck <= cq - w
    a = np.zeros((L, L))
    s = _scores(q, k)
    a[in_window] = np.exp(s[in_window])
    lin = phi(q) @ phi(k).T
    a[in_history] = lin[in_history]
    den = a.sum(axis=1)
    out = (a @ v) / den[:, None]
    return (out, den) if return_den else out


def chunk_states(k, v, C: int):
    """Per-chunk contributions U_c = phi(K_c)^T V_c (d x d) and u_c = sum phi(k_t)."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    L, d = k.shape
    N = L // C
    fk = phi(k)
    U = np.zeros((N, d, v.shape[1]))
    u = np.zeros((N, d))
    for c in range(N):
        sl = slice(c * C, (c + 1) * C)
        U[c] = fk[sl].T @ v[sl]
        u[c] = fk[sl].sum(axis=0)
    return U, u


def state_scan(k, v, C: int, w: int):
    """State seen by each query chunk: S_c = sum_{j <= c-w} U_j, z_c likewise.

    Zero for c < w.  With w = 0 the own chunk is included.
    """
    U, u = chunk_states(k, v, C)
    N = U.shape[0]
    S = np.zeros_like(U)
    z = np.zeros_like(u)
    for c in range(N):
        last = c - w  # last folded chunk
        if last >= 0:
            S[c] = U[: last + 1].sum(axis=0)
            z[c] = u[: last + 1].sum(axis=0)
    return S, z


def state_after(k, v, C: int, w: int, T: int):
    """State after T committed streaming steps: every chunk j <= T - w folded.

    This is the state the next chunk (index T) attends to.
    """
    U, u = chunk_states(k[: T * C], v[: T * C], C)
    last = T - w
    if last < 0:
        return np.zeros(U.shape[1:]), np.zeros(u.shape[1:])
    return U[: last + 1].sum(axis=0), u[: last + 1].sum(axis=0)


def hybrid(q, k, v, C: int, w: int, return_den: bool = False):
    """Chunked evaluation of the definition: per query chunk, the window block
    of exponentials plus the history folded into (S_c, z_c)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L, d = q.shape
    N = L // C
    S, z = state_scan(k, v, C, w)
    fq = phi(q)
    out = np.empty((L, v.shape[1]))
    den_all = np.empty(L)
    for c in range(N):
        rows = slice(c * C, (c + 1) * C)
        num = fq[rows] @ S[c]
        den = fq[rows] @ z[c]
        lo, hi = window_range(c, w)
        if lo <= hi:
            keys = slice(lo * C, (hi + 1) * C)
            e = np.exp(_scores(q[rows], k[keys]))
            num = num + e @ v[keys]
            den = den + e.sum(axis=1)
        out[rows] = num / den[:, None]
        den_all[rows] = den
    return (out, den_all) if return_den else out


def hybrid_rows(q, k, v, C: int, w: int, rows, S=None, z=None, return_den=False):
    """The definition evaluated for selected query rows only.

    For full-size workloads: the per-chunk states (S, z from ``state_scan``)
    cost O(L d^2); each row then costs O(w C d).  Pass S, z to reuse them.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    if S is None:
        S, z = state_scan(k, v, C, w)
    rows = np.asarray(rows)
    out = np.empty((rows.size, v.shape[1]))
    den_all = np.empty(rows.size)
    for n, i in enumerate(rows):
        c = int(i) // C
        fq = phi(q[i])
        num = fq @ S[c]
        den = fq @ z[c]
        lo, hi = window_range(c, w)
        if lo <= hi:
            keys = slice(lo * C, (hi + 1) * C)
            e = np.exp(_scores(q[i : i + 1], k[keys]))[0]
            num = num + e @ v[keys]
            den = den + e.sum()
        out[n] = num / den
        den_all[n] = den
    return (out, den_all) if return_den else out


def hybrid_batched(q, k, v, C: int, w: int, return_den: bool = False):
    """``hybrid`` over [B, H, L, d] arrays (any float dtype; computed in float64)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, L, _ = q.shape
    out = np.empty(q.shape[:3] + (v.shape[-1],))
    den = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            out[b, h], den[b, h] = hybrid(q[b, h], k[b, h], v[b, h], C, w, return_den=True)
    return (out, den) if return_den else out


def state_scan_batched(k, v, C: int, w: int):
    """``state_scan`` over [B, H, L, d]: S [B, H, N, d, d], z [B, H, N, d]."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    B, H, L, d = k.shape
    N = L // C
    S = np.empty((B, H, N, d, v.shape[-1]))
    z = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            S[b, h], z[b, h] = state_scan(k[b, h], v[b, h], C, w)
    return S, z


# ---------------------------------------------------------------- block-sparse window
#
# "Long-Horizon Streaming Video Generation via Hybrid Attention with Decoupled
# Distillation" (explainer page), section 2.A, block-sparse sliding-window
# attention: inside the local window, attention is evaluated in blocks as in
# FlashAttention and the blocks judged unimportant are pruned.  The page gives
# no importance criterion, so the kept blocks are an input: a 0/1 mask per
# (query block, key block).  Blocks: query block i of chunk c holds rows
# c*C + qtile*i .. (clipped to the chunk); key block j of that chunk's window
# holds keys kbeg + ktile*j .. (clipped to the window), kbeg being the first
# key of the window.  A pruned block contributes nothing (its a_ij are 0); the
# folded history is not affected.  A query left with no weight at all (no
# kept key and an empty history) gets output 0 and denominator 0.


def sparse_mask_shape(C: int, N: int, w: int, qtile: int = 256, ktile: int = 64):
    """Per-head mask shape (N, query blocks per chunk, key blocks per window)."""
    nqt = -(-C // qtile)
    wl = min(w, N) if w > 0 else 0
    return N, nqt, -(-(wl * C) // ktile)


def brute_block_sparse(q, k, v, C: int, w: int, mask, qtile: int = 256, ktile: int = 64,
                       return_den: bool = False):
    """The pruned definition as one L x L weight matrix (tiny inputs only)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    mask = np.asarray(mask)
    L = q.shape[0]
    s = _scores(q, k)
    lin = phi(q) @ phi(k).T
    a = np.zeros((L, L))
    for i in range(L):
        c = i // C
        qi = (i - c * C) // qtile
        lo, hi = window_range(c, w)
        for j in range(L):
            cj = j // C
            if lo <= cj <= hi:
                if mask[c, qi, (j - lo * C) // ktile]:
                    a[i, j] = math.exp(s[i, j])
            elif cj <= c - w:
                a[i, j] = lin[i, j]
    den = a.sum(axis=1)
    num = a @ v
    out = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)
    return (out, den) if return_den else out


def _window_keep(mask_row, n_keys: int, ktile: int):
    """0/1 per key of a window of n_keys keys from one mask row."""
    keep = np.repeat(np.asarray(mask_row, dtype=bool), ktile)[:n_keys]
    if keep.size < n_keys:
        raise ValueError("mask row too short for the window")
    return keep


def hybrid_block_sparse(q, k, v, C: int, w: int, mask, qtile: int = 256, ktile: int = 64,
                        return_den: bool = False):
    """Chunked evaluation of the pruned definition (one head; mask [N, nqt, nkt])."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    mask = np.asarray(mask)
    L, d = q.shape
    N = L // C
    S, z = state_scan(k, v, C, w)
    fq = phi(q)
    out = np.empty((L, v.shape[1]))
    den_all = np.empty(L)
    for c in range(N):
        lo, hi = window_range(c, w)
        for i in range(-(-C // qtile)):
            rows = slice(c * C + i * qtile, c * C + min(C, (i + 1) * qtile))
            num = fq[rows] @ S[c]
            den = fq[rows] @ z[c]
            if lo <= hi:
                keys = slice(lo * C, (hi + 1) * C)
                keep = _window_keep(mask[c, i], (hi + 1 - lo) * C, ktile)
                e = np.exp(_scores(q[rows], k[keys])) * keep[None, :]
                num = num + e @ v[keys]
                den = den + e.sum(axis=1)
            safe = np.where(den > 0, den, 1.0)
            out[rows] = np.where(den[:, None] > 0, num / safe[:, None], 0.0)
            den_all[rows] = den
    return (out, den_all) if return_den else out


def hybrid_block_sparse_rows(q, k, v, C: int, w: int, mask, rows, S=None, z=None, qtile: int = 256,
                             ktile: int = 64, return_den: bool = False):
    """The pruned definition for selected query rows (one head)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    mask = np.asarray(mask)
    if S is None:
        S, z = state_scan(k, v, C, w)
    rows = np.asarray(rows)
    out = np.empty((rows.size, v.shape[1]))
    den_all = np.empty(rows.size)
    for n, r in enumerate(rows):
        r = int(r)
        c = r // C
        fq = phi(q[r])
        num = fq @ S[c]
        den = fq @ z[c]
        lo, hi = window_range(c, w)
        if lo <= hi:
            keys = slice(lo * C, (hi + 1) * C)
            keep = _window_keep(mask[c, (r - c * C) // qtile], (hi + 1 - lo) * C, ktile)
            e = np.exp(_scores(q[r : r + 1], k[keys]))[0] * keep
            num = num + e @ v[keys]
            den = den + e.sum()
        out[n] = num / den if den > 0 else 0.0
        den_all[n] = den
    return (out, den_all) if return_den else out


def hybrid_block_sparse_batched(q, k, v, C: int, w: int, mask, return_den: bool = False, **tiles):
    """``hybrid_block_sparse`` over [B, H, L, d] with mask [B, H, N, nqt, nkt]."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    mask = np.asarray(mask)
    B, H, L, _ = q.shape
    out = np.empty(q.shape[:3] + (v.shape[-1],))
    den = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            out[b, h], den[b, h] = hybrid_block_sparse(q[b, h], k[b, h], v[b, h], C, w, mask[b, h],
                                                       return_den=True, **tiles)
    return (out, den) if return_den else out


# ---------------------------------------------------------------- pruned streaming step
#
# Hybrid Forcing explainer, section 1 (the streaming generator keeps the
# window's chunks in a KV cache) and section 2.A (its window attention is
# block-sparse).  Reading taken for a pruned streaming step (the pages fix no
# block layout for the cache): the step for chunk t attends to the chunks of
# its window as the cache holds them -- one slot per chunk, chunk c in slot
# c mod w, the slots in order 0, 1, .. (before the ring is full, slots 0 .. t)
# -- and the key blocks are ktile keys each, counted from slot 0's first key.
# Query blocks are qtile rows of the new chunk.  One mask per step,
# [nqt, nkt]; entries past the keys in use are ignored.  A pruned block adds
# nothing; the folded history is that of the plain step (chunks <= t - w).
# Softmax is order-free, so with every block kept this is the plain hybrid.


def stream_slot_chunks(t: int, w: int):
    """The chunks of step t's window in cache-slot order (slot s holds chunk c = s mod w)."""
    if w < 1:
        raise ValueError("a streaming window has at least one chunk")
    if t + 1 <= w:
        return list(range(t + 1))
    first = t - w + 1
    return [first + ((s - first) % w) for s in range(w)]


def stream_block_sparse(q, k, v, C: int, w: int, masks, qtile: int = 256, ktile: int = 64,
                        return_den: bool = False):
    """Pruned streaming steps over a whole stream (one head): chunk t of q
    attends to its window in cache-slot order with mask masks[t] ([nqt, nkt])
    and to the folded history; returns [L, d] (and the denominators)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    masks = np.asarray(masks)
    L, d = q.shape
    N = L // C
    S, z = state_scan(k, v, C, w)
    fq = phi(q)
    out = np.empty((L, v.shape[1]))
    den_all = np.empty(L)
    for t in range(N):
        order = stream_slot_chunks(t, w)
        kw = np.concatenate([k[c * C:(c + 1) * C] for c in order])
        vw = np.concatenate([v[c * C:(c + 1) * C] for c in order])
        for i in range(-(-C // qtile)):
            rows = slice(t * C + i * qtile, t * C + min(C, (i + 1) * qtile))
            keep = _window_keep(masks[t, i], kw.shape[0], ktile)
            e = np.exp(_scores(q[rows], kw)) * keep[None, :]
            num = fq[rows] @ S[t] + e @ vw
            den = fq[rows] @ z[t] + e.sum(axis=1)
            safe = np.where(den > 0, den, 1.0)
            out[rows] = np.where(den[:, None] > 0, num / safe[:, None], 0.0)
            den_all[rows] = den
    return (out, den_all) if return_den else out


def stream_block_sparse_rows(q, k, v, C: int, w: int, t: int, mask_t, rows, S=None, z=None, qtile: int = 256,
                             ktile: int = 64):
    """``stream_block_sparse`` for selected rows (within chunk t) of step t only
    (one head; mask_t [nqt, nkt]; S, z: state_scan's slots, computed if absent)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    if S is None:
        S, z = state_scan(k, v, C, w)
    order = stream_slot_chunks(t, w)
    kw = np.concatenate([k[c * C:(c + 1) * C] for c in order])
    vw = np.concatenate([v[c * C:(c + 1) * C] for c in order])
    out = np.empty((len(rows), v.shape[1]))
    for n, r in enumerate(rows):
        r = int(r)
        keep = _window_keep(np.asarray(mask_t)[r // qtile], kw.shape[0], ktile)
        e = np.exp(_scores(q[t * C + r : t * C + r + 1], kw))[0] * keep
        fq = phi(q[t * C + r])
        num = e @ vw + fq @ S[t]
        den = e.sum() + fq @ z[t]
        out[n] = num / den if den > 0 else 0.0
    return out


def stream_block_sparse_batched(q, k, v, C: int, w: int, masks, return_den: bool = False, **tiles):
    """``stream_block_sparse`` over [B, H, L, d] with masks [B, H, N, nqt, nkt]."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    masks = np.asarray(masks)
    B, H, L, _ = q.shape
    out = np.empty(q.shape[:3] + (v.shape[-1],))
    den = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            out[b, h], den[b, h] = stream_block_sparse(q[b, h], k[b, h], v[b, h], C, w, masks[b, h],
                                                       return_den=True, **tiles)
    return (out, den) if return_den else out


# ---------------------------------------------------------------- bidirectional hybrid
#
# "ReHyAt: Recurrent Hybrid Attention for Video Diffusion Transformers",
# abstract: the hybrid replaces the softmax attention of video diffusion
# transformers, whose attention is bidirectional over the whole clip.  Reading
# taken for the bidirectional form: the softmax window is symmetric around the
# query's chunk, and every chunk outside it -- before or after -- is folded
# into the linear term, so that a window covering every chunk is plain dense
# (unmasked) softmax attention and window 0 is plain (non-causal) linear
# attention:
#
#     W(i) = { j : |floor(j/C) - c| <= w - 1 }           (empty if w == 0)
#     H(i) = every other key
#
# The linear term splits into a past part and a future part:
#     S_pre_c = sum_{c' <= c - w} U_c'   (with w = 0: c' <= c, own chunk included)
#     S_suf_c = sum_{c' >= c + max(w, 1)} U_c'
# and likewise z.  out_i = (sum_W e^s v + phi(q_i)^T (S_pre_c + S_suf_c)) /
# (sum_W e^s + phi(q_i) . (z_pre_c + z_suf_c)).


def window_range_bidir(c: int, w: int, N: int):
    """Chunks [lo, hi] of the symmetric softmax window of chunk c (empty if w == 0)."""
    if w <= 0:
        return c + 1, c
    return max(0, c - w + 1), min(N - 1, c + w - 1)


def brute_bidir(q, k, v, C: int, w: int, return_den: bool = False):
    """The bidirectional definition as one L x L weight matrix (tiny inputs only)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L = q.shape[0]
    cid = np.arange(L) // C
    dist = np.abs(cid[None, :] - cid[:, None])
    in_window = dist <= w - 1 if w > 0 else np.zeros((L, L), bool)
    a = np.where(in_window, np.exp(_scores(q, k)), phi(q) @ phi(k).T)
    den = a.sum(axis=1)
    out = (a @ v) / den[:, None]
    return (out, den) if return_den else out


def state_scan_bidir(k, v, C: int, w: int):
    """Past and future states of every chunk: (S_pre, z_pre, S_suf, z_suf)."""
    U, u = chunk_states(k, v, C)
    N = U.shape[0]
    S_pre, z_pre = state_scan(k, v, C, w)
    S_suf, z_suf = np.zeros_like(U), np.zeros_like(u)
    first = max(w, 1)
    for c in range(N):
        if c + first <= N - 1:
            S_suf[c] = U[c + first:].sum(axis=0)
            z_suf[c] = u[c + first:].sum(axis=0)
    return S_pre, z_pre, S_suf, z_suf


def hybrid_bidir(q, k, v, C: int, w: int, return_den: bool = False):
    """Chunked evaluation of the bidirectional definition (one head)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L, d = q.shape
    N = L // C
    S_pre, z_pre, S_suf, z_suf = state_scan_bidir(k, v, C, w)
    fq = phi(q)
    out = np.empty((L, v.shape[1]))
    den_all = np.empty(L)
    for c in range(N):
        rows = slice(c * C, (c + 1) * C)
        num = fq[rows] @ (S_pre[c] + S_suf[c])
        den = fq[rows] @ (z_pre[c] + z_suf[c])
        lo, hi = window_range_bidir(c, w, N)
        if lo <= hi:
            keys = slice(lo * C, (hi + 1) * C)
            e = np.exp(_scores(q[rows], k[keys]))
            num = num + e @ v[keys]
            den = den + e.sum(axis=1)
        out[rows] = num / den[:, None]
        den_all[rows] = den
    return (out, den_all) if return_den else out


def hybrid_bidir_rows(q, k, v, C: int, w: int, rows, states=None, return_den: bool = False):
    """The bidirectional definition for selected rows; states from state_scan_bidir."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    N = q.shape[0] // C
    S_pre, z_pre, S_suf, z_suf = states if states is not None else state_scan_bidir(k, v, C, w)
    rows = np.asarray(rows)
    out = np.empty((rows.size, v.shape[1]))
    den_all = np.empty(rows.size)
    for n, r in enumerate(rows):
        r = int(r)
        c = r // C
        fq = phi(q[r])
        num = fq @ (S_pre[c] + S_suf[c])
        den = fq @ (z_pre[c] + z_suf[c])
        lo, hi = window_range_bidir(c, w, N)
        if lo <= hi:
            keys = slice(lo * C, (hi + 1) * C)
            e = np.exp(_scores(q[r : r + 1], k[keys]))[0]
            num = num + e @ v[keys]
            den = den + e.sum()
        out[n] = num / den
        den_all[n] = den
    return (out, den_all) if return_den else out


def hybrid_bidir_batched(q, k, v, C: int, w: int, return_den: bool = False):
    """``hybrid_bidir`` over [B, H, L, d]."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, L, _ = q.shape
    out = np.empty(q.shape[:3] + (v.shape[-1],))
    den = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            out[b, h], den[b, h] = hybrid_bidir(q[b, h], k[b, h], v[b, h], C, w, return_den=True)
    return (out, den) if return_den else out


def state_scan_bidir_batched(k, v, C: int, w: int):
    """``state_scan_bidir`` over [B, H, L, d]: four arrays [B, H, N, ...]."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    B, H, L, d = k.shape
    N = L // C
    res = [np.empty((B, H, N, d, v.shape[-1])), np.empty((B, H, N, d)),
           np.empty((B, H, N, d, v.shape[-1])), np.empty((B, H, N, d))]
    for b in range(B):
        for h in range(H):
            for arr, val in zip(res, state_scan_bidir(k[b, h], v[b, h], C, w)):
                arr[b, h] = val
    return tuple(res)


# ---------------------------------------------------------------- anchor (sink) chunks
#
# Hybrid Forcing explainer, section 1: the attention-sink workaround keeps the
# first frame(s) of the video attended by every later frame.  Combined with the
# hybrid: the first `a` chunks are anchors -- always in the softmax window of
# every query chunk that they do not lie in the future of, and never folded
# into the linear state:
#
#     W(i) = window(c) + { j : floor(j/C) < a and floor(j/C) <= c }
#     H(i) = { j : a <= floor(j/C) <= c - w }
#
# a = 0 is the plain hybrid.


def brute_anchor(q, k, v, C: int, w: int, a: int, return_den: bool = False):
    """The anchored definition as one L x L weight matrix (tiny inputs only)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L = q.shape[0]
    cid = np.arange(L) // C
    cq, ck = cid[:, None], cid[None, :]
    in_window = ((ck <= cq) & (ck >= cq - w + 1)) if w > 0 else np.zeros((L, L), bool)
    in_window = in_window | ((ck < a) & (ck <= cq))
    in_history = (ck >= a) & (ck <= cq - w) & ~in_window
    s = _scores(q, k)
    wts = np.zeros((L, L))
    wts[in_window] = np.exp(s[in_window])
    lin = phi(q) @ phi(k).T
    wts[in_history] = lin[in_history]
    den = wts.sum(axis=1)
    out = (wts @ v) / den[:, None]
    return (out, den) if return_den else out


def state_scan_anchor(k, v, C: int, w: int, a: int):
    """S_c = sum_{a <= j <= c-w} U_j (z likewise): the history without anchors."""
    U, u = chunk_states(k, v, C)
    N = U.shape[0]
    S, z = np.zeros_like(U), np.zeros_like(u)
    for c in range(N):
        lo, hi = a, c - w
        if hi >= lo:
            S[c] = U[lo : hi + 1].sum(axis=0)
            z[c] = u[lo : hi + 1].sum(axis=0)
    return S, z


def anchor_keys(c: int, C: int, w: int, a: int):
    """Sorted key indices of the anchored softmax window of chunk c."""
    lo, hi = window_range(c, w)
    win = set(range(lo * C, (hi + 1) * C)) if lo <= hi else set()
    anc = set(range(0, min(a, c + 1) * C))
    return np.array(sorted(win | anc), dtype=np.int64)


def hybrid_anchor(q, k, v, C: int, w: int, a: int, return_den: bool = False):
    """Chunked evaluation of the anchored definition (one head)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L, d = q.shape
    N = L // C
    S, z = state_scan_anchor(k, v, C, w, a)
    fq = phi(q)
    out = np.empty((L, v.shape[1]))
    den_all = np.empty(L)
    for c in range(N):
        rows = slice(c * C, (c + 1) * C)
        num = fq[rows] @ S[c]
        den = fq[rows] @ z[c]
        keys = anchor_keys(c, C, w, a)
        if keys.size:
            e = np.exp(_scores(q[rows], k[keys]))
            num = num + e @ v[keys]
            den = den + e.sum(axis=1)
        out[rows] = num / den[:, None]
        den_all[rows] = den
    return (out, den_all) if return_den else out


def hybrid_anchor_rows(q, k, v, C: int, w: int, a: int, rows, S=None, z=None, return_den: bool = False):
    """The anchored definition for selected rows (one head)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    if S is None:
        S, z = state_scan_anchor(k, v, C, w, a)
    rows = np.asarray(rows)
    out = np.empty((rows.size, v.shape[1]))
    den_all = np.empty(rows.size)
    for n, r in enumerate(rows):
        r = int(r)
        c = r // C
        fq = phi(q[r])
        num = fq @ S[c]
        den = fq @ z[c]
        keys = anchor_keys(c, C, w, a)
        if keys.size:
            e = np.exp(_scores(q[r : r + 1], k[keys]))[0]
            num = num + e @ v[keys]
            den = den + e.sum()
        out[n] = num / den
        den_all[n] = den
    return (out, den_all) if return_den else out


def hybrid_anchor_batched(q, k, v, C: int, w: int, a: int, return_den: bool = False):
    """``hybrid_anchor`` over [B, H, L, d]."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, L, _ = q.shape
    out = np.empty(q.shape[:3] + (v.shape[-1],))
    den = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            out[b, h], den[b, h] = hybrid_anchor(q[b, h], k[b, h], v[b, h], C, w, a, return_den=True)
    return (out, den) if return_den else out


def state_scan_anchor_batched(k, v, C: int, w: int, a: int):
    """``state_scan_anchor`` over [B, H, L, d]."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    B, H, L, d = k.shape
    N = L // C
    S = np.empty((B, H, N, d, v.shape[-1]))
    z = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            S[b, h], z[b, h] = state_scan_anchor(k[b, h], v[b, h], C, w, a)
    return S, z


# ---------------------------------------------------------------- backward pass
#
# Gradients of L = sum_i dout_i . out_i for the causal hybrid (the definition
# at the top), written out by the chain rule.  With N_i, D_i the numerator and
# the shared denominator of row i (D_i = exp(lse_i)):
#
#   dN_i = dout_i / D_i,   dD_i = -(dout_i . out_i) / D_i
#   window key j:  E_ij = exp(s_ij),  dE_ij = dN_i . v_j + dD_i
#                  dv_j += E_ij dN_i,  ds_ij = E_ij dE_ij,
#                  dq_i += ds_ij k_j / sqrt(d),  dk_j += ds_ij q_i / sqrt(d)
#   linear term:   dphi(q_i) = S_c dN_i + z_c dD_i   (S_c^T rows)
#                  dS_c = sum_{i in c} phi(q_i) dN_i^T,  dz_c = sum_{i in c} phi(q_i) dD_i
#                  dU_j = sum_{c : j <= c - w} dS_c   (likewise du_j)
#                  dv_t += dU_j^T phi(k_t),  dphi(k_t) = dU_j v_t + du_j
#   and phi'(x) = 1 for x > 0, exp(x) otherwise.


def dphi(x):
    """Derivative of phi = elu + 1."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def hybrid_backward(q, k, v, C: int, w: int, dout):
    """(dq, dk, dv) of sum(dout * hybrid(q, k, v, C, w)) for one head."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    L, d = q.shape
    N = L // C
    scale = 1.0 / math.sqrt(d)
    S, z = state_scan(k, v, C, w)
    U_shape = S.shape
    out, den = hybrid(q, k, v, C, w, return_den=True)
    dN = dout / den[:, None]
    dD = -(dout * out).sum(axis=1) / den
    fq, fk = phi(q), phi(k)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dS, dz = np.zeros(U_shape), np.zeros(z.shape)
    for c in range(N):
        rows = slice(c * C, (c + 1) * C)
        lo, hi = window_range(c, w)
        if lo <= hi:
            keys = slice(lo * C, (hi + 1) * C)
            E = np.exp(_scores(q[rows], k[keys]))
            dE = dN[rows] @ v[keys].T + dD[rows][:, None]
            dv[keys] += E.T @ dN[rows]
            ds = E * dE
            dq[rows] += ds @ k[keys] * scale
            dk[keys] += ds.T @ q[rows] * scale
        gq = dN[rows] @ S[c].T + dD[rows][:, None] * z[c][None, :]
        dq[rows] += gq * dphi(q[rows])
        dS[c] = fq[rows].T @ dN[rows]
        dz[c] = fq[rows].T @ dD[rows]
    for j in range(N):
        first = j + w  # S_c contains U_j for c >= j + w
        if first > N - 1:
            continue
        dU = dS[first:].sum(axis=0)
        du = dz[first:].sum(axis=0)
        toks = slice(j * C, (j + 1) * C)
        dv[toks] += fk[toks] @ dU
        gk = v[toks] @ dU.T + du[None, :]
        dk[toks] += gk * dphi(k[toks])
    return dq, dk, dv


def hybrid_backward_batched(q, k, v, C: int, w: int, dout):
    """``hybrid_backward`` over [B, H, L, d]."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    B, H = q.shape[:2]
    res = [np.empty_like(q), np.empty_like(k), np.empty_like(v)]
    for b in range(B):
        for h in range(H):
            for arr, g in zip(res, hybrid_backward(q[b, h], k[b, h], v[b, h], C, w, dout[b, h])):
                arr[b, h] = g
    return tuple(res)


# ---------------------------------------------------------------------------
# Backward pass of the bidirectional hybrid (the hybrid that stands in for the
# bidirectional attention of video diffusion transformers: ReHyAt, abstract;
# the symmetric-window reading of the bidirectional form above).  The same
# chain rule as ``hybrid_backward``, on ``hybrid_bidir``: the window is
# symmetric, and chunk c's linear term uses S_pre_c + S_suf_c, so the state
# gradient dS_c reaches chunk j's keys through the past part when
# j <= c - w (w = 0: j <= c) and through the future part when
# j >= c + max(w, 1).

def hybrid_bidir_backward(q, k, v, C: int, w: int, dout):
    """(dq, dk, dv) of sum(dout * hybrid_bidir(q, k, v, C, w)) for one head."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    L, d = q.shape
    N = L // C
    scale = 1.0 / math.sqrt(d)
    S_pre, z_pre, S_suf, z_suf = state_scan_bidir(k, v, C, w)
    out, den = hybrid_bidir(q, k, v, C, w, return_den=True)
    dN = dout / den[:, None]  # d loss / d numerator
    dD = -(dout * out).sum(axis=1) / den  # d loss / d denominator
    fq, fk = phi(q), phi(k)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dS, dz = np.zeros(S_pre.shape), np.zeros(z_pre.shape)
    for c in range(N):
        rows = slice(c * C, (c + 1) * C)
        lo, hi = window_range_bidir(c, w, N)
        if lo <= hi:
            keys = slice(lo * C, (hi + 1) * C)
            E = np.exp(_scores(q[rows], k[keys]))
            dE = dN[rows] @ v[keys].T + dD[rows][:, None]
            dv[keys] += E.T @ dN[rows]
            ds = E * dE
            dq[rows] += ds @ k[keys] * scale
            dk[keys] += ds.T @ q[rows] * scale
        S = S_pre[c] + S_suf[c]
        z = z_pre[c] + z_suf[c]
        gq = dN[rows] @ S.T + dD[rows][:, None] * z[None, :]
        dq[rows] += gq * dphi(q[rows])
        dS[c] = fq[rows].T @ dN[rows]
        dz[c] = fq[rows].T @ dD[rows]
    first = max(w, 1)
    for j in range(N):
        # chunks whose linear term holds chunk j: c >= j + w (past part) and
        # c <= j - max(w, 1) (future part)
        users = [c for c in range(N) if c >= j + w or c <= j - first]
        if not users:
            continue
        dU = dS[users].sum(axis=0)
        du = dz[users].sum(axis=0)
        toks = slice(j * C, (j + 1) * C)
        dv[toks] += fk[toks] @ dU
        gk = v[toks] @ dU.T + du[None, :]
        dk[toks] += gk * dphi(k[toks])
    return dq, dk, dv


def hybrid_bidir_backward_batched(q, k, v, C: int, w: int, dout):
    """``hybrid_bidir_backward`` over [B, H, L, d]."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    B, H = q.shape[:2]
    res = [np.empty_like(q), np.empty_like(k), np.empty_like(v)]
    for b in range(B):
        for h in range(H):
            for arr, g in zip(res, hybrid_bidir_backward(q[b, h], k[b, h], v[b, h], C, w, dout[b, h])):
                arr[b, h] = g
    return tuple(res)


# ---------------------------------------------------------------------------
# Backward pass of the anchored hybrid (anchor chunks as above): the chain rule
# of ``hybrid_backward`` on ``hybrid_anchor``.  A query chunk's softmax keys are
# its window and the anchors not in its future; its state holds chunks
# a .. c - w, so only non-anchor key chunks receive a state gradient.

def hybrid_anchor_backward(q, k, v, C: int, w: int, a: int, dout):
    """(dq, dk, dv) of sum(dout * hybrid_anchor(q, k, v, C, w, a)) for one head."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    L, d = q.shape
    N = L // C
    scale = 1.0 / math.sqrt(d)
    S, z = state_scan_anchor(k, v, C, w, a)
    out, den = hybrid_anchor(q, k, v, C, w, a, return_den=True)
    dN = dout / den[:, None]
    dD = -(dout * out).sum(axis=1) / den
    fq, fk = phi(q), phi(k)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dS, dz = np.zeros(S.shape), np.zeros(z.shape)
    for c in range(N):
        rows = slice(c * C, (c + 1) * C)
        keys = anchor_keys(c, C, w, a)
        if keys.size:
            E = np.exp(_scores(q[rows], k[keys]))
            dE = dN[rows] @ v[keys].T + dD[rows][:, None]
            dv[keys] += E.T @ dN[rows]
            ds = E * dE
            dq[rows] += ds @ k[keys] * scale
            dk[keys] += ds.T @ q[rows] * scale
        gq = dN[rows] @ S[c].T + dD[rows][:, None] * z[c][None, :]
        dq[rows] += gq * dphi(q[rows])
        dS[c] = fq[rows].T @ dN[rows]
        dz[c] = fq[rows].T @ dD[rows]
    for j in range(a, N):  # anchors are never in a state
        first = j + w  # S_c holds U_j for c >= j + w
        if first > N - 1:
            continue
        dU = dS[first:].sum(axis=0)
        du = dz[first:].sum(axis=0)
        toks = slice(j * C, (j + 1) * C)
        dv[toks] += fk[toks] @ dU
        gk = v[toks] @ dU.T + du[None, :]
        dk[toks] += gk * dphi(k[toks])
    return dq, dk, dv


def hybrid_anchor_backward_batched(q, k, v, C: int, w: int, a: int, dout):
    """``hybrid_anchor_backward`` over [B, H, L, d]."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    B, H = q.shape[:2]
    res = [np.empty_like(q), np.empty_like(k), np.empty_like(v)]
    for b in range(B):
        for h in range(H):
            for arr, g in zip(res, hybrid_anchor_backward(q[b, h], k[b, h], v[b, h], C, w, a, dout[b, h])):
                arr[b, h] = g
    return tuple(res)


# ---------------------------------------------------------------------------
# Backward pass of the pruned window (the block-sparse definition above): the
# chain rule of ``hybrid_backward`` with the pruned (query block, key block)
# pairs' weights held at zero.  A row left with no weight at all (every block
# pruned and no history) has out = 0 whatever the inputs, so its gradients are
# zero.

def hybrid_block_sparse_backward(q, k, v, C: int, w: int, mask, dout, qtile: int = 256, ktile: int = 64):
    """(dq, dk, dv) of sum(dout * hybrid_block_sparse(q, k, v, C, w, mask)) for one head."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    mask = np.asarray(mask)
    L, d = q.shape
    N = L // C
    scale = 1.0 / math.sqrt(d)
    S, z = state_scan(k, v, C, w)
    out, den = hybrid_block_sparse(q, k, v, C, w, mask, qtile, ktile, return_den=True)
    live = den > 0
    safe = np.where(live, den, 1.0)
    dN = np.where(live[:, None], dout / safe[:, None], 0.0)
    dD = np.where(live, -(dout * out).sum(axis=1) / safe, 0.0)
    fq, fk = phi(q), phi(k)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dS, dz = np.zeros(S.shape), np.zeros(z.shape)
    for c in range(N):
        lo, hi = window_range(c, w)
        for i in range(-(-C // qtile)):
            rows = slice(c * C + i * qtile, c * C + min(C, (i + 1) * qtile))
            if lo <= hi:
                keys = slice(lo * C, (hi + 1) * C)
                keep = _window_keep(mask[c, i], (hi + 1 - lo) * C, ktile)
                E = np.exp(_scores(q[rows], k[keys])) * keep[None, :]
                dE = dN[rows] @ v[keys].T + dD[rows][:, None]
                dv[keys] += E.T @ dN[rows]
                ds = E * dE
                dq[rows] += ds @ k[keys] * scale
                dk[keys] += ds.T @ q[rows] * scale
            gq = dN[rows] @ S[c].T + dD[rows][:, None] * z[c][None, :]
            dq[rows] += gq * dphi(q[rows])
            dS[c] += fq[rows].T @ dN[rows]
            dz[c] += fq[rows].T @ dD[rows]
    for j in range(N):
        first = j + w
        if first > N - 1:
            continue
        dU = dS[first:].sum(axis=0)
        du = dz[first:].sum(axis=0)
        toks = slice(j * C, (j + 1) * C)
        dv[toks] += fk[toks] @ dU
        gk = v[toks] @ dU.T + du[None, :]
        dk[toks] += gk * dphi(k[toks])
    return dq, dk, dv


def hybrid_block_sparse_backward_batched(q, k, v, C: int, w: int, mask, dout, **tiles):
    """``hybrid_block_sparse_backward`` over [B, H, L, d] with mask [B, H, N, nqt, nkt]."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    mask = np.asarray(mask)
    B, H = q.shape[:2]
    res = [np.empty_like(q), np.empty_like(k), np.empty_like(v)]
    for b in range(B):
        for h in range(H):
            g = hybrid_block_sparse_backward(q[b, h], k[b, h], v[b, h], C, w, mask[b, h], dout[b, h], **tiles)
            for arr, x in zip(res, g):
                arr[b, h] = x
    return tuple(res)
