"""Pins of the fp64 oracle against things other than itself (CPU only).

* phi: closed-form values and torch's elu + 1.
* hand-derived closed forms for a six-token case (tests/golden/hand_worked_d1.json).
* brute-force masked quadratic form vs the chunked oracle over many shapes.
* w >= N limit: torch's scaled_dot_product_attention with a block-causal mask;
  C = 1: its is_causal mode; N = 1: plain full attention.
* w = 0 limit: a token-by-token linear-attention recurrence written here.
* invariants: constant V, linearity and translation in V, permutation of a
  chunk's tokens, convex hull.
* the state scan: summed chunk contributions equal one matmul; lag relations.
* planted mistakes in the oracle are caught by at least one of the pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rha_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_d1.json")
_NS = {"e": math.e, "ln2": math.log(2.0), "ln3": math.log(3.0)}


def _ev(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, dict(_NS)))


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _qkv(L, d, seed, qs=1.0, ks=1.0):
    return _rand((L, d), seed, qs), _rand((L, d), seed + 1, ks), _rand((L, d), seed + 2)


# ---------------------------------------------------------------- phi

def test_phi_closed_form():
    assert O.phi(0.0) == 1.0
    assert O.phi(2.0) == 3.0
    assert O.phi(-1.0) == pytest.approx(1.0 / math.e, rel=1e-15)
    assert O.phi(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-15)
    x = np.linspace(-30, 30, 10001)
    assert (O.phi(x) > 0).all()
    # continuous at 0 from both sides
    assert O.phi(-1e-12) == pytest.approx(1.0, abs=1e-11)
    assert O.phi(1e-12) == pytest.approx(1.0, abs=1e-11)


def test_phi_matches_torch_elu_plus_one():
    x = _rand((4096,), 7, 3.0)
    ref = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0) + 1.0
    # torch forms elu + 1 as expm1(x) + 1, which loses absolute precision 1e-16
    np.testing.assert_allclose(O.phi(x), ref.numpy(), rtol=1e-15, atol=2e-16)


# ---------------------------------------------------------------- golden

def _golden_check(case, data):
    q = np.array([[_ev(s)] for s in data["q"]])
    k = np.array([[_ev(s)] for s in data["k"]])
    v = np.array([[_ev(s)] for s in data["v"]])
    C, w = data["C"], case["w"]
    want = np.array([_ev(s) for s in case["out"]])
    errs = []
    for fn in (O.brute_masked, O.hybrid):
        got, den = fn(q, k, v, C, w, return_den=True)
        errs.append(np.max(np.abs(got[:, 0] - want) / np.maximum(1.0, np.abs(want))))
        if "den" in case:
            wd = np.array([_ev(s) for s in case["den"]])
            errs.append(np.max(np.abs(den - wd) / wd))
    S, z = O.state_scan(k, v, C, w)
    errs.append(np.max(np.abs(S[:, 0, 0] - [_ev(s) for s in case["S"]])))
    errs.append(np.max(np.abs(z[:, 0] - [_ev(s) for s in case["z"]])))
    return max(errs)


def _golden_max_err():
    data = json.load(open(GOLDEN))
    return max(_golden_check(case, data) for case in data["cases"])


@pytest.mark.parametrize("case_idx", [0, 1, 2])
def test_hand_worked_closed_forms(case_idx):
    data = json.load(open(GOLDEN))
    assert _golden_check(data["cases"][case_idx], data) < 1e-14


# ---------------------------------------------------------------- brute vs chunked

SWEEP = [
    (C, N, w, d)
    for C in (1, 3, 64)
    for N in (1, 2, 4, 6)
    for w in sorted({0, 1, 2, N, N + 3})
    for d in (4, 64)
    if C * N <= 512
]


def _brute_vs_chunked(C, N, w, d, seed=3):
    q, k, v = _qkv(C * N, d, seed + 10 * C + N, qs=1.5)
    a, da = O.brute_masked(q, k, v, C, w, return_den=True)
    b, db = O.hybrid(q, k, v, C, w, return_den=True)
    return max(np.max(np.abs(a - b)) / np.max(np.abs(a)), np.max(np.abs(da - db) / da))


@pytest.mark.parametrize("C,N,w,d", SWEEP)
def test_brute_equals_chunked(C, N, w, d):
    assert _brute_vs_chunked(C, N, w, d) < 1e-12


def test_hybrid_rows_equals_hybrid():
    q, k, v = _qkv(6 * 37, 16, 91)
    full, den = O.hybrid(q, k, v, 37, 2, return_den=True)
    rows = np.array([0, 36, 37, 73, 74, 111, 150, 221])
    got, gden = O.hybrid_rows(q, k, v, 37, 2, rows, return_den=True)
    np.testing.assert_allclose(got, full[rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gden, den[rows], rtol=1e-13)


# ---------------------------------------------------------------- w >= N limit: SDPA

def _sdpa(q, k, v, mask=None, causal=False):
    t = lambda x: torch.from_numpy(x)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask,
                                                         is_causal=causal)
    return o[0, 0].numpy()


def _block_causal(L, C):
    c = torch.arange(L) // C
    return (c[None, :] <= c[:, None])[None, None]


def _sdpa_limit_err(C=48, N=5, d=64, seed=21):
    q, k, v = _qkv(C * N, d, seed, qs=2.0)
    errs = []
    for w in (N, N + 1, 10 * N):
        errs.append(np.max(np.abs(O.hybrid(q, k, v, C, w) - _sdpa(q, k, v, _block_causal(C * N, C)))))
        errs.append(np.max(np.abs(O.brute_masked(q, k, v, C, w) - _sdpa(q, k, v, _block_causal(C * N, C)))))
    # the last chunk sees every key: plain unmasked attention for its rows
    last = slice((N - 1) * C, N * C)
    errs.append(np.max(np.abs(O.hybrid(q, k, v, C, N)[last] - _sdpa(q, k, v)[last])))
    return max(errs)


def test_window_all_equals_block_causal_sdpa():
    assert _sdpa_limit_err() < 1e-12


def test_chunk1_window_all_equals_causal_sdpa():
    q, k, v = _qkv(97, 32, 5, qs=2.0)
    np.testing.assert_allclose(O.hybrid(q, k, v, 1, 97), _sdpa(q, k, v, causal=True), atol=1e-12)


def test_one_chunk_equals_full_attention():
    q, k, v = _qkv(130, 64, 9, qs=2.0)
    for w in (1, 2, 7):
        np.testing.assert_allclose(O.hybrid(q, k, v, 130, w), _sdpa(q, k, v), atol=1e-12)


# ---------------------------------------------------------------- w = 0 limit: linear RNN

def _torch_phi(x):
    return (torch.nn.functional.elu(torch.from_numpy(x)) + 1.0).numpy()


def _linear_rnn(q, k, v, C):
    """Causal linear attention token by token: the state absorbs every token of
    a chunk before any query of that chunk reads it (C = 1: plain RNN form)."""
    L, d = q.shape
    fq, fk = _torch_phi(q), _torch_phi(k)
    s = np.zeros((d, v.shape[1]))
    z = np.zeros(d)
    out = np.empty_like(v)
    for c0 in range(0, L, C):
        for t in range(c0, c0 + C):
            s += np.outer(fk[t], v[t])
            z += fk[t]
        for t in range(c0, c0 + C):
            out[t] = fq[t] @ s / (fq[t] @ z)
    return out


def _rnn_limit_err():
    errs = []
    for C, N in ((1, 83), (7, 9), (32, 4)):
        q, k, v = _qkv(C * N, 16, 40 + C)
        ref = _linear_rnn(q, k, v, C)
        errs.append(np.max(np.abs(O.hybrid(q, k, v, C, 0) - ref)))
        errs.append(np.max(np.abs(O.brute_masked(q, k, v, C, 0) - ref)))
    return max(errs)


def test_window0_equals_linear_rnn():
    assert _rnn_limit_err() < 1e-12


# ---------------------------------------------------------------- invariants

MIXED = [(20, 6, 2, 16), (33, 5, 3, 32), (16, 8, 1, 8)]


@pytest.mark.parametrize("C,N,w,d", MIXED)
def test_constant_values_reproduce(C, N, w, d):
    q, k, _ = _qkv(C * N, d, 61, qs=3.0)
    v = np.tile(_rand((1, d), 62), (C * N, 1))
    np.testing.assert_allclose(O.hybrid(q, k, v, C, w), v, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("C,N,w,d", MIXED)
def test_linear_and_translation_in_values(C, N, w, d):
    q, k, v1 = _qkv(C * N, d, 71, qs=2.0)
    v2 = _rand(v1.shape, 72)
    f = lambda v: O.hybrid(q, k, v, C, w)
    np.testing.assert_allclose(f(2.5 * v1 - 0.75 * v2), 2.5 * f(v1) - 0.75 * f(v2), atol=1e-12)
    shift = _rand((1, d), 73)
    np.testing.assert_allclose(f(v1 + shift), f(v1) + shift, atol=1e-12)


@pytest.mark.parametrize("C,N,w,d", MIXED)
def test_permuting_a_chunk_permutes_only_its_rows(C, N, w, d):
    q, k, v = _qkv(C * N, d, 81, qs=2.0)
    base = O.hybrid(q, k, v, C, w)
    c = N // 2
    perm = np.arange(C * N)
    perm[c * C:(c + 1) * C] = c * C + np.random.default_rng(82).permutation(C)
    got = O.hybrid(q[perm], k[perm], v[perm], C, w)
    np.testing.assert_allclose(got, base[perm], atol=1e-12)


@pytest.mark.parametrize("C,N,w,d", MIXED)
def test_convex_hull(C, N, w, d):
    q, k, v = _qkv(C * N, d, 91, qs=3.0)
    out = O.hybrid(q, k, v, C, w)
    for i in range(0, C * N, 7):
        c = i // C
        reach = (c + 1) * C  # chunk-causal: every key up to the own chunk has a_ij > 0
        assert (out[i] <= v[:reach].max(axis=0) + 1e-12).all()
        assert (out[i] >= v[:reach].min(axis=0) - 1e-12).all()


def test_future_chunks_do_not_matter():
    C, N, w, d = 24, 5, 2, 16
    q, k, v = _qkv(C * N, d, 101)
    base = O.hybrid(q, k, v, C, w)
    k2, v2 = k.copy(), v.copy()
    k2[3 * C:] += 5.0
    v2[3 * C:] -= 7.0
    np.testing.assert_allclose(O.hybrid(q, k2, v2, C, w)[: 3 * C], base[: 3 * C], atol=0)


# ---------------------------------------------------------------- state scan

def _scan_identity_err(C=40, N=7, d=24, w=2):
    _, k, v = _qkv(C * N, d, 111)
    U, u = O.chunk_states(k, v, C)
    fk = _torch_phi(k)
    errs = [np.max(np.abs(U.sum(axis=0) - fk.T @ v)), np.max(np.abs(u.sum(axis=0) - fk.sum(axis=0)))]
    S, z = O.state_scan(k, v, C, w)
    errs.append(np.max(np.abs(S[:w])))
    errs.append(np.max(np.abs(z[:w])))
    for c in range(w, N):
        lastc = c - w
        ref = fk[: (lastc + 1) * C].T @ v[: (lastc + 1) * C]
        errs.append(np.max(np.abs(S[c] - ref)))
        errs.append(np.max(np.abs(z[c] - fk[: (lastc + 1) * C].sum(axis=0))))
    for c in range(w + 1, N):
        errs.append(np.max(np.abs(S[c] - S[c - 1] - U[c - w])))
    return max(errs)


def test_state_scan_identities():
    assert _scan_identity_err() < 1e-11


def test_state_after_matches_scan():
    C, N, d = 16, 9, 8
    _, k, v = _qkv(C * N, d, 121)
    for w in (1, 3, 9):
        S, z = O.state_scan(k, v, C, w)
        for T in range(1, N):
            sT, zT = O.state_after(k, v, C, w, T)
            np.testing.assert_allclose(sT, S[T], atol=1e-12)
            np.testing.assert_allclose(zT, z[T], atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _all_pins_err():
    return {
        "golden": _golden_max_err(),
        "brute": max(_brute_vs_chunked(C, N, w, d) for (C, N, w, d) in [(3, 6, 2, 4), (64, 4, 1, 64)]),
        "sdpa": _sdpa_limit_err(),
        "rnn": _rnn_limit_err(),
        "scan": _scan_identity_err(),
    }


MUTANTS = {
    "phi_without_plus_one": ("phi", lambda orig: (lambda x: orig(x) - 1.0)),
    "phi_linear_for_negatives": ("phi", lambda orig: (lambda x: np.asarray(x, np.float64) + 1.0)),
    "missing_score_scale": ("_scores", lambda orig: (lambda q, k: q @ k.T)),
    "score_sign_flip": ("_scores", lambda orig: (lambda q, k: -orig(q, k))),
    "window_one_chunk_short": ("window_range",
                               lambda orig: (lambda c, w: (max(0, c - w + 2), c) if w > 0 else (c + 1, c))),
    "transposed_chunk_state": ("chunk_states",
                               lambda orig: (lambda k, v, C: (np.swapaxes(orig(k, v, C)[0], 1, 2),
                                                              orig(k, v, C)[1]))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, make = MUTANTS[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    try:
        errs = _all_pins_err()
    except (OverflowError, FloatingPointError, ValueError):
        return  # the oracle refuses the mutated arithmetic outright: caught
    # NaN (a zero or negative normaliser) counts as caught
    assert any(not (e < 1e-6) for e in errs.values()), errs


def test_unmutated_pins_pass():
    errs = _all_pins_err()
    assert max(errs.values()) < 1e-11, errs


# ---------------------------------------------------------------- block-sparse window
# (explainer page of "Long-Horizon Streaming Video Generation via Hybrid
# Attention with Decoupled Distillation", section 2.A: pruned blocks of the
# local window).  The pruned definition is pinned to brute force and, through
# the all-kept and all-pruned masks, to the dense oracle and a closed form.

SPARSE_SWEEP = [
    (C, N, w, qt, kt)
    for C, N in ((3, 4), (5, 3), (6, 2), (4, 1))
    for w in (1, 2, N + 1)
    for qt, kt in ((2, 2), (3, 5), (C, 1))
]


def _mask(C, N, w, qt, kt, seed, density=0.5):
    shape = O.sparse_mask_shape(C, N, w, qt, kt)
    return (np.random.default_rng(seed).random(shape) < density).astype(np.uint8)


@pytest.mark.parametrize("C,N,w,qt,kt", SPARSE_SWEEP)
def test_block_sparse_brute_equals_chunked(C, N, w, qt, kt):
    q, k, v = _qkv(C * N, 4, 700 + 10 * C + N, qs=1.5)
    m = _mask(C, N, w, qt, kt, 7 * C + N + w)
    a, da = O.brute_block_sparse(q, k, v, C, w, m, qt, kt, return_den=True)
    b, db = O.hybrid_block_sparse(q, k, v, C, w, m, qt, kt, return_den=True)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, da, rtol=1e-12, atol=1e-300)
    rows = np.arange(0, C * N, 2)
    r, dr = O.hybrid_block_sparse_rows(q, k, v, C, w, m, rows, qtile=qt, ktile=kt, return_den=True)
    np.testing.assert_allclose(r, a[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dr, da[rows], rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("C,N,w", [(3, 4, 2), (5, 3, 1), (4, 2, 3)])
def test_block_sparse_all_kept_is_dense(C, N, w):
    q, k, v = _qkv(C * N, 4, 800 + C, qs=1.5)
    ones = np.ones(O.sparse_mask_shape(C, N, w, 2, 3), np.uint8)
    np.testing.assert_allclose(O.brute_block_sparse(q, k, v, C, w, ones, 2, 3), O.brute_masked(q, k, v, C, w),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(O.hybrid_block_sparse(q, k, v, C, w, ones, 2, 3), O.hybrid(q, k, v, C, w),
                               rtol=1e-13, atol=1e-13)


def test_block_sparse_all_pruned_is_linear_only():
    # no window key left: out = phi(q) S_c / phi(q) z_c where the history is
    # non-empty (chunks c >= w), and 0 with denominator 0 where it is empty
    C, N, w = 4, 5, 2
    q, k, v = _qkv(C * N, 3, 850)
    zeros = np.zeros(O.sparse_mask_shape(C, N, w, 2, 3), np.uint8)
    out, den = O.brute_block_sparse(q, k, v, C, w, zeros, 2, 3, return_den=True)
    fq, fk = O.phi(q), O.phi(k)
    for i in range(C * N):
        c = i // C
        if c < w:
            assert den[i] == 0 and np.all(out[i] == 0)
        else:
            hist = slice(0, (c - w + 1) * C)
            wts = fk[hist] @ fq[i]
            np.testing.assert_allclose(out[i], wts @ v[hist] / wts.sum(), rtol=1e-13)
    np.testing.assert_allclose(O.hybrid_block_sparse(q, k, v, C, w, zeros, 2, 3), out, rtol=1e-13, atol=1e-13)


def test_block_sparse_drops_exactly_the_block():
    # pruning key block j of one query block equals giving those keys zero
    # weight: the same query rows computed over the window with those keys
    # deleted (the history untouched) -- checked on the definition directly
    C, N, w, qt, kt = 6, 3, 2, 3, 4
    q, k, v = _qkv(C * N, 5, 870, qs=1.2)
    m = np.ones(O.sparse_mask_shape(C, N, w, qt, kt), np.uint8)
    c, i, j = 2, 1, 1
    m[c, i, j] = 0
    out = O.hybrid_block_sparse(q, k, v, C, w, m, qt, kt)
    lo = (c - w + 1) * C
    keys = [t for t in range(lo, (c + 1) * C) if not (lo + j * kt <= t < lo + (j + 1) * kt)]
    hist = list(range(0, lo))
    for r in range(c * C + i * qt, c * C + (i + 1) * qt):
        e = np.exp(q[r] @ k[keys].T / math.sqrt(5))
        lin = O.phi(k[hist]) @ O.phi(q[r])
        ref = (e @ v[keys] + lin @ v[hist]) / (e.sum() + lin.sum())
        np.testing.assert_allclose(out[r], ref, rtol=1e-12)


# ---------------------------------------------------------------- pruned streaming step
# (Hybrid Forcing explainer, sections 1 and 2.A: the streaming generator's KV
# cache and its block-sparse window).  The step's key blocks are counted over
# the cache slots in slot order (chunk c in slot c mod w).  Pinned to the plain
# hybrid (every block kept), to the pruned window of the whole sequence (before
# the ring turns, and with the mask rolled by the ring's turn when blocks do
# not straddle chunks), and to a pair-by-pair brute force that places each key
# by its own slot arithmetic.

def _stream_masks(C, N, w, qt, kt, seed, density=0.5):
    shape = (N, -(-C // qt), -(-(w * C) // kt))
    return (np.random.default_rng(seed).random(shape) < density).astype(np.uint8)


def _stream_brute(q, k, v, C, w, masks, qt, kt):
    L, d = q.shape
    out, den = np.zeros((L, v.shape[1])), np.zeros(L)
    for i in range(L):
        t = i // C
        fq = O.phi(q[i])
        num, dsum = np.zeros(v.shape[1]), 0.0
        for j in range(L):
            c = j // C
            if max(0, t - w + 1) <= c <= t:
                slot = c % w                      # the chunk's cache slot
                pos = slot * C + (j - c * C)      # its key's row in slot order
                if masks[t, (i - t * C) // qt, pos // kt]:
                    a = math.exp(q[i] @ k[j] / math.sqrt(d))
                    num, dsum = num + a * v[j], dsum + a
            elif c <= t - w:
                a = fq @ O.phi(k[j])
                num, dsum = num + a * v[j], dsum + a
        den[i] = dsum
        out[i] = num / dsum if dsum > 0 else 0.0
    return out, den


STREAM_SPARSE_SWEEP = [(3, 5, 2, 2, 2), (4, 6, 3, 3, 5), (5, 4, 1, 5, 1), (2, 7, 3, 1, 3), (4, 5, 4, 2, 4)]


@pytest.mark.parametrize("C,N,w,qt,kt", STREAM_SPARSE_SWEEP)
def test_stream_sparse_matches_pair_brute_force(C, N, w, qt, kt):
    q, k, v = _qkv(C * N, 4, 6000 + 10 * C + N, qs=1.5)
    m = _stream_masks(C, N, w, qt, kt, 6001 + C + w)
    a, da = _stream_brute(q, k, v, C, w, m, qt, kt)
    b, db = O.stream_block_sparse(q, k, v, C, w, m, qt, kt, return_den=True)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, da, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("C,N,w,qt,kt", STREAM_SPARSE_SWEEP)
def test_stream_sparse_all_kept_is_plain_hybrid(C, N, w, qt, kt):
    q, k, v = _qkv(C * N, 4, 6100 + C, qs=1.5)
    ones = np.ones((N, -(-C // qt), -(-(w * C) // kt)), np.uint8)
    np.testing.assert_allclose(O.stream_block_sparse(q, k, v, C, w, ones, qt, kt), O.hybrid(q, k, v, C, w),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C,N,w,qt,kt", STREAM_SPARSE_SWEEP)
def test_stream_sparse_before_the_ring_turns_is_the_pruned_window(C, N, w, qt, kt):
    # steps t < w: slots 0 .. t hold chunks 0 .. t in order, the whole-sequence
    # window order
    q, k, v = _qkv(C * N, 4, 6200 + C, qs=1.5)
    m = _stream_masks(C, N, w, qt, kt, 6201 + N)
    nkt_seq = O.sparse_mask_shape(C, N, w, qt, kt)[2]
    ref = O.hybrid_block_sparse(q, k, v, C, w, m[:, :, :nkt_seq], qt, kt)
    got = O.stream_block_sparse(q, k, v, C, w, m, qt, kt)
    n = min(w, N) * C
    np.testing.assert_allclose(got[:n], ref[:n], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C,N,w,kt", [(4, 7, 3, 2), (6, 6, 2, 3), (4, 5, 4, 4), (2, 6, 3, 1)])
def test_stream_sparse_turned_ring_is_the_pruned_window_with_a_rolled_mask(C, N, w, kt):
    # with C a multiple of the key block, chronological window block i*m + u
    # (chunk first + i, block u of m = C/kt) is slot-order block
    # ((first + i) mod w) * m + u
    assert C % kt == 0
    qt, m_ = 2, C // kt
    q, k, v = _qkv(C * N, 4, 6300 + C + w, qs=1.5)
    ms = _stream_masks(C, N, w, qt, kt, 6301 + w)
    nkt_seq = O.sparse_mask_shape(C, N, w, qt, kt)[2]
    mc = np.zeros((N, ms.shape[1], nkt_seq), np.uint8)
    for t in range(N):
        first = max(0, t - w + 1)
        for i in range(t - first + 1):
            for u in range(m_):
                mc[t, :, i * m_ + u] = ms[t, :, ((first + i) % w) * m_ + u]
    np.testing.assert_allclose(O.stream_block_sparse(q, k, v, C, w, ms, qt, kt),
                               O.hybrid_block_sparse(q, k, v, C, w, mc, qt, kt), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C,N,w,qt,kt", STREAM_SPARSE_SWEEP)
def test_stream_sparse_rows_match_whole_stream(C, N, w, qt, kt):
    q, k, v = _qkv(C * N, 4, 6600 + C, qs=1.5)
    m = _stream_masks(C, N, w, qt, kt, 6601 + w)
    full = O.stream_block_sparse(q, k, v, C, w, m, qt, kt)
    for t in range(N):
        rows = np.arange(0, C, 2)
        got = O.stream_block_sparse_rows(q, k, v, C, w, t, m[t], rows, qtile=qt, ktile=kt)
        np.testing.assert_allclose(got, full[t * C + rows], rtol=1e-13, atol=1e-13)


def test_stream_sparse_all_pruned_leaves_the_history():
    C, N, w, qt, kt = 3, 5, 2, 2, 2
    q, k, v = _qkv(C * N, 3, 6400)
    zeros = np.zeros((N, 2, 3), np.uint8)
    out, den = O.stream_block_sparse(q, k, v, C, w, zeros, qt, kt, return_den=True)
    assert np.all(den[: w * C] == 0) and np.all(out[: w * C] == 0)
    fq, fk = O.phi(q), O.phi(k)
    for i in range(w * C, C * N):
        hist = slice(0, (i // C - w + 1) * C)
        wts = fk[hist] @ fq[i]
        np.testing.assert_allclose(out[i], wts @ v[hist] / wts.sum(), rtol=1e-13)


def _stream_sparse_pin_err():
    C, N, w, qt, kt = 3, 6, 3, 2, 2
    q, k, v = _qkv(C * N, 4, 6500, qs=1.2)
    m = _stream_masks(C, N, w, qt, kt, 6501)
    a, _ = _stream_brute(q, k, v, C, w, m, qt, kt)
    return float(np.max(np.abs(O.stream_block_sparse(q, k, v, C, w, m, qt, kt) - a)))


STREAM_SPARSE_MUTANTS = {
    "chronological_order": ("stream_slot_chunks",
                            lambda orig: (lambda t, w: list(range(max(0, t - w + 1), t + 1)))),
    "mask_ignored": ("_window_keep", lambda orig: (lambda row, n, kt: np.ones(n, dtype=bool))),
    "mask_one_tile_late": ("_window_keep", lambda orig: (lambda row, n, kt: np.roll(orig(row, n, kt), kt))),
}


@pytest.mark.parametrize("name", sorted(STREAM_SPARSE_MUTANTS))
def test_stream_sparse_planted_mistake_is_caught(name, monkeypatch):
    attr, make = STREAM_SPARSE_MUTANTS[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    assert _stream_sparse_pin_err() > 1e-6


def test_stream_sparse_unmutated_pin_passes():
    assert _stream_sparse_pin_err() < 1e-10


# ---------------------------------------------------------------- bidirectional hybrid
# (ReHyAt abstract: the hybrid stands in for the bidirectional attention of
# video diffusion transformers).  Reading: symmetric window, everything outside
# it -- past and future -- in the linear term.  Pinned to brute force, to
# unmasked SDPA when the window covers every chunk, to non-causal linear
# attention (the token RNN's final state) at w = 0, to the causal hybrid on the
# last chunk, to time reversal, and by a scan identity.

BIDIR_SWEEP = [(C, N, w, d) for C, N in ((1, 7), (3, 4), (5, 3), (16, 5)) for w in (0, 1, 2, 3, N + 1)
               for d in (4, 32)]


@pytest.mark.parametrize("C,N,w,d", BIDIR_SWEEP)
def test_bidir_brute_equals_chunked(C, N, w, d):
    q, k, v = _qkv(C * N, d, 900 + 10 * C + N + w, qs=1.5)
    a, da = O.brute_bidir(q, k, v, C, w, return_den=True)
    b, db = O.hybrid_bidir(q, k, v, C, w, return_den=True)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, da, rtol=1e-12)
    rows = np.arange(0, C * N, 3)
    r, dr = O.hybrid_bidir_rows(q, k, v, C, w, rows, return_den=True)
    np.testing.assert_allclose(r, a[rows], rtol=1e-12, atol=1e-12)


def test_bidir_window_all_is_unmasked_sdpa():
    C, N = 24, 5
    q, k, v = _qkv(C * N, 32, 910, qs=2.0)
    ref = _sdpa(q, k, v)
    for w in (N, N + 2):
        np.testing.assert_allclose(O.hybrid_bidir(q, k, v, C, w), ref, atol=1e-12)
        np.testing.assert_allclose(O.brute_bidir(q, k, v, C, w), ref, atol=1e-12)


def test_bidir_window0_is_noncausal_linear_attention():
    # the token-by-token recurrence with one "chunk" spanning the whole
    # sequence absorbs every token before any query reads the state: plain
    # non-causal linear attention
    for C, N in ((1, 40), (6, 5)):
        q, k, v = _qkv(C * N, 8, 920 + C)
        ref = _linear_rnn(q, k, v, C * N)
        np.testing.assert_allclose(O.hybrid_bidir(q, k, v, C, 0), ref, rtol=1e-12)
        np.testing.assert_allclose(O.brute_bidir(q, k, v, C, 0), ref, rtol=1e-12)


def test_bidir_last_chunk_equals_causal():
    C, N = 7, 6
    q, k, v = _qkv(C * N, 16, 930, qs=1.5)
    last = slice((N - 1) * C, N * C)
    for w in (0, 1, 2, 4):
        np.testing.assert_allclose(O.hybrid_bidir(q, k, v, C, w)[last], O.hybrid(q, k, v, C, w)[last], rtol=1e-12)


def test_bidir_time_reversal():
    C, N = 5, 6
    q, k, v = _qkv(C * N, 8, 940, qs=1.5)
    for w in (0, 1, 2, 3):
        fwd = O.hybrid_bidir(q, k, v, C, w)
        rev = O.hybrid_bidir(q[::-1].copy(), k[::-1].copy(), v[::-1].copy(), C, w)
        np.testing.assert_allclose(rev[::-1], fwd, rtol=1e-12)


def test_bidir_scan_identity():
    # past + future + window contributions = the whole sequence's phi(K)^T V, for every chunk
    C, N = 4, 7
    _, k, v = _qkv(C * N, 6, 950)
    U, u = O.chunk_states(k, v, C)
    tot = O.phi(k).T @ v
    for w in (0, 1, 2, 5, 9):
        Sp, zp, Ss, zs = O.state_scan_bidir(k, v, C, w)
        for c in range(N):
            lo, hi = O.window_range_bidir(c, w, N)
            win = U[lo:hi + 1].sum(axis=0) if lo <= hi else 0.0
            np.testing.assert_allclose(Sp[c] + Ss[c] + win, tot, rtol=1e-12, atol=1e-12)
            if w == 0:
                np.testing.assert_allclose(Sp[c], U[: c + 1].sum(axis=0), rtol=1e-12)


# ---------------------------------------------------------------- anchor (sink) chunks
# (Hybrid Forcing explainer, section 1: the attention-sink workaround keeps the
# first frame attended).  The first `a` chunks are always in the softmax window
# of the queries they do not lie in the future of, and never in the state.

ANCHOR_SWEEP = [(C, N, w, a) for C, N in ((1, 8), (3, 5), (4, 4), (7, 3)) for w in (0, 1, 2, N + 1)
                for a in (0, 1, 2, N)]


@pytest.mark.parametrize("C,N,w,a", ANCHOR_SWEEP)
def test_anchor_brute_equals_chunked(C, N, w, a):
    q, k, v = _qkv(C * N, 6, 1000 + 10 * C + N + w + 100 * a, qs=1.5)
    x, dx = O.brute_anchor(q, k, v, C, w, a, return_den=True)
    y, dy = O.hybrid_anchor(q, k, v, C, w, a, return_den=True)
    np.testing.assert_allclose(y, x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dy, dx, rtol=1e-12)
    rows = np.arange(1, C * N, 2)
    r = O.hybrid_anchor_rows(q, k, v, C, w, a, rows)
    np.testing.assert_allclose(r, x[rows], rtol=1e-12, atol=1e-12)


def test_anchor_zero_is_plain_hybrid():
    C, N = 5, 6
    q, k, v = _qkv(C * N, 8, 1100, qs=1.5)
    for w in (0, 1, 2, 3):
        np.testing.assert_allclose(O.hybrid_anchor(q, k, v, C, w, 0), O.hybrid(q, k, v, C, w), rtol=1e-13)
        np.testing.assert_allclose(O.brute_anchor(q, k, v, C, w, 0), O.brute_masked(q, k, v, C, w), rtol=1e-13)


def test_all_chunks_anchored_is_block_causal_sdpa():
    # every chunk an anchor (or a window covering all): all of the causal past in the softmax
    C, N = 16, 4
    q, k, v = _qkv(C * N, 32, 1110, qs=2.0)
    ref = _sdpa(q, k, v, _block_causal(C * N, C))
    for w, a in ((0, N), (1, N), (2, N + 3), (N, 1)):
        np.testing.assert_allclose(O.hybrid_anchor(q, k, v, C, w, a), ref, atol=1e-12)
        np.testing.assert_allclose(O.brute_anchor(q, k, v, C, w, a), ref, atol=1e-12)


def test_anchor_state_is_plain_state_without_anchor_chunks():
    C, N = 4, 7
    _, k, v = _qkv(C * N, 5, 1120)
    U, u = O.chunk_states(k, v, C)
    for w in (0, 1, 2):
        S0, z0 = O.state_scan(k, v, C, w)
        for a in (1, 2, 3):
            S, z = O.state_scan_anchor(k, v, C, w, a)
            for c in range(N):
                hi = min(a - 1, c - w)  # anchors the plain state would hold
                dropped = U[: hi + 1].sum(axis=0) if hi >= 0 else 0.0
                dz = u[: hi + 1].sum(axis=0) if hi >= 0 else 0.0
                np.testing.assert_allclose(S[c], S0[c] - dropped, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(z[c], z0[c] - dz, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward pass
# The chain-rule gradients are pinned to central finite differences of the
# forward oracle along random directions, and to torch autograd through a
# separately written dense (L x L) torch form of the definition.

def _loss(q, k, v, C, w, dout):
    return float((O.hybrid(q, k, v, C, w) * dout).sum())


@pytest.mark.parametrize("C,N,w", [(3, 4, 2), (5, 3, 1), (4, 4, 0), (2, 5, 9), (6, 3, 3)])
def test_backward_matches_finite_differences(C, N, w):
    d = 5
    q, k, v = _qkv(C * N, d, 1200 + C * N + w, qs=1.2)
    dout = _rand((C * N, d), 1300 + w)
    dq, dk, dv = O.hybrid_backward(q, k, v, C, w, dout)
    rng = np.random.default_rng(1400 + C)
    eps = 1e-5
    for which, g in ((0, dq), (1, dk), (2, dv)):
        for _ in range(3):
            dirn = rng.standard_normal(q.shape)
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which] += eps * dirn
            args_m[which] -= eps * dirn
            fd = (_loss(*args_p, C, w, dout) - _loss(*args_m, C, w, dout)) / (2 * eps)
            an = float((g * dirn).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def _torch_dense_hybrid(q, k, v, C, w):
    """The definition as a dense masked L x L weight matrix, in torch ops."""
    L, d = q.shape
    c = torch.arange(L) // C
    cq, ck = c[:, None], c[None, :]
    win = ((ck <= cq) & (ck >= cq - w + 1)) if w > 0 else torch.zeros((L, L), dtype=torch.bool)
    hist = ck <= cq - w
    s = q @ k.T / math.sqrt(d)
    lin = (torch.nn.functional.elu(q) + 1) @ (torch.nn.functional.elu(k) + 1).T
    a = torch.where(win, torch.exp(s), torch.where(hist, lin, torch.zeros_like(s)))
    return (a @ v) / a.sum(dim=1, keepdim=True)


@pytest.mark.parametrize("C,N,w", [(4, 5, 2), (7, 3, 1), (3, 4, 0), (5, 4, 6)])
def test_backward_matches_torch_autograd(C, N, w):
    d = 8
    q, k, v = _qkv(C * N, d, 1500 + C + w, qs=1.5)
    dout = _rand((C * N, d), 1600 + N)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_hybrid(tq, tk, tv, C, w) * torch.from_numpy(dout)).sum().backward()
    dq, dk, dv = O.hybrid_backward(q, k, v, C, w, dout)
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_dphi_closed_form():
    x = np.array([-3.0, -1e-3, 0.0, 1e-3, 2.0])
    np.testing.assert_allclose(O.dphi(x), [math.exp(-3.0), math.exp(-1e-3), 1.0, 1.0, 1.0], rtol=1e-15)


@pytest.mark.parametrize("C,N,w", [(6, 4, 4), (5, 3, 7), (1, 23, 23)])
def test_backward_window_all_equals_sdpa_gradient(C, N, w):
    """A window covering every chunk is block-causal softmax attention: the
    oracle's gradients equal torch autograd through fp64 SDPA with that mask."""
    d = 16
    q, k, v = _qkv(C * N, d, 1700 + C + N, qs=1.5)
    dout = _rand((C * N, d), 1800 + C)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True)[None, None] for x in (q, k, v))
    for t in (tq, tk, tv):
        t.retain_grad()
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=_block_causal(C * N, C))
    (o[0, 0] * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_backward(q, k, v, C, w, dout), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref[0, 0].numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("C,N", [(1, 30), (4, 6)])
def test_backward_window0_equals_linear_attention_gradient(C, N):
    """w = 0 is causal linear attention (the state includes the own chunk):
    the oracle's gradients equal torch autograd through a cumulative-sum form."""
    d = 6
    q, k, v = _qkv(C * N, d, 1900 + C, qs=1.2)
    dout = _rand((C * N, d), 2000 + C)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    fq = torch.nn.functional.elu(tq) + 1
    fk = torch.nn.functional.elu(tk) + 1
    kv = torch.cumsum(fk[:, :, None] * tv[:, None, :], dim=0)  # [L, d, d]: running sum of phi(k) v^T
    ks = torch.cumsum(fk, dim=0)
    last = (torch.arange(C * N) // C) * C + C - 1  # each row reads the state after its chunk's last token
    o = torch.einsum("ld,lde->le", fq, kv[last]) / (fq * ks[last]).sum(dim=1, keepdim=True)
    (o * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_backward(q, k, v, C, 0, dout), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


def _backward_pin_errs():
    """Largest deviation of the oracle's gradients from (a) finite differences
    of its own forward and (b) torch autograd through the dense form."""
    C, N, w, d = 3, 4, 2, 5
    q, k, v = _qkv(C * N, d, 2100, qs=1.2)
    dout = _rand((C * N, d), 2101)
    grads = O.hybrid_backward(q, k, v, C, w, dout)
    rng = np.random.default_rng(2102)
    fd_err = 0.0
    for which, g in enumerate(grads):
        dirn = rng.standard_normal(q.shape)
        ap, am = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
        ap[which] += 1e-5 * dirn
        am[which] -= 1e-5 * dirn
        fd = (_loss(*ap, C, w, dout) - _loss(*am, C, w, dout)) / 2e-5
        fd_err = max(fd_err, abs(fd - float((g * dirn).sum())))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_hybrid(tq, tk, tv, C, w) * torch.from_numpy(dout)).sum().backward()
    ag_err = max(float(np.max(np.abs(g - t.grad.numpy()))) for g, t in zip(grads, (tq, tk, tv)))
    return fd_err, ag_err


BACKWARD_MUTANTS = {
    "dphi_constant_one": ("dphi", lambda orig: (lambda x: np.ones_like(np.asarray(x, np.float64)))),
    "dphi_of_phi": ("dphi", lambda orig: (lambda x: orig(x) + 0.5 * (np.asarray(x) < 0))),
    "window_one_chunk_short": ("window_range",
                               lambda orig: (lambda c, w: (max(0, c - w + 2), c) if w > 0 else (c + 1, c))),
    "score_sign_flip": ("_scores", lambda orig: (lambda q, k: -orig(q, k))),
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_planted_mistake_is_caught(name, monkeypatch):
    attr, make = BACKWARD_MUTANTS[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    assert max(_backward_pin_errs()) > 1e-6


def test_backward_unmutated_pins_pass():
    assert max(_backward_pin_errs()) < 1e-8


# ------------------------------------------------- backward pass, bidirectional
# ``hybrid_bidir_backward`` is pinned like the causal one: central finite
# differences of the bidirectional forward oracle, torch autograd through a
# separately written dense form, and the two limits with a known gradient
# (a window covering every chunk is unmasked softmax attention; w = 0 is
# non-causal linear attention).

def _loss_bidir(q, k, v, C, w, dout):
    return float((O.hybrid_bidir(q, k, v, C, w) * dout).sum())


def _torch_dense_bidir(q, k, v, C, w):
    """The bidirectional definition as a dense L x L weight matrix, in torch ops."""
    L, d = q.shape
    c = torch.arange(L) // C
    win = ((c[None, :] - c[:, None]).abs() <= w - 1) if w > 0 else torch.zeros((L, L), dtype=torch.bool)
    s = q @ k.T / math.sqrt(d)
    lin = (torch.nn.functional.elu(q) + 1) @ (torch.nn.functional.elu(k) + 1).T
    a = torch.where(win, torch.exp(s), lin)
    return (a @ v) / a.sum(dim=1, keepdim=True)


@pytest.mark.parametrize("C,N,w", [(3, 5, 2), (5, 3, 1), (4, 4, 0), (2, 5, 9), (3, 6, 3)])
def test_bidir_backward_matches_finite_differences(C, N, w):
    d = 5
    q, k, v = _qkv(C * N, d, 2200 + C * N + w, qs=1.2)
    dout = _rand((C * N, d), 2300 + w)
    grads = O.hybrid_bidir_backward(q, k, v, C, w, dout)
    rng = np.random.default_rng(2400 + C)
    eps = 1e-5
    for which, g in enumerate(grads):
        for _ in range(3):
            dirn = rng.standard_normal(q.shape)
            ap, am = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
            ap[which] += eps * dirn
            am[which] -= eps * dirn
            fd = (_loss_bidir(*ap, C, w, dout) - _loss_bidir(*am, C, w, dout)) / (2 * eps)
            an = float((g * dirn).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("C,N,w", [(4, 5, 2), (7, 3, 1), (3, 4, 0), (5, 4, 6), (2, 7, 3)])
def test_bidir_backward_matches_torch_autograd(C, N, w):
    d = 8
    q, k, v = _qkv(C * N, d, 2500 + C + w, qs=1.5)
    dout = _rand((C * N, d), 2600 + N)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_bidir(tq, tk, tv, C, w) * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_bidir_backward(q, k, v, C, w, dout), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("C,N,w", [(6, 4, 4), (5, 3, 7)])
def test_bidir_backward_window_all_equals_unmasked_sdpa_gradient(C, N, w):
    d = 16
    q, k, v = _qkv(C * N, d, 2700 + C + N, qs=1.5)
    dout = _rand((C * N, d), 2800 + C)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True)[None, None] for x in (q, k, v))
    for t in (tq, tk, tv):
        t.retain_grad()
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    (o[0, 0] * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_bidir_backward(q, k, v, C, w, dout), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref[0, 0].numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("C,N", [(1, 12), (4, 5)])
def test_bidir_backward_window0_equals_noncausal_linear_attention_gradient(C, N):
    d = 6
    q, k, v = _qkv(C * N, d, 2900 + C, qs=1.2)
    dout = _rand((C * N, d), 3000 + C)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    fq = torch.nn.functional.elu(tq) + 1
    fk = torch.nn.functional.elu(tk) + 1
    o = (fq @ (fk.T @ tv)) / (fq @ fk.sum(dim=0))[:, None]
    (o * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_bidir_backward(q, k, v, C, 0, dout), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


def _bidir_backward_pin_errs():
    C, N, w, d = 3, 5, 2, 5
    q, k, v = _qkv(C * N, d, 3100, qs=1.2)
    dout = _rand((C * N, d), 3101)
    grads = O.hybrid_bidir_backward(q, k, v, C, w, dout)
    rng = np.random.default_rng(3102)
    fd_err = 0.0
    for which, g in enumerate(grads):
        dirn = rng.standard_normal(q.shape)
        ap, am = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
        ap[which] += 1e-5 * dirn
        am[which] -= 1e-5 * dirn
        fd = (_loss_bidir(*ap, C, w, dout) - _loss_bidir(*am, C, w, dout)) / 2e-5
        fd_err = max(fd_err, abs(fd - float((g * dirn).sum())))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_bidir(tq, tk, tv, C, w) * torch.from_numpy(dout)).sum().backward()
    ag_err = max(float(np.max(np.abs(g - t.grad.numpy()))) for g, t in zip(grads, (tq, tk, tv)))
    return fd_err, ag_err


def _future_one_chunk_late(orig):
    def scan(k, v, C, w):
        S_pre, z_pre, S_suf, z_suf = orig(k, v, C, w)
        U, u = O.chunk_states(k, v, C)
        N = U.shape[0]
        first = max(w, 1)
        for c in range(N):  # drop the nearest future chunk from every future state
            if c + first <= N - 1:
                S_suf[c] = S_suf[c] - U[c + first]
                z_suf[c] = z_suf[c] - u[c + first]
        return S_pre, z_pre, S_suf, z_suf
    return scan


BIDIR_BACKWARD_MUTANTS = {
    "dphi_constant_one": ("dphi", lambda orig: (lambda x: np.ones_like(np.asarray(x, np.float64)))),
    "window_one_chunk_short": ("window_range_bidir",
                               lambda orig: (lambda c, w, N: (max(0, c - w + 2), min(N - 1, c + w - 1)) if w > 0
                                             else (c + 1, c))),
    "future_state_one_chunk_late": ("state_scan_bidir", _future_one_chunk_late),
    "score_sign_flip": ("_scores", lambda orig: (lambda q, k: -orig(q, k))),
}


@pytest.mark.parametrize("name", sorted(BIDIR_BACKWARD_MUTANTS))
def test_bidir_backward_planted_mistake_is_caught(name, monkeypatch):
    attr, make = BIDIR_BACKWARD_MUTANTS[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    assert max(_bidir_backward_pin_errs()) > 1e-6


def test_bidir_backward_unmutated_pins_pass():
    assert max(_bidir_backward_pin_errs()) < 1e-8


# ------------------------------------------------------ backward pass, anchored
# ``hybrid_anchor_backward`` is pinned to finite differences of the anchored
# forward, torch autograd through a separately written dense anchored form,
# the plain backward at a = 0, and block-causal SDPA autograd when every chunk
# is an anchor.

def _loss_anchor(q, k, v, C, w, a, dout):
    return float((O.hybrid_anchor(q, k, v, C, w, a) * dout).sum())


def _torch_dense_anchor(q, k, v, C, w, a):
    """The anchored definition as a dense masked L x L weight matrix, in torch ops."""
    L, d = q.shape
    c = torch.arange(L) // C
    cq, ck = c[:, None], c[None, :]
    win = ((ck <= cq) & (ck >= cq - w + 1)) if w > 0 else torch.zeros((L, L), dtype=torch.bool)
    win = win | ((ck < a) & (ck <= cq))
    hist = (ck >= a) & (ck <= cq - w) & ~win
    s = q @ k.T / math.sqrt(d)
    lin = (torch.nn.functional.elu(q) + 1) @ (torch.nn.functional.elu(k) + 1).T
    wts = torch.where(win, torch.exp(s), torch.where(hist, lin, torch.zeros_like(s)))
    return (wts @ v) / wts.sum(dim=1, keepdim=True)


@pytest.mark.parametrize("C,N,w,a", [(3, 5, 2, 1), (4, 4, 1, 2), (3, 5, 0, 1), (2, 6, 2, 3), (3, 4, 5, 1)])
def test_anchor_backward_matches_finite_differences(C, N, w, a):
    d = 5
    q, k, v = _qkv(C * N, d, 3200 + C * N + w + a, qs=1.2)
    dout = _rand((C * N, d), 3300 + w + a)
    grads = O.hybrid_anchor_backward(q, k, v, C, w, a, dout)
    rng = np.random.default_rng(3400 + C + a)
    eps = 1e-5
    for which, g in enumerate(grads):
        for _ in range(3):
            dirn = rng.standard_normal(q.shape)
            ap, am = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
            ap[which] += eps * dirn
            am[which] -= eps * dirn
            fd = (_loss_anchor(*ap, C, w, a, dout) - _loss_anchor(*am, C, w, a, dout)) / (2 * eps)
            an = float((g * dirn).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("C,N,w,a", [(4, 5, 2, 1), (3, 6, 1, 2), (3, 4, 0, 2), (2, 7, 3, 3), (5, 3, 2, 5)])
def test_anchor_backward_matches_torch_autograd(C, N, w, a):
    d = 8
    q, k, v = _qkv(C * N, d, 3500 + C + w + a, qs=1.5)
    dout = _rand((C * N, d), 3600 + N)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_anchor(tq, tk, tv, C, w, a) * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_anchor_backward(q, k, v, C, w, a, dout), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("C,N,w", [(3, 5, 2), (4, 4, 0), (2, 5, 9)])
def test_anchor_backward_zero_anchors_is_plain_backward(C, N, w):
    d = 6
    q, k, v = _qkv(C * N, d, 3700 + C + w, qs=1.2)
    dout = _rand((C * N, d), 3800 + w)
    for ours, ref in zip(O.hybrid_anchor_backward(q, k, v, C, w, 0, dout), O.hybrid_backward(q, k, v, C, w, dout)):
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C,N,w", [(4, 5, 1), (3, 4, 0)])
def test_anchor_backward_all_anchored_equals_block_causal_sdpa_gradient(C, N, w):
    d = 16
    q, k, v = _qkv(C * N, d, 3900 + C + N, qs=1.5)
    dout = _rand((C * N, d), 4000 + C)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True)[None, None] for x in (q, k, v))
    for t in (tq, tk, tv):
        t.retain_grad()
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=_block_causal(C * N, C))
    (o[0, 0] * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_anchor_backward(q, k, v, C, w, N, dout), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref[0, 0].numpy(), rtol=1e-10, atol=1e-12)


def _anchor_backward_pin_errs():
    C, N, w, a, d = 3, 5, 2, 1, 5
    q, k, v = _qkv(C * N, d, 4100, qs=1.2)
    dout = _rand((C * N, d), 4101)
    grads = O.hybrid_anchor_backward(q, k, v, C, w, a, dout)
    rng = np.random.default_rng(4102)
    fd_err = 0.0
    for which, g in enumerate(grads):
        dirn = rng.standard_normal(q.shape)
        ap, am = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
        ap[which] += 1e-5 * dirn
        am[which] -= 1e-5 * dirn
        fd = (_loss_anchor(*ap, C, w, a, dout) - _loss_anchor(*am, C, w, a, dout)) / 2e-5
        fd_err = max(fd_err, abs(fd - float((g * dirn).sum())))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_anchor(tq, tk, tv, C, w, a) * torch.from_numpy(dout)).sum().backward()
    ag_err = max(float(np.max(np.abs(g - t.grad.numpy()))) for g, t in zip(grads, (tq, tk, tv)))
    return fd_err, ag_err


ANCHOR_BACKWARD_MUTANTS = {
    "dphi_constant_one": ("dphi", lambda orig: (lambda x: np.ones_like(np.asarray(x, np.float64)))),
    "anchors_dropped_from_keys": ("anchor_keys",
                                  lambda orig: (lambda c, C, w, a: orig(c, C, w, 0))),
    "anchors_folded_into_state": ("state_scan_anchor", lambda orig: (lambda k, v, C, w, a: orig(k, v, C, w, 0))),
    "score_sign_flip": ("_scores", lambda orig: (lambda q, k: -orig(q, k))),
}


@pytest.mark.parametrize("name", sorted(ANCHOR_BACKWARD_MUTANTS))
def test_anchor_backward_planted_mistake_is_caught(name, monkeypatch):
    attr, make = ANCHOR_BACKWARD_MUTANTS[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    assert max(_anchor_backward_pin_errs()) > 1e-6


def test_anchor_backward_unmutated_pins_pass():
    assert max(_anchor_backward_pin_errs()) < 1e-8


# -------------------------------------------------- backward pass, pruned window
# ``hybrid_block_sparse_backward`` is pinned to finite differences of the
# pruned forward, torch autograd through a separately written dense masked
# form, the plain backward when every block is kept, and zero gradients for
# rows left with no weight.

def _loss_sparse(q, k, v, C, w, m, qt, kt, dout):
    return float((O.hybrid_block_sparse(q, k, v, C, w, m, qt, kt) * dout).sum())


def _torch_dense_sparse(q, k, v, C, w, m, qt, kt):
    """The pruned definition as a dense L x L weight matrix, in torch ops."""
    L, d = q.shape
    idx = torch.arange(L)
    c = idx // C
    cq, ck = c[:, None], c[None, :]
    lo = torch.clamp(cq - w + 1, min=0)
    win = ((ck <= cq) & (ck >= lo)) if w > 0 else torch.zeros((L, L), dtype=torch.bool)
    qblk = ((idx - c * C) // qt)[:, None].expand(L, L)
    kblk = torch.clamp(idx[None, :] - lo * C, min=0) // kt
    mt = torch.from_numpy(np.asarray(m)).bool()
    keep = mt[cq.expand(L, L), qblk, torch.clamp(kblk, max=mt.shape[2] - 1)]
    hist = ck <= cq - w
    s = q @ k.T / math.sqrt(d)
    lin = (torch.nn.functional.elu(q) + 1) @ (torch.nn.functional.elu(k) + 1).T
    wts = torch.where(win & keep, torch.exp(s), torch.where(hist, lin, torch.zeros_like(s)))
    den = wts.sum(dim=1, keepdim=True)
    out = (wts @ v) / torch.where(den > 0, den, torch.ones_like(den))
    return torch.where(den > 0, out, torch.zeros_like(out))


SPARSE_BWD = [(3, 4, 2, 2, 2), (5, 3, 1, 3, 5), (4, 4, 3, 2, 3), (4, 5, 2, 4, 4)]


@pytest.mark.parametrize("C,N,w,qt,kt", SPARSE_BWD)
def test_sparse_backward_matches_finite_differences(C, N, w, qt, kt):
    d = 5
    q, k, v = _qkv(C * N, d, 4200 + C * N + w, qs=1.2)
    m = _mask(C, N, w, qt, kt, 4300 + C + w, density=0.6)
    dout = _rand((C * N, d), 4400 + w)
    grads = O.hybrid_block_sparse_backward(q, k, v, C, w, m, dout, qt, kt)
    rng = np.random.default_rng(4500 + C)
    eps = 1e-5
    for which, g in enumerate(grads):
        for _ in range(3):
            dirn = rng.standard_normal(q.shape)
            ap, am = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
            ap[which] += eps * dirn
            am[which] -= eps * dirn
            fd = (_loss_sparse(*ap, C, w, m, qt, kt, dout) - _loss_sparse(*am, C, w, m, qt, kt, dout)) / (2 * eps)
            an = float((g * dirn).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("C,N,w,qt,kt", SPARSE_BWD)
def test_sparse_backward_matches_torch_autograd(C, N, w, qt, kt):
    d = 8
    q, k, v = _qkv(C * N, d, 4600 + C + w, qs=1.5)
    m = _mask(C, N, w, qt, kt, 4700 + C + w, density=0.5)
    dout = _rand((C * N, d), 4800 + N)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_sparse(tq, tk, tv, C, w, m, qt, kt) * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip(O.hybrid_block_sparse_backward(q, k, v, C, w, m, dout, qt, kt), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("C,N,w", [(3, 4, 2), (5, 3, 1), (4, 2, 3)])
def test_sparse_backward_all_kept_is_plain_backward(C, N, w):
    d = 6
    q, k, v = _qkv(C * N, d, 4900 + C, qs=1.2)
    ones = np.ones(O.sparse_mask_shape(C, N, w, 2, 3), np.uint8)
    dout = _rand((C * N, d), 5000 + C)
    for ours, ref in zip(O.hybrid_block_sparse_backward(q, k, v, C, w, ones, dout, 2, 3),
                         O.hybrid_backward(q, k, v, C, w, dout)):
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_sparse_backward_rows_without_weight_have_zero_gradient():
    # every block pruned: chunks c < w have no weight at all (out = 0), so
    # their queries get no gradient and nothing reaches keys through them
    C, N, w, d = 4, 4, 2, 5
    q, k, v = _qkv(C * N, d, 5100)
    zeros = np.zeros(O.sparse_mask_shape(C, N, w, 2, 3), np.uint8)
    dout = _rand((C * N, d), 5101)
    dq, dk, dv = O.hybrid_block_sparse_backward(q, k, v, C, w, zeros, dout, 2, 3)
    assert np.all(dq[: w * C] == 0)
    # the rest is the gradient of the linear-only form, checked by autograd
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_sparse(tq, tk, tv, C, w, zeros, 2, 3) * torch.from_numpy(dout)).sum().backward()
    for ours, ref in zip((dq, dk, dv), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


def _sparse_backward_pin_err():
    C, N, w, qt, kt, d = 4, 4, 2, 2, 3, 5
    q, k, v = _qkv(C * N, d, 5200, qs=1.2)
    m = _mask(C, N, w, qt, kt, 5201, density=0.5)
    dout = _rand((C * N, d), 5202)
    grads = O.hybrid_block_sparse_backward(q, k, v, C, w, m, dout, qt, kt)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    (_torch_dense_sparse(tq, tk, tv, C, w, m, qt, kt) * torch.from_numpy(dout)).sum().backward()
    return max(float(np.max(np.abs(g - t.grad.numpy()))) for g, t in zip(grads, (tq, tk, tv)))


SPARSE_BACKWARD_MUTANTS = {
    "mask_ignored": ("_window_keep", lambda orig: (lambda row, n, kt: np.ones(n, dtype=bool))),
    "mask_one_tile_late": ("_window_keep",
                           lambda orig: (lambda row, n, kt: np.roll(orig(row, n, kt), kt))),
    "dphi_constant_one": ("dphi", lambda orig: (lambda x: np.ones_like(np.asarray(x, np.float64)))),
}


@pytest.mark.parametrize("name", sorted(SPARSE_BACKWARD_MUTANTS))
def test_sparse_backward_planted_mistake_is_caught(name, monkeypatch):
    attr, make = SPARSE_BACKWARD_MUTANTS[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    assert _sparse_backward_pin_err() > 1e-6


def test_sparse_backward_unmutated_pin_passes():
    assert _sparse_backward_pin_err() < 1e-8
