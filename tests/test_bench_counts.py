"""Host-side checks of bench.py's algorithmic counts (no GPU): the Wan-1.3B
figures the roofline divides by, and the pruned-window count."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synth import CONFIGS  # noqa: E402


def test_wan13b_counts():
    wl = CONFIGS["wan13b"]
    BH = wl.B * wl.H
    assert bench.fwd_flops(wl.C, wl.N, wl.w, wl.d, BH) == 908_250_071_040
    assert bench.fwd_bytes(wl.C, wl.N, wl.w, wl.d, BH) == 416_821_248
    assert abs(bench.scan_bytes(wl.C, wl.N, wl.w, wl.d, BH) / 1e6 - 189.2) < 0.1


def test_sparse_count_all_kept_equals_dense_and_scales():
    C, N, w, d, B, H = 300, 5, 2, 128, 1, 2
    nqt, nkt = -(-C // 256), -(-(w * C) // 64)
    ones = np.ones((B, H, N, nqt, nkt), np.uint8)
    dense = bench.fwd_flops(C, N, w, d, B * H)
    assert bench.sparse_fwd_flops(C, N, w, d, ones) == dense
    zeros = np.zeros_like(ones)
    lin = bench.sparse_fwd_flops(C, N, w, d, zeros)
    assert lin == sum(C * (2 * d * d + 2 * d) for c in range(N) if c >= w) * B * H
    # dropping one full key block of one query block removes rows * 64 * 4d
    m = ones.copy()
    m[0, 0, 3, 0, 2] = 0
    assert dense - bench.sparse_fwd_flops(C, N, w, d, m) == 256 * 64 * 4 * d


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bidir_count_limits():
    C, N, d, BH = 100, 6, 128, 3
    # w >= N: every key of every query in the window, no state
    assert bench.bidir_fwd_flops(C, N, N, d, BH) == (C * N) * (4 * d * C * N) * BH
    # w = 0: state only
    assert bench.bidir_fwd_flops(C, N, 0, d, BH) == C * N * (2 * d * d + 2 * d) * BH
    # the last chunk of a causal w = 2 problem sees what a bidirectional one does
    w = 2
    assert bench.bidir_fwd_flops(C, N, w, d, BH) > bench.fwd_flops(C, N, w, d, BH)


def test_anchor_count_limits():
    C, N, w, d, BH = 100, 6, 2, 128, 2
    assert bench.anchor_fwd_flops(C, N, w, 0, d, BH) == bench.fwd_flops(C, N, w, d, BH)
    # every chunk an anchor: block-causal dense attention, no state
    dense = sum(C * 4 * d * (c + 1) * C for c in range(N)) * BH
    assert bench.anchor_fwd_flops(C, N, w, N, d, BH) == dense


def test_bwd_count_is_two_and_a_half_forward_products_plus_state_terms():
    C, N, w, d, BH = 100, 5, 2, 128, 2
    pairs = sum(C * min(c + 1, w) * C for c in range(N)) * BH
    state_rows = sum(C for c in range(N) if c >= w) * BH
    folded = sum(C for c in range(N) if c <= N - 1 - w) * BH
    assert bench.bwd_flops(C, N, w, d, BH) == pairs * 10 * d + (state_rows + folded) * 4 * d * d


def test_bidir_bwd_count_by_brute_force():
    # pairs of the symmetric window counted token by token; state terms for
    # rows with any chunk outside their window and keys in some other chunk's
    # past (c >= j + w) or future (c <= j - max(w, 1)) state
    for C, N, w in ((3, 5, 2), (2, 4, 0), (2, 3, 5), (1, 6, 1)):
        d, BH = 4, 2
        L = C * N
        pairs = sum(1 for i in range(L) for j in range(L) if w > 0 and abs(i // C - j // C) <= w - 1)
        rows = sum(1 for i in range(L) if any(not (w > 0 and abs(i // C - c) <= w - 1) for c in range(N)))
        keys = sum(1 for j in range(L) if any(c >= j // C + w or c <= j // C - max(w, 1) for c in range(N)))
        assert bench.bidir_bwd_flops(C, N, w, d, BH) == BH * (pairs * 10 * d + (rows + keys) * 4 * d * d)


def test_anchor_bwd_count_limits_and_brute_force():
    C, N, w, d, BH = 3, 6, 2, 4, 2
    assert bench.anchor_bwd_flops(C, N, w, 0, d, BH) == bench.bwd_flops(C, N, w, d, BH)
    for a in (1, 2, 7):
        L = C * N
        keys = lambda i, j: (j // C <= i // C) and (j // C >= i // C - w + 1 or j // C < a)
        pairs = sum(1 for i in range(L) for j in range(L) if keys(i, j))
        rows = sum(1 for i in range(L) if i // C - w >= a)
        folded = sum(1 for j in range(L) if a <= j // C <= N - 1 - w)
        assert bench.anchor_bwd_flops(C, N, w, a, d, BH) == BH * (pairs * 10 * d + (rows + folded) * 4 * d * d)


def test_sparse_bwd_count_limits_and_brute_force():
    C, N, w, d, B, H = 300, 5, 2, 128, 1, 2
    nqt, nkt = -(-C // 256), -(-(w * C) // 64)
    ones = np.ones((B, H, N, nqt, nkt), np.uint8)
    assert bench.sparse_bwd_flops(C, N, w, d, ones) == bench.bwd_flops(C, N, w, d, B * H)
    # token by token on a tiny problem with 2-row query blocks and 3-key key blocks
    C, N, w, d, B, H = 5, 4, 2, 4, 1, 2
    rng = np.random.default_rng(3)
    m = (rng.random((B, H, N, 3, 4)) < 0.5).astype(np.uint8)
    pairs = 0
    for h in range(H):
        for i in range(N * C):
            c = i // C
            lo = max(0, c - w + 1) * C
            for j in range(lo, (c + 1) * C):
                pairs += int(m[0, h, c, (i - c * C) // 2, (j - lo) // 3])
    rows = sum(C for c in range(N) if c >= w) * B * H
    folded = sum(C for c in range(N) if c <= N - 1 - w) * B * H
    assert bench.sparse_bwd_flops(C, N, w, d, m, qtile=2, ktile=3) == pairs * 10 * d + (rows + folded) * 4 * d * d


def test_stream_sparse_count_all_kept_and_one_block():
    C, w, d, B, H = 1560, 9, 128, 1, 12
    nqt, nkt = -(-C // 256), -(-(w * C) // 64)
    ones = np.ones((B, H, nqt, nkt), np.uint8)
    full = bench.stream_sparse_step_flops(C, w, d, ones)
    assert full == bench.stream_step_flops(C, w, d, B * H)
    m = ones.copy()
    m[0, 3, 6, nkt - 1] = 0  # the last query block (24 rows) x the last key block (24 keys)
    assert full - bench.stream_sparse_step_flops(C, w, d, m) == 24 * 24 * 4 * d
