"""Shared helpers for the GPU parity tests: run librha on seeded inputs and
compare against the fp64 oracle element by element."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import Workload, gen_qkv

# rel-L2 bars: bf16 storage with bf16 matrix-core products and float32
# accumulation, and all-float32 arithmetic.
TOL = {"bf16": 1e-2, "f32": 1e-4}


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm((np.asarray(got, np.float64) - ref).ravel())
    den = np.linalg.norm(np.asarray(ref, np.float64).ravel())
    return float(num / den) if den > 0 else float(num)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def inputs(wl: Workload, L=None):
    """Seeded CPU inputs [B,H,L,d] (storage dtype) and their float64 copies."""
    q, k, v = gen_qkv(wl, L)
    return (q, k, v), (to64(q), to64(k), to64(v))


def per_chunk_rel_l2(got: np.ndarray, ref: np.ndarray, C: int) -> np.ndarray:
    """rel-L2 of every (b, h, chunk) block, shape [B, H, N]."""
    B, H, L, d = ref.shape
    N = L // C
    g = np.asarray(got, np.float64).reshape(B, H, N, C * d)
    r = ref.reshape(B, H, N, C * d)
    return np.linalg.norm(g - r, axis=-1) / np.linalg.norm(r, axis=-1)


def sample_rows(C: int, N: int, n_random: int, seed: int, tile=128) -> np.ndarray:
    """Rows that hit chunk edges, tile edges and a ragged tail, plus random ones."""
    rows = set()
    for c in range(N):
        base = c * C
        for r in (0, 1, C - 1, C - 2, tile - 1, tile, C - (C % tile or tile), C - (C % tile or tile) - 1):
            if 0 <= r < C:
                rows.add(base + r)
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, C * N, n_random))
    return np.array(sorted(rows))
