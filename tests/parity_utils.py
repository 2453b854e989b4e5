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
# A tighter bar for the unstressed workloads (q ~ N(0,1)): there the linear
# term carries most of the normaliser, so dropping a window chunk or
# mis-weighting a term moves rel-L2 by only about 1e-2 -- the bar itself --
# while the kernels' rounding gives about 2e-3.  Checked per (b, h, chunk).
ALARM = {"bf16": 5e-3, "f32": 5e-5}


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


class GroupedRows:
    """Sampled output rows gathered per group (b, h, chunk or step), so that a
    wrong chunk is not averaged away in one global rel-L2."""

    def __init__(self, name: str):
        self.name = name
        self.got, self.ref = {}, {}

    def add(self, key, got: np.ndarray, ref: np.ndarray):
        self.got.setdefault(key, []).append(np.asarray(got, np.float64).reshape(-1))
        self.ref.setdefault(key, []).append(np.asarray(ref, np.float64).reshape(-1))

    def add_by_chunk(self, prefix, got: np.ndarray, ref: np.ndarray, rows, C: int):
        ids = np.asarray(rows) // C
        for c in np.unique(ids):
            self.add(prefix + (int(c),), got[ids == c], ref[ids == c])

    def check(self, tol: float, alarm: float = None):
        """Asserts the global rel-L2 and the worst group's against tol (and,
        if given, the worst group's against alarm); returns both."""
        g = np.concatenate([np.concatenate(v) for v in self.got.values()])
        r = np.concatenate([np.concatenate(v) for v in self.ref.values()])
        glob = rel_l2(g, r)
        per = {k: rel_l2(np.concatenate(self.got[k]), np.concatenate(self.ref[k])) for k in self.got}
        worst_key = max(per, key=per.get)
        worst = per[worst_key]
        print(f"[parity] {self.name}: sampled rel-L2 {glob:.3e}, worst of {len(per)} groups {worst:.3e} "
              f"at {worst_key}", flush=True)
        assert glob <= tol, f"{self.name}: rel-L2 {glob:.3e}"
        assert worst <= tol, f"{self.name}: group {worst_key} rel-L2 {worst:.3e}"
        if alarm is not None:
            assert worst <= alarm, f"{self.name}: group {worst_key} rel-L2 {worst:.3e} above {alarm:.0e}"
        return glob, worst


def sample_rows(C: int, N: int, n_random: int, seed: int, tile=256) -> np.ndarray:
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
