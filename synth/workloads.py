"""Workload table and seeded Gaussian input generation.

Shapes follow the latent-frame geometry of the Wan 2.1 video DiTs named on the
ReHyAt pages (480p: 30x52 = 1560 patches per latent frame, 720p: 45x80 = 3600;
21 latent frames per clip), with one chunk = one latent frame.  No real
activations are available, so N(0,1) tensors stand in for them.

Seeding: every (workload, tensor, batch, head) gets its own NumPy
``SeedSequence([workload_id, tensor_id, b, h])`` stream, so any single head can
be regenerated without drawing the rest.  Values are drawn in float64, scaled,
then rounded (round-to-nearest-even, via torch's CPU cast) to the storage dtype.
Both the oracle and the GPU path consume exactly the rounded values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

TENSOR_ID = {"q": 0, "k": 1, "v": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int          # seed namespace
    B: int
    H: int
    d: int
    C: int            # chunk length in tokens (one latent frame)
    N: int            # number of chunks in the full sequence
    w: int            # window in chunks, counting the query's own chunk
    dtype: str        # "f32" or "bf16"
    qscale: float = 1.0
    kscale: float = 1.0
    vscale: float = 1.0
    prefill: int = 0  # streaming: chunks pushed before the timed steps
    steps: int = 0    # streaming: timed decode steps

    @property
    def L(self) -> int:
        return self.N * self.C

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # 4 chunks x 64 tokens, own-chunk softmax + linear state of earlier chunks
    "tiny": Workload("tiny", 0, B=1, H=2, d=64, C=64, N=4, w=1, dtype="f32"),
    # Wan 2.1 1.3B at 480p: 21 latent frames x 1560 tokens, 3-frame window
    "wan13b": Workload("wan13b", 1, B=1, H=12, d=128, C=1560, N=21, w=3, dtype="bf16", kscale=0.5),
    # streaming decode: 9-frame window (8 cached + the new frame), 21-frame
    # prefill then 60 committed steps (81 chunks in all)
    "stream": Workload("stream", 2, B=1, H=12, d=128, C=1560, N=81, w=9, dtype="bf16",
                       prefill=21, steps=60),
    # Wan 2.1 14B at 720p: 21 latent frames x 3600 tokens, 2-frame window
    "wan14b": Workload("wan14b", 3, B=1, H=40, d=128, C=3600, N=21, w=2, dtype="bf16"),
    # 6x horizon: 126 latent frames x 1560 tokens, 3-frame window
    "long": Workload("long", 4, B=1, H=12, d=128, C=1560, N=126, w=3, dtype="bf16"),
}


def to_storage(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """Round float64 values to the storage dtype (RNE) and return a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown dtype {dtype}")


def gen_head(wl: Workload, tensor: str, b: int, h: int, L: Optional[int] = None,
             t0: int = 0) -> torch.Tensor:
    """One head's [L, d] tensor in storage dtype (CPU).

    Tokens [t0, t0+L) of the head's stream are returned; the stream for a
    (workload, tensor, b, h) is fixed, so a slice equals the same rows of the
    whole sequence.
    """
    L = wl.L if L is None else L
    ss = np.random.SeedSequence([wl.wid, TENSOR_ID[tensor], b, h])
    rng = np.random.default_rng(ss)
    if t0:
        rng.standard_normal((t0, wl.d))  # advance the stream
    x = rng.standard_normal((L, wl.d))
    scale = {"q": wl.qscale, "k": wl.kscale, "v": wl.vscale}[tensor]
    if scale != 1.0:
        x = x * scale
    return to_storage(x, wl.dtype)


def gen_qkv(wl: Workload, L: Optional[int] = None):
    """q, k, v as contiguous CPU tensors of shape [B, H, L, d] in storage dtype."""
    L = wl.L if L is None else L
    out = []
    for name in ("q", "k", "v"):
        heads = [gen_head(wl, name, b, h, L) for b in range(wl.B) for h in range(wl.H)]
        out.append(torch.stack(heads).reshape(wl.B, wl.H, L, wl.d))
    return tuple(out)


def gen_block_mask(shape, density: float, seed: int) -> torch.Tensor:
    """Seeded 0/1 uint8 mask (CPU) of the given shape: each entry kept with
    probability ``density`` -- a stand-in for a block-importance criterion,
    which the pages do not give."""
    rng = np.random.default_rng(np.random.SeedSequence([9000, seed]))
    return torch.from_numpy((rng.random(tuple(shape)) < density).astype(np.uint8))
