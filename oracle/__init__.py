"""fp64 CPU oracle of chunk-wise recurrent hybrid attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The library path
(``linear_attention_video_chunked_amd``) never imports it and shares no code
with it; the two meet only in the seeded input generator (``synth``).

See ``oracle.rha_oracle`` for the definitions and their sources.
"""
from .rha_oracle import (
    phi,
    window_range,
    brute_masked,
    chunk_states,
    state_scan,
    state_after,
    hybrid,
    hybrid_rows,
    hybrid_batched,
    state_scan_batched,
    sparse_mask_shape,
    brute_block_sparse,
    hybrid_block_sparse,
    hybrid_block_sparse_rows,
    hybrid_block_sparse_batched,
    window_range_bidir,
    brute_bidir,
    state_scan_bidir,
    hybrid_bidir,
    hybrid_bidir_rows,
    hybrid_bidir_batched,
    state_scan_bidir_batched,
    brute_anchor,
    state_scan_anchor,
    anchor_keys,
    hybrid_anchor,
    hybrid_anchor_rows,
    hybrid_anchor_batched,
    state_scan_anchor_batched,
)

__all__ = [
    "phi",
    "window_range",
    "brute_masked",
    "chunk_states",
    "state_scan",
    "state_after",
    "hybrid",
    "hybrid_rows",
    "hybrid_batched",
    "state_scan_batched",
    "sparse_mask_shape",
    "brute_block_sparse",
    "hybrid_block_sparse",
    "hybrid_block_sparse_rows",
    "hybrid_block_sparse_batched",
    "window_range_bidir",
    "brute_bidir",
    "state_scan_bidir",
    "hybrid_bidir",
    "hybrid_bidir_rows",
    "hybrid_bidir_batched",
    "state_scan_bidir_batched",
    "brute_anchor",
    "state_scan_anchor",
    "anchor_keys",
    "hybrid_anchor",
    "hybrid_anchor_rows",
    "hybrid_anchor_batched",
    "state_scan_anchor_batched",
]
