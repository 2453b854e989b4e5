"""Python binding of librha (chunk-wise recurrent hybrid attention, MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``librha.so`` (built from ``csrc/`` by ``build.py``).  PyTorch
supplies device memory and the current HIP stream.  If the library has not
been built, every call raises ``LibraryNotBuilt``; there is no fallback.

Functions mirror the C ABI in ``include/rha.h``:

* ``state_scan(k, v, C, w)``                     -> S [B,H,N,d,d], z [B,H,N,d]
* ``hybrid_fwd(q, k, v, S, z, C, w)``            -> out [B,H,L,d] (and lse)
* ``hybrid_fwd_sparse(q, k, v, S, z, C, w, m)``  the same with pruned window blocks
* ``state_scan_bidir`` / ``hybrid_fwd_bidir``     symmetric window, past + future states
* ``hybrid_bwd(q, k, v, S, z, out, lse, dout, C, w)`` -> dq, dk, dv (float32)
* ``hybrid_bwd_sparse(q, k, v, S, z, m, out, lse, dout, C, w)`` the same for pruned window blocks
* ``hybrid_bwd_bidir(q, k, v, states, out, lse, dout, C, w)`` the same for the bidirectional hybrid
* ``StreamState`` + ``stream_step(...)``         one chunk of streaming decode
* ``stream_step_sparse(..., block_mask)``          the step with pruned window blocks
* ``stream_step_noalloc(...)``                    the same step with the library's own scratch
"""
from ._rha import (
    LibraryNotBuilt,
    RhaError,
    StreamState,
    hybrid_bwd,
    hybrid_bwd_bidir,
    hybrid_bwd_sparse,
    hybrid_fwd,
    hybrid_fwd_bidir,
    hybrid_fwd_sparse,
    lib,
    lib_path,
    sparse_mask_shape,
    state_scan,
    state_scan_bidir,
    stream_mask_shape,
    stream_step,
    stream_step_noalloc,
    stream_step_sparse,
    version,
)

__all__ = [
    "LibraryNotBuilt",
    "RhaError",
    "StreamState",
    "hybrid_bwd",
    "hybrid_bwd_bidir",
    "hybrid_bwd_sparse",
    "hybrid_fwd",
    "hybrid_fwd_bidir",
    "hybrid_fwd_sparse",
    "lib",
    "lib_path",
    "sparse_mask_shape",
    "state_scan",
    "state_scan_bidir",
    "stream_mask_shape",
    "stream_step",
    "stream_step_sparse",
    "stream_step_noalloc",
    "version",
]
