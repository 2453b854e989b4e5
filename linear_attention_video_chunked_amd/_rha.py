"""ctypes marshalling for librha.so.  See ``include/rha.h`` for the contract."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librha.so")

RHA_F32, RHA_BF16 = 0, 1
_STATUS = {0: "RHA_OK", 1: "RHA_ERR_INVALID_ARG", 2: "RHA_ERR_UNSUPPORTED", 3: "RHA_ERR_CURSOR", 4: "RHA_ERR_HIP"}


class LibraryNotBuilt(RuntimeError):
    pass


class RhaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("chunk_len", ctypes.c_int32),
        ("n_chunks", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("anchor_chunks", ctypes.c_int32),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
    ]


class Cursor(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int64)]


_lib = None
_vp = ctypes.c_void_p


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load librha.so (once).  Raises LibraryNotBuilt if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise LibraryNotBuilt(
            f"{_LIB_PATH} is missing: build it with `python -m linear_attention_video_chunked_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Problem)
    L.rha_state_scan.argtypes = [P, _vp, _vp, _vp, _vp, _vp]
    L.rha_hybrid_fwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.rha_hybrid_fwd_sparse.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.rha_state_scan_bidir.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.rha_hybrid_bwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.rha_hybrid_bwd_sparse.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
    L.rha_hybrid_bwd_workspace_size.argtypes = [P]
    L.rha_hybrid_bwd_workspace_size.restype = ctypes.c_size_t
    L.rha_hybrid_fwd_bidir.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.rha_hybrid_bwd_bidir.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_size_t, _vp]
    L.rha_hybrid_bwd_bidir_workspace_size.argtypes = [P]
    L.rha_hybrid_bwd_bidir_workspace_size.restype = ctypes.c_size_t
    L.rha_stream_step.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(Cursor),
                                  ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.rha_stream_step_sparse.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(Cursor),
                                         ctypes.c_int32, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.rha_stream_workspace_size.argtypes = [P]
    L.rha_stream_workspace_size.restype = ctypes.c_size_t
    L.rha_stream_step_noalloc.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(Cursor),
                                          ctypes.c_int32, _vp, _vp, _vp]
    for name in ("rha_state_scan", "rha_hybrid_fwd", "rha_hybrid_fwd_sparse", "rha_state_scan_bidir",
                 "rha_hybrid_fwd_bidir", "rha_hybrid_bwd", "rha_hybrid_bwd_sparse", "rha_hybrid_bwd_bidir", "rha_stream_step", "rha_stream_step_sparse",
                 "rha_stream_step_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    L.rha_status_string.argtypes = [ctypes.c_int]
    L.rha_status_string.restype = ctypes.c_char_p
    L.rha_last_error.argtypes = []
    L.rha_last_error.restype = ctypes.c_char_p
    L.rha_version.argtypes = []
    L.rha_version.restype = ctypes.c_int32
    _lib = L
    return L


def version() -> int:
    return int(lib().rha_version())


def _check(status: int):
    if status != 0:
        raise RhaError(status, lib().rha_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RHA_BF16
    if t.dtype == torch.float32:
        return RHA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _problem(x: torch.Tensor, C: int, w: int, n_chunks: int, anchors: int = 0) -> Problem:
    if x.dim() != 4:
        raise ValueError("tensors are [B, H, T, d]")
    if x.stride(3) != 1:
        raise ValueError("feature dimension must be contiguous")
    B, H, _, d = x.shape
    return Problem(B, H, d, C, n_chunks, w, _dtype_code(x), anchors, x.stride(0), x.stride(1), x.stride(2))


def _on_gpu(ref: torch.Tensor, name: str = "q"):
    """The library computes on the GPU only: host tensors would hand host
    pointers to the kernels.  Raised before any library call."""
    if ref.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got device {ref.device})")


def _same_layout(ref: torch.Tensor, *others: torch.Tensor):
    _on_gpu(ref)
    for o in others:
        if o.shape != ref.shape or o.stride() != ref.stride() or o.dtype != ref.dtype:
            raise ValueError("q, k, v and out must share shape, strides and dtype")
        if o.device != ref.device:
            raise ValueError("all tensors must be on the same device")


def _check_f32(ref: torch.Tensor, t: torch.Tensor, name: str, shape):
    """t: float32, contiguous, of the given shape, on ref's device."""
    if t.device != ref.device:
        raise ValueError(f"{name} must be on {ref.device} (got {t.device})")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32 (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def state_scan(k: torch.Tensor, v: torch.Tensor, C: int, w: int,
               S: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
               stream=None, anchors: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """rha_state_scan: S[b,h,c] = sum_{chunks anchors <= j <= c-w} phi(K_j)^T V_j, z likewise."""
    _same_layout(k, v)
    B, H, L, d = k.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    if S is None:
        S = torch.empty((B, H, N, d, d), dtype=torch.float32, device=k.device)
    if z is None:
        z = torch.empty((B, H, N, d), dtype=torch.float32, device=k.device)
    _check_f32(k, S, "S", (B, H, N, d, d))
    _check_f32(k, z, "z", (B, H, N, d))
    prob = _problem(k, C, w, N, anchors)
    _check(lib().rha_state_scan(ctypes.byref(prob), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _stream(stream)))
    return S, z


def hybrid_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: torch.Tensor, z: torch.Tensor,
               C: int, w: int, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               return_lse: bool = False, stream=None, anchors: int = 0):
    """rha_hybrid_fwd: the fused window + linear-state attention pass."""
    if out is None:
        out = torch.empty_like(q)
    _same_layout(q, k, v, out)
    B, H, L, d = q.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    _check_f32(q, S, "S", (B, H, N, d, d))
    _check_f32(q, z, "z", (B, H, N, d))
    if return_lse and lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_f32(q, lse, "lse", (B, H, L))
    prob = _problem(q, C, w, N, anchors)
    _check(lib().rha_hybrid_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _ptr(out),
                                _ptr(lse), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def hybrid_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: torch.Tensor, z: torch.Tensor,
               out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor, C: int, w: int, stream=None,
               anchors: int = 0):
    """rha_hybrid_bwd: (dq, dk, dv) float32 [B,H,L,d] of sum(dout * out) for the
    causal hybrid (out, lse from hybrid_fwd on the same inputs and anchors)."""
    _same_layout(q, k, v, out, dout)
    B, H, L, d = q.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    _check_f32(q, S, "S", (B, H, N, d, d))
    _check_f32(q, z, "z", (B, H, N, d))
    _check_f32(q, lse, "lse", (B, H, L))
    prob = _problem(q, C, w, N, anchors)
    nbytes = int(lib().rha_hybrid_bwd_workspace_size(ctypes.byref(prob)))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    dq = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    _check(lib().rha_hybrid_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _ptr(out), _ptr(lse),
                                _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nbytes, _stream(stream)))
    return dq, dk, dv


def state_scan_bidir(k: torch.Tensor, v: torch.Tensor, C: int, w: int, stream=None):
    """rha_state_scan_bidir -> (S_past, z_past, S_future, z_future), float32 [B,H,N,d,d] / [B,H,N,d]."""
    _same_layout(k, v)
    B, H, L, d = k.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    st = [torch.empty((B, H, N, d, d), dtype=torch.float32, device=k.device),
          torch.empty((B, H, N, d), dtype=torch.float32, device=k.device),
          torch.empty((B, H, N, d, d), dtype=torch.float32, device=k.device),
          torch.empty((B, H, N, d), dtype=torch.float32, device=k.device)]
    prob = _problem(k, C, w, N)
    _check(lib().rha_state_scan_bidir(ctypes.byref(prob), _ptr(k), _ptr(v), *(_ptr(x) for x in st),
                                      _stream(stream)))
    return tuple(st)


def hybrid_fwd_bidir(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, states, C: int, w: int,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = False, stream=None):
    """rha_hybrid_fwd_bidir: symmetric window + past and future linear states
    (``states`` as returned by state_scan_bidir for the same window)."""
    if out is None:
        out = torch.empty_like(q)
    _same_layout(q, k, v, out)
    B, H, L, d = q.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    Sp, zp, Sf, zf = states
    for name, S, z in (("past", Sp, zp), ("future", Sf, zf)):
        _check_f32(q, S, f"S_{name}", (B, H, N, d, d))
        _check_f32(q, z, f"z_{name}", (B, H, N, d))
    if return_lse and lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_f32(q, lse, "lse", (B, H, L))
    prob = _problem(q, C, w, N)
    _check(lib().rha_hybrid_fwd_bidir(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(Sp), _ptr(zp), _ptr(Sf),
                                      _ptr(zf), _ptr(out), _ptr(lse), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def hybrid_bwd_bidir(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, states, out: torch.Tensor,
                     lse: torch.Tensor, dout: torch.Tensor, C: int, w: int, stream=None):
    """rha_hybrid_bwd_bidir: (dq, dk, dv) float32 [B,H,L,d] of sum(dout * out)
    for the bidirectional hybrid (``states`` from state_scan_bidir; out, lse
    from hybrid_fwd_bidir on the same inputs)."""
    _same_layout(q, k, v, out, dout)
    B, H, L, d = q.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    Sp, zp, Sf, zf = states
    for name, S, z in (("past", Sp, zp), ("future", Sf, zf)):
        _check_f32(q, S, f"S_{name}", (B, H, N, d, d))
        _check_f32(q, z, f"z_{name}", (B, H, N, d))
    _check_f32(q, lse, "lse", (B, H, L))
    prob = _problem(q, C, w, N)
    nbytes = int(lib().rha_hybrid_bwd_bidir_workspace_size(ctypes.byref(prob)))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    dq = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    _check(lib().rha_hybrid_bwd_bidir(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(Sp), _ptr(zp), _ptr(Sf),
                                      _ptr(zf), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(ws), nbytes, _stream(stream)))
    return dq, dk, dv


# Block sizes of the pruned window (RHA_SPARSE_QTILE / RHA_SPARSE_KTILE).
SPARSE_QTILE = 256
SPARSE_KTILE = 64


def sparse_mask_shape(B: int, H: int, C: int, N: int, w: int):
    """Shape [B, H, N, nqt, nkt] of the block mask of hybrid_fwd_sparse."""
    nqt = -(-C // SPARSE_QTILE)
    wl = min(w, N) if w > 0 else 0
    return (B, H, N, nqt, -(-(wl * C) // SPARSE_KTILE))


def hybrid_fwd_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: torch.Tensor, z: torch.Tensor,
                      C: int, w: int, block_mask: torch.Tensor, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None):
    """rha_hybrid_fwd_sparse: hybrid_fwd with pruned (query block, key block)
    pairs of the window; block_mask is uint8 [B,H,N,nqt,nkt] (sparse_mask_shape)."""
    if out is None:
        out = torch.empty_like(q)
    _same_layout(q, k, v, out)
    B, H, L, d = q.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    _check_f32(q, S, "S", (B, H, N, d, d))
    _check_f32(q, z, "z", (B, H, N, d))
    if (tuple(block_mask.shape) != sparse_mask_shape(B, H, C, N, w) or block_mask.dtype != torch.uint8
            or not block_mask.is_contiguous() or block_mask.device != q.device):
        raise ValueError(f"block_mask must be contiguous uint8 {sparse_mask_shape(B, H, C, N, w)} on q's device")
    if return_lse and lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_f32(q, lse, "lse", (B, H, L))
    prob = _problem(q, C, w, N)
    _check(lib().rha_hybrid_fwd_sparse(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z),
                                       _ptr(block_mask), _ptr(out), _ptr(lse), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def hybrid_bwd_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: torch.Tensor, z: torch.Tensor,
                      block_mask: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                      C: int, w: int, stream=None):
    """rha_hybrid_bwd_sparse: (dq, dk, dv) float32 [B,H,L,d] of sum(dout * out)
    for the pruned window (out, lse from hybrid_fwd_sparse with the same mask)."""
    _same_layout(q, k, v, out, dout)
    B, H, L, d = q.shape
    if L % C:
        raise ValueError(f"sequence length {L} is not a multiple of chunk length {C}")
    N = L // C
    _check_f32(q, S, "S", (B, H, N, d, d))
    _check_f32(q, z, "z", (B, H, N, d))
    _check_f32(q, lse, "lse", (B, H, L))
    if (tuple(block_mask.shape) != sparse_mask_shape(B, H, C, N, w) or block_mask.dtype != torch.uint8
            or not block_mask.is_contiguous() or block_mask.device != q.device):
        raise ValueError(f"block_mask must be contiguous uint8 {sparse_mask_shape(B, H, C, N, w)} on q's device")
    prob = _problem(q, C, w, N)
    nbytes = int(lib().rha_hybrid_bwd_workspace_size(ctypes.byref(prob)))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    dq = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    _check(lib().rha_hybrid_bwd_sparse(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z),
                                       _ptr(block_mask), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                       _ptr(dv), _ptr(ws), nbytes, _stream(stream)))
    return dq, dk, dv


class StreamState:
    """Caller-owned streaming state: KV cache of w window slots (a ring) and
    `anchors` anchor slots, S, z, cursor, and the step's scratch workspace
    (rha_stream_workspace_size bytes; none if split=False or the library would
    not split this problem)."""

    def __init__(self, B: int, H: int, d: int, C: int, w: int, dtype=torch.bfloat16, device="cuda",
                 split: bool = True, anchors: int = 0):
        if anchors < 0:
            raise ValueError("anchors must be >= 0")
        self.B, self.H, self.d, self.C, self.w, self.anchors = B, H, d, C, w, anchors
        self.k_cache = torch.zeros((B, H, w + anchors, C, d), dtype=dtype, device=device)
        self.v_cache = torch.zeros((B, H, w + anchors, C, d), dtype=dtype, device=device)
        self.S = torch.zeros((B, H, d, d), dtype=torch.float32, device=device)
        self.z = torch.zeros((B, H, d), dtype=torch.float32, device=device)
        self.cursor = Cursor(0)
        self.workspace = None
        if split:
            prob = Problem(batch=B, heads=H, head_dim=d, chunk_len=C, n_chunks=1, window=w,
                           dtype=RHA_BF16 if dtype == torch.bfloat16 else RHA_F32, anchor_chunks=anchors,
                           stride_b=H * C * d, stride_h=C * d, stride_t=d)
            nbytes = int(lib().rha_stream_workspace_size(ctypes.byref(prob)))
            if nbytes > 0:
                self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    @property
    def t(self) -> int:
        return int(self.cursor.t)

    def clone(self) -> "StreamState":
        n = StreamState.__new__(StreamState)
        n.B, n.H, n.d, n.C, n.w, n.anchors = self.B, self.H, self.d, self.C, self.w, self.anchors
        n.k_cache, n.v_cache = self.k_cache.clone(), self.v_cache.clone()
        n.S, n.z = self.S.clone(), self.z.clone()
        n.cursor = Cursor(self.cursor.t)
        n.workspace = None if self.workspace is None else torch.empty_like(self.workspace)
        return n


def stream_step(st: StreamState, q_new: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                commit: bool = True, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """rha_stream_step: attend one new chunk to the cache + state; on commit fold
    the chunk that leaves the window and advance the cursor."""
    if out is None:
        out = torch.empty_like(q_new)
    prob = _stream_checks(st, q_new, k_new, v_new, out, lse)
    _check(lib().rha_stream_step(ctypes.byref(prob), _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(st.k_cache),
                                 _ptr(st.v_cache), _ptr(st.S), _ptr(st.z), ctypes.byref(st.cursor),
                                 ctypes.c_int32(1 if commit else 0), _ptr(out), _ptr(lse), _ptr(st.workspace),
                                 ctypes.c_size_t(0 if st.workspace is None else st.workspace.numel()),
                                 _stream(stream)))
    return out


def stream_mask_shape(B: int, H: int, C: int, w: int):
    """Shape [B, H, nqt, nkt] of one step's block mask for stream_step_sparse."""
    return (B, H, -(-C // SPARSE_QTILE), -(-(w * C) // SPARSE_KTILE))


def stream_step_sparse(st: StreamState, q_new: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       block_mask: torch.Tensor, commit: bool = True, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rha_stream_step_sparse: stream_step with pruned blocks of the window;
    block_mask is uint8 [B, H, nqt, nkt] (stream_mask_shape), key blocks over
    the window's keys in cache-slot order."""
    if out is None:
        out = torch.empty_like(q_new)
    prob = _stream_checks(st, q_new, k_new, v_new, out, lse)
    shape = stream_mask_shape(st.B, st.H, st.C, st.w)
    if (tuple(block_mask.shape) != shape or block_mask.dtype != torch.uint8 or not block_mask.is_contiguous()
            or block_mask.device != q_new.device):
        raise ValueError(f"block_mask must be contiguous uint8 {shape} on the chunk's device")
    _check(lib().rha_stream_step_sparse(ctypes.byref(prob), _ptr(q_new), _ptr(k_new), _ptr(v_new),
                                        _ptr(st.k_cache), _ptr(st.v_cache), _ptr(st.S), _ptr(st.z),
                                        ctypes.byref(st.cursor), ctypes.c_int32(1 if commit else 0),
                                        _ptr(block_mask), _ptr(out), _ptr(lse), _ptr(st.workspace),
                                        ctypes.c_size_t(0 if st.workspace is None else st.workspace.numel()),
                                        _stream(stream)))
    return out


def _stream_checks(st: StreamState, q_new, k_new, v_new, out, lse) -> Problem:
    _same_layout(q_new, k_new, v_new, out)
    B, H, C, d = q_new.shape
    if (B, H, C, d) != (st.B, st.H, st.C, st.d):
        raise ValueError("chunk shape does not match the stream state")
    if q_new.dtype != st.k_cache.dtype:
        raise ValueError("chunk dtype does not match the cache")
    for name, t in (("k_cache", st.k_cache), ("v_cache", st.v_cache), ("S", st.S), ("z", st.z)):
        if t.device != q_new.device:
            raise ValueError(f"stream state {name} is on {t.device}, the chunk on {q_new.device}")
    if st.workspace is not None and st.workspace.device != q_new.device:
        raise ValueError(f"stream workspace is on {st.workspace.device}, the chunk on {q_new.device}")
    if lse is not None:
        _check_f32(q_new, lse, "lse", (B, H, C))
    return _problem(q_new, C, st.w, 1, st.anchors)


# Bytes of device scratch the no-allocation step holds per GPU (RHA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 48 << 20


def stream_step_noalloc(st: StreamState, q_new: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        commit: bool = True, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rha_stream_step_noalloc: the streaming step with the library's own
    per-GPU scratch in place of a workspace (st.workspace is not used); for
    callers that cannot allocate device memory.  Pass ``out`` (and ``lse``)
    to keep this call free of allocation on the Python side too."""
    if out is None:
        out = torch.empty_like(q_new)
    _same_layout(q_new, k_new, v_new, out)
    B, H, C, d = q_new.shape
    if (B, H, C, d) != (st.B, st.H, st.C, st.d):
        raise ValueError("chunk shape does not match the stream state")
    if q_new.dtype != st.k_cache.dtype:
        raise ValueError("chunk dtype does not match the cache")
    for name, t in (("k_cache", st.k_cache), ("v_cache", st.v_cache), ("S", st.S), ("z", st.z)):
        if t.device != q_new.device:
            raise ValueError(f"stream state {name} is on {t.device}, the chunk on {q_new.device}")
    if lse is not None:
        _check_f32(q_new, lse, "lse", (B, H, C))
    prob = _problem(q_new, C, st.w, 1, st.anchors)
    _check(lib().rha_stream_step_noalloc(ctypes.byref(prob), _ptr(q_new), _ptr(k_new), _ptr(v_new),
                                         _ptr(st.k_cache), _ptr(st.v_cache), _ptr(st.S), _ptr(st.z),
                                         ctypes.byref(st.cursor), ctypes.c_int32(1 if commit else 0), _ptr(out),
                                         _ptr(lse), _stream(stream)))
    return out
