"""C-ABI checks that need no GPU: the library loads, exports every function
include/rha.h declares, and rejects bad arguments before enqueuing anything.

Only argument errors are exercised here: each call below fails validation, so
no HIP runtime call is made.
"""
import ctypes
import os
import re

import pytest

from linear_attention_video_chunked_amd import _rha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rha.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_rha.lib_path()):
        from linear_attention_video_chunked_amd import build
        build.build(verbose=False)
    return _rha.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rha_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("rha_state_scan", "rha_hybrid_fwd", "rha_stream_step", "rha_status_string",
              "rha_last_error", "rha_version"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in _rha._STATUS.items():
        assert L.rha_status_string(code).decode() == name
    assert L.rha_version() >= 100


def _prob(**kw):
    base = dict(batch=1, heads=2, head_dim=128, chunk_len=64, n_chunks=4, window=2, dtype=_rha.RHA_BF16,
                anchor_chunks=0, stride_b=2 * 256 * 128, stride_h=256 * 128, stride_t=128)
    base.update(kw)
    return _rha.Problem(**base)


# fake, 256-byte aligned addresses: never dereferenced because validation fails first
P = ctypes.c_void_p(0x100000)
BAD = ctypes.c_void_p(0x100008)


def _scan(L, prob, k=P, v=P, S=P, z=P):
    return L.rha_state_scan(ctypes.byref(prob) if prob is not None else None, k, v, S, z, None)


def _fwd(L, prob, q=P, k=P, v=P, S=P, z=P, out=P, lse=None):
    return L.rha_hybrid_fwd(ctypes.byref(prob) if prob is not None else None, q, k, v, S, z, out, lse, None)


@pytest.mark.parametrize("field,value,code", [
    ("batch", -1, 1), ("heads", -3, 1), ("head_dim", 96, 2), ("head_dim", 256, 2),
    ("chunk_len", 0, 1), ("n_chunks", -1, 1), ("window", -1, 1), ("dtype", 7, 1),
    ("anchor_chunks", -1, 1), ("stride_t", 64, 1), ("stride_t", 132, 1), ("stride_h", -128, 1),
])
def test_invalid_problem_fields(L, field, value, code):
    prob = _prob(**{field: value})
    assert _scan(L, prob) == code
    assert L.rha_last_error().decode() != ""
    assert _fwd(L, prob) == code


def test_null_problem(L):
    assert _scan(L, None) == 1
    assert _fwd(L, None) == 1


@pytest.mark.parametrize("which", ["k", "v", "S", "z"])
def test_scan_null_and_misaligned_pointers(L, which):
    prob = _prob()
    assert _scan(L, prob, **{which: None}) == 1
    assert "NULL" in L.rha_last_error().decode()
    assert _scan(L, prob, **{which: BAD}) == 1
    assert "aligned" in L.rha_last_error().decode()


@pytest.mark.parametrize("which", ["q", "k", "v", "S", "z", "out"])
def test_fwd_null_and_misaligned_pointers(L, which):
    prob = _prob()
    assert _fwd(L, prob, **{which: None}) == 1
    assert _fwd(L, prob, **{which: BAD}) == 1


def test_fwd_misaligned_lse(L):
    assert _fwd(L, _prob(), lse=ctypes.c_void_p(0x100002)) == 1


def test_empty_problems_are_no_ops(L):
    # nothing to compute: OK without touching any pointer
    for kw in (dict(batch=0), dict(heads=0), dict(n_chunks=0)):
        prob = _prob(**kw)
        assert _scan(L, prob, k=None, v=None, S=None, z=None) == 0
        assert _fwd(L, prob, q=None, k=None, v=None, S=None, z=None, out=None) == 0


def test_f32_strides_must_be_16_byte_multiples(L):
    assert _scan(L, _prob(dtype=_rha.RHA_F32, stride_t=130)) == 1
    # 132 float32 = 528 bytes is a multiple of 16
    prob = _prob(dtype=_rha.RHA_F32, stride_t=132, head_dim=128)
    assert _scan(L, prob, k=None) == 1  # still fails, but on the pointer, not the stride
    assert "NULL" in L.rha_last_error().decode()


def _step(L, prob, cursor, commit=1, **ptrs):
    a = dict(q=P, k=P, v=P, kc=P, vc=P, S=P, z=P, out=P)
    a.update(ptrs)
    return L.rha_stream_step(ctypes.byref(prob), a["q"], a["k"], a["v"], a["kc"], a["vc"], a["S"], a["z"],
                             cursor, commit, a["out"], None, a.get("ws"), a.get("ws_bytes", 0), None)


def test_stream_validation(L):
    prob = _prob(window=0)
    cur = _rha.Cursor(0)
    assert _step(L, prob, ctypes.byref(cur)) == 1  # streaming needs w >= 1
    prob = _prob(window=3)
    assert _step(L, prob, None) == 3
    cur = _rha.Cursor(-1)
    assert _step(L, prob, ctypes.byref(cur)) == 3
    cur = _rha.Cursor(5)
    assert _step(L, prob, ctypes.byref(cur), kc=None) == 1
    assert cur.t == 5  # nothing happened
    assert _step(L, prob, ctypes.byref(cur), out=BAD) == 1
    assert cur.t == 5


def test_stream_workspace_checks(L):
    prob = _prob(window=3)
    cur = _rha.Cursor(5)
    assert _step(L, prob, ctypes.byref(cur), ws=BAD, ws_bytes=1 << 20) == 1
    assert "workspace" in L.rha_last_error().decode()
    assert cur.t == 5
    # no split for float32 problems, nor for invalid ones
    assert L.rha_stream_workspace_size(ctypes.byref(_prob(window=3, dtype=_rha.RHA_F32, stride_t=128))) == 0
    assert L.rha_stream_workspace_size(ctypes.byref(_prob(window=3, dtype=_rha.RHA_F32, head_dim=64, stride_t=64))) == 0
    assert L.rha_stream_workspace_size(ctypes.byref(_prob(window=0))) == 0
    assert L.rha_stream_workspace_size(None) == 0


def _sstep(L, prob, cursor, mask=P, commit=1, **ptrs):
    a = dict(q=P, k=P, v=P, kc=P, vc=P, S=P, z=P, out=P)
    a.update(ptrs)
    return L.rha_stream_step_sparse(ctypes.byref(prob), a["q"], a["k"], a["v"], a["kc"], a["vc"], a["S"], a["z"],
                                    cursor, commit, mask, a["out"], None, None, 0, None)


def test_stream_sparse_checks(L):
    cur = _rha.Cursor(5)
    # the pruned step: bf16, head_dim 128, no anchors, a mask; the plain step's rules
    assert _sstep(L, _prob(window=3, dtype=_rha.RHA_F32, stride_t=128), ctypes.byref(cur)) == 2
    assert _sstep(L, _prob(window=3, head_dim=64, stride_t=64), ctypes.byref(cur)) == 2
    assert _sstep(L, _prob(window=3, anchor_chunks=1), ctypes.byref(cur)) == 2
    assert "anchor" in L.rha_last_error().decode()
    assert _sstep(L, _prob(window=3), ctypes.byref(cur), mask=None) == 1
    assert "block_mask" in L.rha_last_error().decode()
    assert _sstep(L, _prob(window=0), ctypes.byref(cur)) == 1
    assert _sstep(L, _prob(window=3), None) == 3
    assert _sstep(L, _prob(window=3), ctypes.byref(cur), kc=None) == 1
    big = _prob(window=3, chunk_len=4096 * 16, stride_b=0, stride_h=0)
    assert _sstep(L, big, ctypes.byref(cur)) == 2 and "key blocks" in L.rha_last_error().decode()
    assert cur.t == 5  # nothing happened
    # an empty problem needs no mask and still advances the cursor
    assert _sstep(L, _prob(batch=0, window=3), ctypes.byref(cur), mask=None, q=None) == 0
    assert cur.t == 6
    assert _rha.stream_mask_shape(1, 12, 1560, 9) == (1, 12, 7, 220)


def test_stream_empty_problem_advances_cursor(L):
    prob = _prob(batch=0, window=3)
    cur = _rha.Cursor(4)
    assert _step(L, prob, ctypes.byref(cur), commit=1, q=None) == 0
    assert cur.t == 5
    assert _step(L, prob, ctypes.byref(cur), commit=0, q=None) == 0
    assert cur.t == 5


def test_too_large_problem_rejected(L):
    prob = _prob(chunk_len=1 << 20, n_chunks=1 << 12)
    assert _scan(L, prob) == 1
    assert "too large" in L.rha_last_error().decode()


def test_head_byte_span_limit(L):
    # 32-bit buffer offsets: one head's keys (plus two tiles of slack) must
    # span less than 2 GiB; token-major strides make that the binding limit
    prob = _prob(chunk_len=4096, n_chunks=16, stride_t=16384)
    assert _scan(L, prob) == 1
    assert "2 GiB" in L.rha_last_error().decode()


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_rha, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_rha, "_lib", None)
    with pytest.raises(_rha.LibraryNotBuilt):
        _rha.lib()


def _sparse(L, prob, mask=P, q=P, k=P, v=P, S=P, z=P, out=P, lse=None):
    return L.rha_hybrid_fwd_sparse(ctypes.byref(prob), q, k, v, S, z, mask, out, lse, None)


def test_sparse_window_checks(L):
    # pruned windows: bf16 with head_dim 128 only, a mask, and at most 2048 key blocks per window
    assert _sparse(L, _prob(dtype=_rha.RHA_F32, stride_t=128)) == 2
    assert _sparse(L, _prob(head_dim=64, stride_t=64)) == 2
    assert "RHA_BF16" in L.rha_last_error().decode()
    assert _sparse(L, _prob(), mask=None) == 1
    assert "block_mask" in L.rha_last_error().decode()
    assert _sparse(L, _prob(chunk_len=4096 * 16, n_chunks=4, window=3, stride_b=0, stride_h=0)) == 2
    assert "key blocks" in L.rha_last_error().decode()
    assert _sparse(L, _prob(), q=None) == 1
    assert _sparse(L, _prob(window=-1)) == 1
    # the binding's mask shape: [B, H, N, ceil(C / 256), ceil(min(w, N) * C / 64)]
    assert _rha.sparse_mask_shape(1, 12, 1560, 21, 3) == (1, 12, 21, 7, 74)
    assert _rha.sparse_mask_shape(2, 3, 100, 4, 9) == (2, 3, 4, 1, 7)
    assert _rha.sparse_mask_shape(1, 1, 64, 4, 0) == (1, 1, 4, 1, 0)


def test_bidir_checks(L):
    # bidirectional calls: bf16 with head_dim 128 only; every state pointer required
    args = [P] * 7
    f32 = _prob(dtype=_rha.RHA_F32, stride_t=128)
    assert L.rha_state_scan_bidir(ctypes.byref(f32), *args[:6], None) == 2
    assert L.rha_hybrid_fwd_bidir(ctypes.byref(f32), *([P] * 9), None, None) == 2
    assert "RHA_BF16" in L.rha_last_error().decode()
    d64 = _prob(head_dim=64, stride_t=64)
    assert L.rha_state_scan_bidir(ctypes.byref(d64), *args[:6], None) == 2
    ok = _prob()
    assert L.rha_state_scan_bidir(ctypes.byref(ok), P, P, P, P, None, P, None) == 1
    assert "S_future" in L.rha_last_error().decode()
    assert L.rha_hybrid_fwd_bidir(ctypes.byref(ok), P, P, P, P, P, P, None, P, None, None) == 1
    assert "z_future" in L.rha_last_error().decode()
    assert L.rha_hybrid_fwd_bidir(ctypes.byref(_prob(window=-2)), *([P] * 9), None, None) == 1


def test_anchor_checks(L):
    # anchor chunks: bf16 with head_dim 128 for the whole-sequence calls; not for
    # pruned or bidirectional calls (the streaming step keeps them in cache
    # slots of their own, any dtype: only a negative count is refused there)
    assert _scan(L, _prob(anchor_chunks=1, dtype=_rha.RHA_F32, stride_t=128)) == 2
    assert _fwd(L, _prob(anchor_chunks=2, head_dim=64, stride_t=64)) == 2
    assert "anchor" in L.rha_last_error().decode()
    assert _sparse(L, _prob(anchor_chunks=1)) == 2
    assert L.rha_state_scan_bidir(ctypes.byref(_prob(anchor_chunks=1)), P, P, P, P, P, P, None) == 2
    cur = _rha.Cursor(0)
    assert _step(L, _prob(anchor_chunks=-1, window=2), ctypes.byref(cur)) == 1
    assert "anchor_chunks" in L.rha_last_error().decode()
    assert cur.t == 0
    # anchor and window tiles listed per query chunk: at most 2048 tiles of 64 keys
    big = _prob(anchor_chunks=20, n_chunks=40, window=20, chunk_len=4000, stride_b=0, stride_h=0)
    assert _fwd(L, big) == 2 and "key tiles" in L.rha_last_error().decode()


def test_backward_checks(L):
    args = [P] * 12
    assert L.rha_hybrid_bwd(ctypes.byref(_prob(dtype=_rha.RHA_F32, stride_t=128)), *args, 1 << 30, None) == 2
    # the bidirectional backward takes no anchor chunks (the causal one does)
    bargs = [P] * 14
    assert L.rha_hybrid_bwd_bidir(ctypes.byref(_prob(anchor_chunks=1)), *bargs, 1 << 30, None) == 2
    assert L.rha_hybrid_bwd_bidir(ctypes.byref(_prob(dtype=_rha.RHA_F32, stride_t=128)), *bargs, 1 << 30, None) == 2
    ok = _prob()
    need_b = L.rha_hybrid_bwd_bidir_workspace_size(ctypes.byref(ok))
    assert need_b > L.rha_hybrid_bwd_workspace_size(ctypes.byref(ok))  # two sets of state gradients
    assert L.rha_hybrid_bwd_bidir(ctypes.byref(ok), *bargs, need_b - 1, None) == 1
    assert "workspace" in L.rha_last_error().decode()
    assert L.rha_hybrid_bwd_bidir(ctypes.byref(ok), *bargs[:5], None, *bargs[6:], need_b, None) == 1  # S_future
    assert "S_future" in L.rha_last_error().decode()
    need = L.rha_hybrid_bwd_workspace_size(ctypes.byref(ok))
    assert need > 0
    assert L.rha_hybrid_bwd(ctypes.byref(ok), *args, need - 1, None) == 1
    assert "workspace" in L.rha_last_error().decode()
    assert L.rha_hybrid_bwd(ctypes.byref(ok), *args[:6], None, *args[7:], need, None) == 1  # lse required
    assert "lse" in L.rha_last_error().decode()
    # the pruned backward: the pruned forward's rules, the plain workspace
    sargs = [P] * 13
    assert L.rha_hybrid_bwd_sparse(ctypes.byref(_prob(anchor_chunks=1)), *sargs, 1 << 30, None) == 2
    assert L.rha_hybrid_bwd_sparse(ctypes.byref(_prob(dtype=_rha.RHA_F32, stride_t=128)), *sargs, 1 << 30,
                                   None) == 2
    big = _prob(chunk_len=4096 * 16, n_chunks=4, window=3, stride_b=0, stride_h=0)
    assert L.rha_hybrid_bwd_sparse(ctypes.byref(big), *sargs, 1 << 40, None) == 2
    assert "key blocks" in L.rha_last_error().decode()
    assert L.rha_hybrid_bwd_sparse(ctypes.byref(ok), *sargs[:5], None, *sargs[6:], need, None) == 1  # mask
    assert "block_mask" in L.rha_last_error().decode()
    assert L.rha_hybrid_bwd_sparse(ctypes.byref(ok), *sargs, need - 1, None) == 1
    assert "workspace" in L.rha_last_error().decode()
    assert L.rha_hybrid_bwd_sparse(ctypes.byref(ok), *sargs[:7], None, *sargs[8:], need, None) == 1  # lse
    assert "lse" in L.rha_last_error().decode()
