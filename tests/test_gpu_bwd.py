"""GPU parity of the backward pass (rha_hybrid_bwd) against the fp64 oracle's
chain-rule gradients (themselves pinned to finite differences and to torch
autograd on the CPU).

dq, dk, dv of sum(dout * out) for seeded q, k, v, dout at mid sizes (ragged
chunks, w = 0, 1, 2, 3, >= N, q x4) and sampled rows at the Wan-1.3B shape.
Bar: rel-L2 <= 1e-2 per gradient tensor, as for the forward outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, Workload, gen_block_mask, gen_qkv, to_storage
import linear_attention_video_chunked_amd as rha
from parity_utils import GroupedRows, sample_rows, TOL, rel_l2, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rha.lib()


def _dout(wl, seed):
    rng = np.random.default_rng(np.random.SeedSequence([wl.wid, 7, seed]))
    return to_storage(rng.standard_normal((wl.B, wl.H, wl.L, wl.d)), wl.dtype)


def _run(wl, q, k, v, dout):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    S, z = rha.state_scan(kd, vd, wl.C, wl.w)
    out, lse = rha.hybrid_fwd(qd, kd, vd, S, z, wl.C, wl.w, return_lse=True)
    dq, dk, dv = rha.hybrid_bwd(qd, kd, vd, S, z, out, lse, gd, wl.C, wl.w)
    torch.cuda.synchronize()
    return dq, dk, dv


# name: (B, H, C, N, w, qscale, kscale)
CASES = {
    "C200_N5_w2": (1, 2, 200, 5, 2, 1.0, 0.5),
    "C300_N4_w1": (1, 2, 300, 4, 1, 1.0, 1.0),
    "C100_N6_w3_q4": (1, 1, 100, 6, 3, 4.0, 0.5),
    "C130_N4_w0": (1, 2, 130, 4, 0, 1.0, 1.0),
    "C64_N5_w9": (1, 2, 64, 5, 9, 2.0, 1.0),
    "C256_N3_w2_B2": (2, 1, 256, 3, 2, 1.0, 0.5),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_against_oracle(name):
    B, H, C, N, w, qs, ks = CASES[name]
    wl = Workload(name, 1500 + sorted(CASES).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                  qscale=qs, kscale=ks)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 1)
    dq, dk, dv = _run(wl, q, k, v, dout)
    ref = oracle.hybrid_backward_batched(to64(q), to64(k), to64(v), wl.C, wl.w, to64(dout))
    errs = [rel_l2(to64(g), r) for g, r in zip((dq, dk, dv), ref)]
    print(f"{name}: rel-L2 dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    for e, nm in zip(errs, ("dq", "dk", "dv")):
        assert e <= TOL["bf16"], f"{nm}: rel-L2 {e:.3e}"


@pytest.mark.timeout(600)
def test_backward_wan13b_sampled_rows():
    wl = CONFIGS["wan13b"]
    print(f"[parity] bwd wan13b: H{wl.H} C{wl.C} N{wl.N} w{wl.w}", flush=True)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 2)
    dq, dk, dv = _run(wl, q, k, v, dout)
    # the oracle's full backward for a few heads; compare sampled rows
    # rows at chunk edges, tile edges and the short tails, plus random ones;
    # each gradient checked per chunk as well as over all sampled rows
    rows = sample_rows(wl.C, wl.N, 4 * wl.N, seed=17)
    grouped = [GroupedRows(f"bwd wan13b {nm}") for nm in ("dq", "dk", "dv")]
    for h in (0, 7):
        ref = oracle.hybrid_backward(to64(q)[0, h], to64(k)[0, h], to64(v)[0, h], wl.C, wl.w, to64(dout)[0, h])
        for i, (g, r) in enumerate(zip((dq, dk, dv), ref)):
            grouped[i].add_by_chunk((0, h), to64(g[0, h])[rows], r[rows], rows, wl.C)
    for gr in grouped:
        gr.check(TOL["bf16"])


# layout cases for the gradients: ragged 130-row chunks (a 2-row tail past one
# 128-key tile of the key-gradient kernel), with a window and without one
LAYOUT = {"C130_N4_w2_B2": (2, 2, 130, 4, 2), "C130_N4_w0_B2": (2, 2, 130, 4, 0)}


def _layout_wl(name):
    B, H, C, N, w = LAYOUT[name]
    return Workload(name, 1600 + sorted(LAYOUT).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                    qscale=1.0, kscale=0.5)


@pytest.mark.parametrize("name", sorted(LAYOUT))
def test_backward_strided_sequence_major_matches_contiguous(name):
    # q, k, v, out, dout in [B, L, H, d] storage viewed as [B, H, L, d]
    wl = _layout_wl(name)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 3)
    ref = _run(wl, q, k, v, dout)
    oref = oracle.hybrid_backward_batched(to64(q), to64(k), to64(v), wl.C, wl.w, to64(dout))
    for g, r, nm in zip(ref, oref, ("dq", "dk", "dv")):
        e = rel_l2(to64(g), r)
        assert e <= TOL["bf16"], f"{nm}: rel-L2 {e:.3e}"
    qs, ks, vs, gs = (t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (q, k, v, dout))
    assert qs.stride(2) == wl.H * wl.d
    S, z = rha.state_scan(ks, vs, wl.C, wl.w)
    out = torch.empty_like(qs)
    _, lse = rha.hybrid_fwd(qs, ks, vs, S, z, wl.C, wl.w, out=out, return_lse=True)
    got = rha.hybrid_bwd(qs, ks, vs, S, z, out, lse, gs, wl.C, wl.w)
    torch.cuda.synchronize()
    for g, r, nm in zip(got, ref, ("dq", "dk", "dv")):
        assert torch.equal(g, r), f"{nm} differs from the contiguous call"


@pytest.mark.parametrize("name", sorted(LAYOUT))
def test_backward_guard_bands_through_abi(name):
    # dq, dk, dv and the workspace inside sentinel-filled buffers, called
    # through the C ABI directly: nothing outside them changes, and the
    # gradients equal the binding's call on the same inputs
    import ctypes
    from linear_attention_video_chunked_amd import _rha as R
    wl = _layout_wl(name)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 4)
    ref = _run(wl, q, k, v, dout)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    S, z = rha.state_scan(kd, vd, wl.C, wl.w)
    out, lse = rha.hybrid_fwd(qd, kd, vd, S, z, wl.C, wl.w, return_lse=True)
    n = wl.B * wl.H * wl.L * wl.d
    pad = 4096  # floats on each side
    bigs = [torch.full((n + 2 * pad,), 9.0, dtype=torch.float32, device=DEV) for _ in range(3)]
    views = [b[pad: pad + n] for b in bigs]
    prob = R._problem(qd, wl.C, wl.w, wl.N)
    nbytes = int(R.lib().rha_hybrid_bwd_workspace_size(ctypes.byref(prob)))
    assert nbytes > 0
    wpad = 4096  # bytes on each side (16-byte aligned)
    wbig = torch.full((nbytes + 2 * wpad,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = wbig[wpad: wpad + nbytes]
    R._check(R.lib().rha_hybrid_bwd(ctypes.byref(prob), R._ptr(qd), R._ptr(kd), R._ptr(vd), R._ptr(S), R._ptr(z),
                                    R._ptr(out), R._ptr(lse), R._ptr(gd), R._ptr(views[0]), R._ptr(views[1]),
                                    R._ptr(views[2]), R._ptr(ws), nbytes, R._stream(None)))
    torch.cuda.synchronize()
    for b, nm in zip(bigs, ("dq", "dk", "dv")):
        assert (b[:pad] == 9.0).all() and (b[pad + n:] == 9.0).all(), f"{nm}: guard band written"
    assert (wbig[:wpad] == 0xA5).all() and (wbig[wpad + nbytes:] == 0xA5).all(), "workspace guard band written"
    for vw, r, nm in zip(views, ref, ("dq", "dk", "dv")):
        assert torch.equal(vw.view(r.shape), r), f"{nm} differs from the binding's call"


# ---------------------------------------------------------------- bidirectional
# rha_hybrid_bwd_bidir against the oracle's bidirectional chain rule (pinned to
# finite differences of the bidirectional forward and to torch autograd).

def _run_bidir(wl, q, k, v, dout):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    states = rha.state_scan_bidir(kd, vd, wl.C, wl.w)
    out, lse = rha.hybrid_fwd_bidir(qd, kd, vd, states, wl.C, wl.w, return_lse=True)
    grads = rha.hybrid_bwd_bidir(qd, kd, vd, states, out, lse, gd, wl.C, wl.w)
    torch.cuda.synchronize()
    return grads


# name: (B, H, C, N, w, qscale, kscale)
BIDIR_CASES = {
    "C200_N5_w2": (1, 2, 200, 5, 2, 1.0, 0.5),
    "C300_N4_w1": (1, 2, 300, 4, 1, 1.0, 1.0),
    "C100_N6_w3_q4": (1, 1, 100, 6, 3, 4.0, 0.5),
    "C130_N4_w0": (1, 2, 130, 4, 0, 1.0, 1.0),
    "C64_N5_w9": (1, 2, 64, 5, 9, 2.0, 1.0),
    "C280_N5_w2_B2": (2, 1, 280, 5, 2, 1.0, 0.5),
}


@pytest.mark.parametrize("name", sorted(BIDIR_CASES))
def test_bidir_backward_against_oracle(name):
    B, H, C, N, w, qs, ks = BIDIR_CASES[name]
    wl = Workload(name, 1700 + sorted(BIDIR_CASES).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                  qscale=qs, kscale=ks)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 5)
    grads = _run_bidir(wl, q, k, v, dout)
    ref = oracle.hybrid_bidir_backward_batched(to64(q), to64(k), to64(v), wl.C, wl.w, to64(dout))
    errs = [rel_l2(to64(g), r) for g, r in zip(grads, ref)]
    print(f"{name}: rel-L2 dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    for e, nm in zip(errs, ("dq", "dk", "dv")):
        assert e <= TOL["bf16"], f"{nm}: rel-L2 {e:.3e}"
    # and per chunk
    for g, r, nm in zip(grads, ref, ("dq", "dk", "dv")):
        g64 = to64(g)
        for c in range(N):
            sl = slice(c * C, (c + 1) * C)
            e = rel_l2(g64[:, :, sl], r[:, :, sl])
            assert e <= TOL["bf16"], f"{nm} chunk {c}: rel-L2 {e:.3e}"


def test_bidir_backward_window_all_equals_causal_call_when_one_chunk():
    # with a single chunk the symmetric and the causal window coincide and no
    # chunk has a state: both backward calls compute the same softmax gradient
    wl = Workload("bidir_one", 1750, B=1, H=2, d=128, C=300, N=1, w=3, dtype="bf16", qscale=1.0, kscale=0.5)
    q, k, v, dout = (t.to(DEV) for t in (*gen_qkv(wl), _dout(wl, 6)))
    S, z = rha.state_scan(k, v, wl.C, wl.w)
    out, lse = rha.hybrid_fwd(q, k, v, S, z, wl.C, wl.w, return_lse=True)
    states = rha.state_scan_bidir(k, v, wl.C, wl.w)
    a = rha.hybrid_bwd_bidir(q, k, v, states, out, lse, dout, wl.C, wl.w)
    b = rha.hybrid_bwd(q, k, v, S, z, out, lse, dout, wl.C, wl.w)
    torch.cuda.synchronize()
    for x, y, nm in zip(a, b, ("dq", "dk", "dv")):
        assert torch.equal(x, y), nm


@pytest.mark.timeout(600)
def test_bidir_backward_wan13b_sampled_rows():
    wl = CONFIGS["wan13b"]
    print(f"[parity] bidir bwd wan13b: H{wl.H} C{wl.C} N{wl.N} w{wl.w}", flush=True)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 7)
    grads = _run_bidir(wl, q, k, v, dout)
    rows = sample_rows(wl.C, wl.N, 4 * wl.N, seed=19)
    grouped = [GroupedRows(f"bidir bwd wan13b {nm}") for nm in ("dq", "dk", "dv")]
    h = 5
    ref = oracle.hybrid_bidir_backward(to64(q)[0, h], to64(k)[0, h], to64(v)[0, h], wl.C, wl.w, to64(dout)[0, h])
    for i, (g, r) in enumerate(zip(grads, ref)):
        grouped[i].add_by_chunk((0, h), to64(g[0, h])[rows], r[rows], rows, wl.C)
    for gr in grouped:
        gr.check(TOL["bf16"])


# ---------------------------------------------------------------- anchored
# rha_hybrid_bwd with anchor (sink) chunks against the oracle's anchored chain
# rule (pinned to finite differences of the anchored forward and torch autograd).

def _run_anchor(wl, a, q, k, v, dout):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    S, z = rha.state_scan(kd, vd, wl.C, wl.w, anchors=a)
    out, lse = rha.hybrid_fwd(qd, kd, vd, S, z, wl.C, wl.w, return_lse=True, anchors=a)
    grads = rha.hybrid_bwd(qd, kd, vd, S, z, out, lse, gd, wl.C, wl.w, anchors=a)
    torch.cuda.synchronize()
    return grads


# name: (B, H, C, N, w, a, qscale, kscale)
ANCHOR_CASES = {
    "C200_N5_w2_a1": (1, 2, 200, 5, 2, 1, 1.0, 0.5),
    "C130_N5_w1_a2": (1, 2, 130, 5, 1, 2, 1.0, 1.0),
    "C100_N6_w0_a1": (1, 1, 100, 6, 0, 1, 1.0, 0.5),
    "C64_N5_w3_a3": (1, 2, 64, 5, 3, 3, 2.0, 1.0),
    "C280_N4_w2_a1_q4": (2, 1, 280, 4, 2, 1, 4.0, 0.5),
    "C150_N3_w1_a5": (1, 2, 150, 3, 1, 5, 1.0, 1.0),
}


@pytest.mark.parametrize("name", sorted(ANCHOR_CASES))
def test_anchor_backward_against_oracle(name):
    B, H, C, N, w, a, qs, ks = ANCHOR_CASES[name]
    wl = Workload(name, 1800 + sorted(ANCHOR_CASES).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                  qscale=qs, kscale=ks)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 8)
    grads = _run_anchor(wl, a, q, k, v, dout)
    ref = oracle.hybrid_anchor_backward_batched(to64(q), to64(k), to64(v), wl.C, wl.w, a, to64(dout))
    for g, r, nm in zip(grads, ref, ("dq", "dk", "dv")):
        g64 = to64(g)
        e = rel_l2(g64, r)
        print(f"{name} {nm}: rel-L2 {e:.2e}")
        assert e <= TOL["bf16"], f"{nm}: rel-L2 {e:.3e}"
        for c in range(N):
            sl = slice(c * C, (c + 1) * C)
            ec = rel_l2(g64[:, :, sl], r[:, :, sl])
            assert ec <= TOL["bf16"], f"{nm} chunk {c}: rel-L2 {ec:.3e}"


def test_anchor_backward_zero_anchors_equals_plain_call():
    wl = Workload("anchor0", 1850, B=1, H=2, d=128, C=200, N=4, w=2, dtype="bf16", qscale=1.0, kscale=0.5)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 9)
    for x, y, nm in zip(_run_anchor(wl, 0, q, k, v, dout), _run(wl, q, k, v, dout), ("dq", "dk", "dv")):
        assert torch.equal(x, y), nm


@pytest.mark.timeout(600)
def test_anchor_backward_wan13b_sampled_rows():
    wl = CONFIGS["wan13b"]
    a = 1
    print(f"[parity] anchored bwd wan13b: H{wl.H} C{wl.C} N{wl.N} w{wl.w} a{a}", flush=True)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 10)
    grads = _run_anchor(wl, a, q, k, v, dout)
    rows = sample_rows(wl.C, wl.N, 4 * wl.N, seed=23)
    grouped = [GroupedRows(f"anchored bwd wan13b {nm}") for nm in ("dq", "dk", "dv")]
    h = 9
    ref = oracle.hybrid_anchor_backward(to64(q)[0, h], to64(k)[0, h], to64(v)[0, h], wl.C, wl.w, a, to64(dout)[0, h])
    for i, (g, r) in enumerate(zip(grads, ref)):
        grouped[i].add_by_chunk((0, h), to64(g[0, h])[rows], r[rows], rows, wl.C)
    for gr in grouped:
        gr.check(TOL["bf16"])


# ---------------------------------------------------------------------------
# rha_hybrid_bwd_sparse (pruned blocks of the window) against the oracle's
# pruned chain rule (pinned to finite differences of the pruned forward, to
# torch autograd through a separately written dense masked form, and to the
# plain backward when every block is kept).

def _run_sparse(wl, mask, q, k, v, dout):
    qd, kd, vd, gd, md = (t.to(DEV) for t in (q, k, v, dout, mask))
    S, z = rha.state_scan(kd, vd, wl.C, wl.w)
    out, lse = rha.hybrid_fwd_sparse(qd, kd, vd, S, z, wl.C, wl.w, md, return_lse=True)
    grads = rha.hybrid_bwd_sparse(qd, kd, vd, S, z, md, out, lse, gd, wl.C, wl.w)
    torch.cuda.synchronize()
    return grads, lse


# name: (B, H, C, N, w, qscale, kscale); windows of 400, 900, 1560 and 256
# keys end 16, 4, 24 and 0 keys into their last 64-key block, and chunks of
# 300 and 520 rows hold a short second or third 256-row query block
SPARSE_CASES = {
    "C200_N5_w2": (1, 2, 200, 5, 2, 1.0, 0.5),
    "C300_N4_w3_q4": (1, 2, 300, 4, 3, 4.0, 0.5),
    "C520_N3_w9": (1, 1, 520, 3, 9, 2.0, 1.0),
    "C64_N6_w4_B2": (2, 1, 64, 6, 4, 1.0, 1.0),
}


def _sparse_wl(name):
    B, H, C, N, w, qs, ks = SPARSE_CASES[name]
    return Workload(name, 1900 + sorted(SPARSE_CASES).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                    qscale=qs, kscale=ks)


@pytest.mark.parametrize("density", [0.85, 0.5, 0.15])
@pytest.mark.parametrize("name", sorted(SPARSE_CASES))
def test_sparse_backward_against_oracle(name, density):
    wl = _sparse_wl(name)
    shape = rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w)
    mask = gen_block_mask(shape, density, seed=wl.wid * 10 + int(density * 100))
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 11)
    grads, lse = _run_sparse(wl, mask, q, k, v, dout)
    ref = oracle.hybrid_block_sparse_backward_batched(to64(q), to64(k), to64(v), wl.C, wl.w, mask.numpy(),
                                                      to64(dout))
    # rows left with no weight: dq exactly 0
    empty = np.isneginf(to64(lse))
    assert np.all(to64(grads[0])[empty] == 0)
    for g, r, nm in zip(grads, ref, ("dq", "dk", "dv")):
        g64 = to64(g)
        e = rel_l2(g64, r)
        print(f"{name} density {density} {nm}: rel-L2 {e:.2e} ({empty.sum()} rows without weight)")
        assert e <= TOL["bf16"], f"{nm}: rel-L2 {e:.3e}"
        for c in range(wl.N):
            sl = slice(c * wl.C, (c + 1) * wl.C)
            if np.linalg.norm(r[:, :, sl]) > 0:
                ec = rel_l2(g64[:, :, sl], r[:, :, sl])
                assert ec <= TOL["bf16"], f"{nm} chunk {c}: rel-L2 {ec:.3e}"
            else:
                assert np.all(g64[:, :, sl] == 0), f"{nm} chunk {c}: nonzero where the oracle is zero"


@pytest.mark.parametrize("name", sorted(SPARSE_CASES))
def test_sparse_backward_all_kept_is_bitwise_plain(name):
    wl = _sparse_wl(name)
    ones = torch.ones(rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w), dtype=torch.uint8)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 12)
    grads, _ = _run_sparse(wl, ones, q, k, v, dout)
    for x, y, nm in zip(grads, _run(wl, q, k, v, dout), ("dq", "dk", "dv")):
        assert torch.equal(x, y), nm


@pytest.mark.parametrize("name", ["C200_N5_w2", "C300_N4_w3_q4"])
def test_sparse_backward_all_pruned_is_linear_only(name):
    wl = _sparse_wl(name)
    zeros = torch.zeros(rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w), dtype=torch.uint8)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 13)
    grads, lse = _run_sparse(wl, zeros, q, k, v, dout)
    assert bool(torch.isneginf(lse[:, :, : wl.w * wl.C]).all())
    ref = oracle.hybrid_block_sparse_backward_batched(to64(q), to64(k), to64(v), wl.C, wl.w, zeros.numpy(),
                                                      to64(dout))
    # no weight before chunk w: dq = 0 there; the keys of the last w chunks
    # are in no query's state: dk = dv = 0 there
    assert np.all(to64(grads[0])[:, :, : wl.w * wl.C] == 0)
    for g in grads[1:]:
        assert np.all(to64(g)[:, :, (wl.N - wl.w) * wl.C:] == 0)
    for g, r, nm in zip(grads, ref, ("dq", "dk", "dv")):
        e = rel_l2(to64(g), r)
        assert e <= TOL["bf16"], f"{nm}: rel-L2 {e:.3e}"


@pytest.mark.timeout(600)
def test_sparse_backward_wan13b_sampled_rows():
    wl = CONFIGS["wan13b"]
    print(f"[parity] pruned bwd wan13b: H{wl.H} C{wl.C} N{wl.N} w{wl.w}, half the blocks kept", flush=True)
    q, k, v = gen_qkv(wl)
    dout = _dout(wl, 14)
    mask = gen_block_mask(rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w), 0.5, seed=31)
    grads, _ = _run_sparse(wl, mask, q, k, v, dout)
    rows = sample_rows(wl.C, wl.N, 4 * wl.N, seed=29)
    grouped = [GroupedRows(f"pruned bwd wan13b {nm}") for nm in ("dq", "dk", "dv")]
    h = 4
    ref = oracle.hybrid_block_sparse_backward(to64(q)[0, h], to64(k)[0, h], to64(v)[0, h], wl.C, wl.w,
                                              mask[0, h].numpy(), to64(dout)[0, h])
    for i, (g, r) in enumerate(zip(grads, ref)):
        grouped[i].add_by_chunk((0, h), to64(g[0, h])[rows], r[rows], rows, wl.C)
    for gr in grouped:
        gr.check(TOL["bf16"])
