"""GPU parity of rha_stream_step: a stream of chunks equals the hybrid over
the concatenated sequence (oracle), the folded state equals the oracle's
prefix, and equals rha_state_scan bitwise; resuming from copied buffers and
re-running an uncommitted chunk change nothing."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, Workload, gen_qkv
import linear_attention_video_chunked_amd as rha
from parity_utils import ALARM, TOL, GroupedRows, rel_l2, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rha.lib()


def chunk(x, t, C):
    return x[:, :, t * C:(t + 1) * C].to(DEV)


def run_stream(wl, q, k, v, T, lse=False, split=True):
    st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w,
                         dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32, device=DEV, split=split)
    outs, lses = [], []
    for t in range(T):
        l = torch.empty((wl.B, wl.H, wl.C), dtype=torch.float32, device=DEV) if lse else None
        outs.append(rha.stream_step(st, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C), lse=l))
        lses.append(l)
    torch.cuda.synchronize()
    return st, outs, lses


SMALL = {
    "bf16_d128_C100_w3": Workload("s1", 300, B=1, H=2, d=128, C=100, N=12, w=3, dtype="bf16"),
    "bf16_d128_C100_w3_q4": Workload("s2", 301, B=2, H=2, d=128, C=100, N=10, w=3, dtype="bf16", qscale=4.0),
    "bf16_d128_C57_w1": Workload("s3", 302, B=1, H=2, d=128, C=57, N=8, w=1, dtype="bf16"),
    "bf16_d64_C64_w2": Workload("s4", 303, B=1, H=3, d=64, C=64, N=9, w=2, dtype="bf16"),
    "f32_d64_C48_w2": Workload("s5", 304, B=1, H=2, d=64, C=48, N=7, w=2, dtype="f32"),
    "f32_d128_C20_w4": Workload("s6", 305, B=1, H=1, d=128, C=20, N=9, w=4, dtype="f32"),
    # 256-row chunks and a 4-chunk window: enough key tiles for the split path
    "bf16_d128_C256_w4": Workload("s7", 306, B=1, H=2, d=128, C=256, N=8, w=4, dtype="bf16"),
    "bf16_d128_C300_w4_q4": Workload("s8", 307, B=1, H=1, d=128, C=300, N=7, w=4, dtype="bf16", qscale=4.0),
    # w = 1: the chunk leaving the window is the new chunk itself (the split fold reads it from k_new, v_new)
    "bf16_d128_C300_w1": Workload("s9", 308, B=1, H=2, d=128, C=300, N=6, w=1, dtype="bf16"),
    # chunks ending 24 rows past a 256-row tile, and 24-row chunks (the short-tail pass)
    "bf16_d128_C280_w3": Workload("s10", 309, B=1, H=2, d=128, C=280, N=8, w=3, dtype="bf16"),
    "bf16_d128_C24_w4_q4": Workload("s11", 310, B=1, H=2, d=128, C=24, N=9, w=4, dtype="bf16", qscale=4.0),
}


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_stream_matches_oracle_on_concatenation(name, split):
    wl = SMALL[name]
    q, k, v = gen_qkv(wl)
    st, outs, lses = run_stream(wl, q, k, v, wl.N, lse=True, split=split)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    ref, den = oracle.hybrid_batched(q64, k64, v64, wl.C, wl.w, return_den=True)
    tol = TOL[wl.dtype]
    for t, o in enumerate(outs):
        sl = slice(t * wl.C, (t + 1) * wl.C)
        e = rel_l2(to64(o), ref[:, :, sl])
        assert e <= tol, f"step {t}: rel-L2 {e:.3e}"
        assert np.abs(to64(lses[t]) - np.log(den[:, :, sl])).max() <= (1e-2 if wl.dtype == "bf16" else 1e-4)
    for b in range(wl.B):
        for h in range(wl.H):
            Sref, zref = oracle.state_after(k64[b, h], v64[b, h], wl.C, wl.w, wl.N)
            assert rel_l2(to64(st.S[b, h]), Sref) <= tol
            assert rel_l2(to64(st.z[b, h]), zref) <= tol
    assert st.t == wl.N


@pytest.mark.parametrize("name", ["bf16_d128_C256_w4", "bf16_d128_C300_w4_q4", "bf16_d128_C280_w3"])
def test_split_window_matches_unsplit(name):
    # the key window spread over several workgroups per query tile (with the
    # merge kernel) against one workgroup per tile: the same up to rounding
    wl = SMALL[name]
    st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV)
    assert st.workspace is not None, "this problem should use the split path"
    q, k, v = gen_qkv(wl)
    _, outs_a, lses_a = run_stream(wl, q, k, v, wl.N, lse=True, split=True)
    _, outs_b, lses_b = run_stream(wl, q, k, v, wl.N, lse=True, split=False)
    for t, (a, b) in enumerate(zip(outs_a, outs_b)):
        assert rel_l2(to64(a), to64(b)) <= 5e-3, f"step {t}"
        assert (lses_a[t] - lses_b[t]).abs().max().item() <= 1e-3


@pytest.mark.parametrize("name", ["bf16_d128_C100_w3", "bf16_d128_C300_w4_q4", "bf16_d128_C300_w1"])
def test_stream_state_equals_state_scan(name):
    # without a workspace the fold is the scan's own per-chunk kernel added in
    # the scan's order: bitwise equal; with one (token groups summed first)
    # equal to float rounding
    wl = SMALL[name]
    q, k, v = gen_qkv(wl)
    S_scan, z_scan = rha.state_scan(k.to(DEV), v.to(DEV), wl.C, wl.w)
    for split in (False, True):
        st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV, split=split)
        for t in range(wl.N - 1):
            rha.stream_step(st, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C))
            torch.cuda.synchronize()
            Sr, zr = S_scan[:, :, t + 1], z_scan[:, :, t + 1]
            if not split:
                assert torch.equal(st.S, Sr), f"S after commit {t}"
                assert torch.equal(st.z, zr), f"z after commit {t}"
            else:
                for a, r in ((st.S, Sr), (st.z, zr)):
                    err = ((a.double() - r.double()).norm() / max(r.double().norm().item(), 1e-30)).item()
                    assert err <= 1e-6, f"split fold, commit {t}: rel {err:.2e}"


def test_uncommitted_rerun_and_resume_are_exact():
    wl = SMALL["bf16_d128_C100_w3_q4"]
    q, k, v = gen_qkv(wl)
    st_a, outs_a, _ = run_stream(wl, q, k, v, wl.N)
    st_b = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV)
    outs_b = []
    half = wl.N // 2
    for t in range(wl.N):
        if t == half:
            # checkpoint: host copies of the whole constant-size state, restored into fresh buffers
            saved = [x.cpu() for x in (st_b.k_cache, st_b.v_cache, st_b.S, st_b.z)]
            cur = st_b.t
            st_b = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV)
            for dst, src in zip((st_b.k_cache, st_b.v_cache, st_b.S, st_b.z), saved):
                dst.copy_(src)
            st_b.cursor.t = cur
        # an uncommitted pass with other data first (as a denoising step would)
        noise = torch.randn_like(chunk(q, t, wl.C))
        rha.stream_step(st_b, noise, noise, noise, commit=False)
        assert st_b.t == t
        outs_b.append(rha.stream_step(st_b, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C)))
    torch.cuda.synchronize()
    for a, b in zip(outs_a, outs_b):
        assert torch.equal(a, b)
    assert torch.equal(st_a.S, st_b.S) and torch.equal(st_a.z, st_b.z)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("qscale", [1.0, 4.0])
def test_stream_workload_full_size(qscale):
    """9-frame window, 21-chunk prefill then 60 committed steps (81 chunks);
    also with q x 4 (peaked softmax weights, where a wrong window moves the
    result far more)."""
    wl = CONFIGS["stream"].replace(qscale=qscale)
    print(f"[parity] stream: H{wl.H} C{wl.C} w{wl.w} chunks {wl.N} q x{qscale}", flush=True)
    q, k, v = gen_qkv(wl)
    S_scan, z_scan = rha.state_scan(k.to(DEV), v.to(DEV), wl.C, wl.w)
    st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV)
    rng = np.random.default_rng(7)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    Sref, zref = oracle.state_scan_batched(k64, v64, wl.C, wl.w)
    grouped = GroupedRows(f"stream q x{qscale}")
    for t in range(wl.N):
        o = rha.stream_step(st, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C))
        if t + 1 < wl.N and (t + 1) % 20 == 0:
            torch.cuda.synchronize()
            # the split fold sums token groups first: equal to the scan up to rounding
            for x, r in ((st.S, S_scan[:, :, t + 1]), (st.z, z_scan[:, :, t + 1])):
                assert rel_l2(to64(x), to64(r)) <= 1e-6, f"state after commit {t}"
        rows = np.unique(np.concatenate([[0, 255, 256, wl.C - 25, wl.C - 24, wl.C - 1], rng.integers(0, wl.C, 8)]))
        og = o.cpu()
        for b in range(wl.B):
            for h in range(wl.H):
                ref = oracle.hybrid_rows(q64[b, h], k64[b, h], v64[b, h], wl.C, wl.w, t * wl.C + rows,
                                         S=Sref[b, h], z=zref[b, h])
                grouped.add((b, h, t), og[b, h, rows].double().numpy(), ref)
    torch.cuda.synchronize()
    # per (head, step): every step's window and state are checked on their own
    grouped.check(TOL["bf16"], ALARM["bf16"] if qscale == 1.0 else None)
    for b in range(wl.B):
        for h in range(wl.H):
            Sf, zf = oracle.state_after(k64[b, h], v64[b, h], wl.C, wl.w, wl.N)
            assert rel_l2(to64(st.S[b, h]), Sf) <= TOL["bf16"]
            assert rel_l2(to64(st.z[b, h]), zf) <= TOL["bf16"]


# ---- anchor (attention-sink) chunks: the first `a` chunks stay in every
# later chunk's softmax window and never enter the state (the anchored
# definition over the concatenated stream, oracle.hybrid_anchor)
ANCHORED = {
    "bf16_d128_C100_w3_a2": (Workload("sa1", 320, B=1, H=2, d=128, C=100, N=10, w=3, dtype="bf16"), 2),
    # short tails (C % 256 = 24) and peaked scores
    "bf16_d128_C280_w3_a1_q4": (Workload("sa2", 321, B=1, H=2, d=128, C=280, N=8, w=3, dtype="bf16", qscale=4.0), 1),
    # more anchors than window chunks, the split path
    "bf16_d128_C256_w2_a3": (Workload("sa3", 322, B=1, H=2, d=128, C=256, N=9, w=2, dtype="bf16"), 3),
    # w = 1 (the chunk leaving the window is the new chunk itself)
    "bf16_d128_C300_w1_a2": (Workload("sa4", 323, B=1, H=1, d=128, C=300, N=6, w=1, dtype="bf16"), 2),
    "f32_d64_C48_w2_a2": (Workload("sa5", 324, B=1, H=2, d=64, C=48, N=8, w=2, dtype="f32"), 2),
}


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("name", sorted(ANCHORED))
def test_stream_anchors_match_oracle(name, split):
    wl, a = ANCHORED[name]
    q, k, v = gen_qkv(wl)
    st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, anchors=a,
                         dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32, device=DEV, split=split)
    assert tuple(st.k_cache.shape) == (wl.B, wl.H, wl.w + a, wl.C, wl.d)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    ref, den = oracle.hybrid_anchor_batched(q64, k64, v64, wl.C, wl.w, a, return_den=True)
    tol = TOL[wl.dtype]
    for t in range(wl.N):
        lse = torch.empty((wl.B, wl.H, wl.C), dtype=torch.float32, device=DEV)
        o = rha.stream_step(st, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C), lse=lse)
        torch.cuda.synchronize()
        sl = slice(t * wl.C, (t + 1) * wl.C)
        e = rel_l2(to64(o), ref[:, :, sl])
        assert e <= tol, f"step {t}: rel-L2 {e:.3e}"
        assert np.abs(to64(lse) - np.log(den[:, :, sl])).max() <= (1e-2 if wl.dtype == "bf16" else 1e-4), f"step {t}"
    # the state after N commits: chunks a .. N-w (the anchors never folded)
    for b in range(wl.B):
        for h in range(wl.H):
            U, u = oracle.chunk_states(k64[b, h], v64[b, h], wl.C)
            lo, hi = a, wl.N - wl.w
            Sref = U[lo:hi + 1].sum(axis=0) if hi >= lo else np.zeros(U.shape[1:])
            zref = u[lo:hi + 1].sum(axis=0) if hi >= lo else np.zeros(u.shape[1:])
            assert rel_l2(to64(st.S[b, h]), Sref) <= tol
            assert rel_l2(to64(st.z[b, h]), zref) <= tol
    assert st.t == wl.N


def test_stream_anchor_slots_keep_the_first_chunks():
    # the anchor slots hold chunks 0 .. a-1 bitwise after the window has moved on
    wl, a = ANCHORED["bf16_d128_C100_w3_a2"]
    q, k, v = gen_qkv(wl)
    st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, anchors=a, device=DEV)
    for t in range(wl.N):
        rha.stream_step(st, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C))
    torch.cuda.synchronize()
    for j in range(a):
        assert torch.equal(st.k_cache[:, :, wl.w + j], chunk(k, j, wl.C))
        assert torch.equal(st.v_cache[:, :, wl.w + j], chunk(v, j, wl.C))


# ---- pruned streaming steps (rha_stream_step_sparse): one block mask per
# step over the window's keys in cache-slot order, against the oracle's pruned
# streaming definition (pinned to brute force, to the plain hybrid and to the
# whole-sequence pruned window)
SPARSE_STREAM = {
    # ring turns several times; 100-key chunks, so key blocks span two chunks
    "bf16_d128_C100_w3": Workload("sp1", 330, B=1, H=2, d=128, C=100, N=9, w=3, dtype="bf16"),
    # two query blocks per chunk (256 + 44 rows), q x4
    "bf16_d128_C300_w4_q4": Workload("sp2", 331, B=1, H=1, d=128, C=300, N=7, w=4, dtype="bf16", qscale=4.0),
    # chunks ending 24 rows past a 256-row tile (the short-tail pass), B = 2
    "bf16_d128_C280_w3_B2": Workload("sp3", 332, B=2, H=1, d=128, C=280, N=6, w=3, dtype="bf16"),
    # 24-row chunks (tails only) and w = 1
    "bf16_d128_C24_w4": Workload("sp4", 333, B=1, H=2, d=128, C=24, N=9, w=4, dtype="bf16"),
    "bf16_d128_C128_w1": Workload("sp5", 334, B=1, H=2, d=128, C=128, N=5, w=1, dtype="bf16"),
}


def _stream_masks(wl, density, seed):
    from synth import gen_block_mask
    shape = rha.stream_mask_shape(wl.B, wl.H, wl.C, wl.w)
    return gen_block_mask((wl.N,) + shape, density, seed)  # [N, B, H, nqt, nkt]


def run_sparse_stream(wl, q, k, v, masks, split):
    st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV, split=split)
    outs, lses = [], []
    for t in range(wl.N):
        l = torch.empty((wl.B, wl.H, wl.C), dtype=torch.float32, device=DEV)
        outs.append(rha.stream_step_sparse(st, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C),
                                           masks[t].contiguous().to(DEV), lse=l))
        lses.append(l)
    torch.cuda.synchronize()
    return st, outs, lses


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("density", [0.85, 0.5, 0.15])
@pytest.mark.parametrize("name", sorted(SPARSE_STREAM))
def test_stream_sparse_matches_oracle(name, density, split):
    wl = SPARSE_STREAM[name]
    q, k, v = gen_qkv(wl)
    masks = _stream_masks(wl, density, wl.wid * 10 + int(100 * density))
    st, outs, lses = run_sparse_stream(wl, q, k, v, masks, split)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    m = masks.numpy().transpose(1, 2, 0, 3, 4)  # [B, H, N, nqt, nkt]
    ref, den = oracle.stream_block_sparse_batched(q64, k64, v64, wl.C, wl.w, m, return_den=True)
    for t, (o, l) in enumerate(zip(outs, lses)):
        sl = slice(t * wl.C, (t + 1) * wl.C)
        og, lg, dt = to64(o), to64(l), den[:, :, sl]
        empty = dt == 0
        assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty])), f"step {t}: rows without weight"
        if (~empty).any():
            e = rel_l2(np.where(empty[..., None], 0.0, og), ref[:, :, sl])
            assert e <= TOL["bf16"], f"step {t}: rel-L2 {e:.3e}"
            assert np.abs(lg[~empty] - np.log(dt[~empty])).max() <= 1e-2
    for b in range(wl.B):
        for h in range(wl.H):
            Sref, zref = oracle.state_after(k64[b, h], v64[b, h], wl.C, wl.w, wl.N)
            assert rel_l2(to64(st.S[b, h]), Sref) <= TOL["bf16"]
            assert rel_l2(to64(st.z[b, h]), zref) <= TOL["bf16"]


@pytest.mark.parametrize("name", sorted(SPARSE_STREAM))
def test_stream_sparse_all_kept_equals_plain_step(name):
    wl = SPARSE_STREAM[name]
    q, k, v = gen_qkv(wl)
    ones = torch.ones((wl.N,) + rha.stream_mask_shape(wl.B, wl.H, wl.C, wl.w), dtype=torch.uint8)
    st1, outs1, lses1 = run_sparse_stream(wl, q, k, v, ones, split=False)
    st0, outs0, lses0 = run_stream(wl, q, k, v, wl.N, lse=True, split=False)
    for t in range(wl.N):
        assert torch.equal(outs1[t], outs0[t]) and torch.equal(lses1[t], lses0[t]), f"step {t}"
    assert torch.equal(st1.S, st0.S) and torch.equal(st1.z, st0.z)


@pytest.mark.timeout(900)
def test_stream_sparse_workload_half_kept_sampled_rows():
    """The 9-frame streaming workload's first 30 chunks, half the blocks of
    each step kept: sampled rows of every step against the oracle."""
    wl = CONFIGS["stream"].replace(N=30)
    print(f"[parity] pruned stream: H{wl.H} C{wl.C} w{wl.w} chunks {wl.N}", flush=True)
    q, k, v = gen_qkv(wl)
    masks = _stream_masks(wl, 0.5, 41)
    st = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV)
    rng = np.random.default_rng(11)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    Sref, zref = oracle.state_scan_batched(k64, v64, wl.C, wl.w)
    grouped = GroupedRows("pruned stream")
    heads = (0, 5, 11)
    for t in range(wl.N):
        o = rha.stream_step_sparse(st, chunk(q, t, wl.C), chunk(k, t, wl.C), chunk(v, t, wl.C),
                                   masks[t].contiguous().to(DEV))
        rows = np.unique(np.concatenate([[0, 255, 256, wl.C - 25, wl.C - 24, wl.C - 1], rng.integers(0, wl.C, 6)]))
        og = o.cpu()
        for h in heads:
            ref = oracle.stream_block_sparse_rows(q64[0, h], k64[0, h], v64[0, h], wl.C, wl.w, t,
                                                  masks[t, 0, h].numpy(), rows, S=Sref[0, h], z=zref[0, h])
            grouped.add((0, h, t), og[0, h, rows].double().numpy(), ref)
    torch.cuda.synchronize()
    grouped.check(TOL["bf16"])
