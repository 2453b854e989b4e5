"""GPU parity of the bidirectional hybrid (rha_state_scan_bidir +
rha_hybrid_fwd_bidir) against the fp64 oracle.

Reading (ReHyAt, abstract: the hybrid replaces the bidirectional attention of
video diffusion transformers): symmetric softmax window of w chunks each way
(own chunk included), every other chunk -- past and future -- in the linear
term.  Whole outputs at mid sizes (ragged chunks, w = 0, 1, 2, 3, all; q x4),
the four state tensors, and sampled rows at the Wan-1.3B shape.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, Workload, gen_qkv
import linear_attention_video_chunked_amd as rha
from parity_utils import ALARM, GroupedRows, sample_rows, TOL, per_chunk_rel_l2, rel_l2, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rha.lib()


# name: (B, H, C, N, w, qscale, kscale)
CASES = {
    "C200_N5_w2": (2, 2, 200, 5, 2, 1.0, 0.5),
    "C300_N4_w1": (1, 2, 300, 4, 1, 1.0, 1.0),
    "C300_N6_w3_q4": (1, 2, 300, 6, 3, 4.0, 0.5),
    "C130_N5_w0": (1, 2, 130, 5, 0, 1.0, 1.0),
    "C100_N4_w9": (1, 2, 100, 4, 9, 2.0, 1.0),
    "C64_N7_w4": (1, 1, 64, 7, 4, 1.0, 1.0),
    "C280_N5_w2": (1, 2, 280, 5, 2, 1.0, 0.5),  # 24-row tails
    "C16_N9_w3": (1, 2, 16, 9, 3, 2.0, 1.0),    # tails only
}


def _wl(name):
    B, H, C, N, w, qs, ks = CASES[name]
    return Workload(name, 1300 + sorted(CASES).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                    qscale=qs, kscale=ks)


@pytest.mark.parametrize("name", sorted(CASES))
def test_bidir_against_oracle(name):
    wl = _wl(name)
    q, k, v = gen_qkv(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    states = rha.state_scan_bidir(kd, vd, wl.C, wl.w)
    out, lse = rha.hybrid_fwd_bidir(qd, kd, vd, states, wl.C, wl.w, return_lse=True)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    ref, den = oracle.hybrid_bidir_batched(q64, k64, v64, wl.C, wl.w, return_den=True)
    o = to64(out)
    g = rel_l2(o, ref)
    pc = per_chunk_rel_l2(o, ref, wl.C)
    assert g <= TOL["bf16"], f"rel-L2 {g:.3e}"
    assert pc.max() <= TOL["bf16"], f"worst chunk {pc.max():.3e}"
    assert np.abs(to64(lse) - np.log(den)).max() <= 1e-2
    refs = oracle.state_scan_bidir_batched(k64, v64, wl.C, wl.w)
    for got, want, nm in zip(states, refs, ("S_past", "z_past", "S_future", "z_future")):
        gg = to64(got)
        if np.any(want != 0):
            assert rel_l2(gg, want) <= TOL["bf16"], nm
        # slots with no chunk on that side are exactly zero
        empty = np.all(want.reshape(want.shape[0], want.shape[1], want.shape[2], -1) == 0, axis=-1)
        assert np.all(gg.reshape(gg.shape[0], gg.shape[1], gg.shape[2], -1)[empty] == 0), nm
    print(f"{name}: rel-L2 {g:.3e}, worst chunk {pc.max():.3e}")


def test_bidir_window_all_matches_dense_softmax():
    # w >= N: every key in the softmax window, no state: unmasked attention
    wl = Workload("bidir_all", 1390, B=1, H=2, d=128, C=160, N=3, w=3, dtype="bf16")
    q, k, v = gen_qkv(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    states = rha.state_scan_bidir(kd, vd, wl.C, wl.w)
    out = rha.hybrid_fwd_bidir(qd, kd, vd, states, wl.C, wl.w)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double())
    torch.cuda.synchronize()
    assert rel_l2(to64(out), ref.numpy()) <= TOL["bf16"]
    assert all(torch.count_nonzero(x) == 0 for x in states)


@pytest.mark.timeout(600)
def test_bidir_wan13b_sampled_rows():
    wl = CONFIGS["wan13b"]
    print(f"[parity] bidir wan13b: H{wl.H} C{wl.C} N{wl.N} w{wl.w}", flush=True)
    q, k, v = gen_qkv(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    states = rha.state_scan_bidir(kd, vd, wl.C, wl.w)
    out = rha.hybrid_fwd_bidir(qd, kd, vd, states, wl.C, wl.w)
    torch.cuda.synchronize()
    og = out.cpu()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    grouped = GroupedRows("bidir wan13b")
    for h in range(0, wl.H, 4):
        st = oracle.state_scan_bidir(k64[0, h], v64[0, h], wl.C, wl.w)
        rows = sample_rows(wl.C, wl.N, 4 * wl.N, seed=11 + h)
        want = oracle.hybrid_bidir_rows(q64[0, h], k64[0, h], v64[0, h], wl.C, wl.w, rows, states=st)
        grouped.add_by_chunk((0, h), og[0, h, rows].double().numpy(), want, rows, wl.C)
        for x, r in zip(states, st):
            assert rel_l2(to64(x[0, h]), r) <= TOL["bf16"]
    grouped.check(TOL["bf16"], ALARM["bf16"])
