"""GPU parity of anchor (sink) chunks (rha_state_scan / rha_hybrid_fwd with
anchor_chunks = a > 0) against the fp64 oracle.

Reading (Hybrid Forcing explainer, section 1: the attention-sink workaround
keeps the first frame attended): chunks 0 .. a-1 are in the softmax window of
every query chunk they do not lie in the future of, and out of the state.
Whole outputs and states at mid sizes (anchor segment ending mid-tile, window
touching or overlapping the anchors, w = 0, a >= N, q x4) and sampled rows at
the Wan-1.3B shape with the first frame as the sink.
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


# name: (B, H, C, N, w, a, qscale, kscale)
CASES = {
    "C200_N6_w2_a1": (2, 2, 200, 6, 2, 1, 1.0, 0.5),
    "C300_N5_w1_a2": (1, 2, 300, 5, 1, 2, 1.0, 1.0),
    "C100_N7_w3_a1_q4": (1, 2, 100, 7, 3, 1, 4.0, 0.5),
    "C130_N5_w0_a2": (1, 2, 130, 5, 0, 2, 1.0, 1.0),
    "C64_N6_w2_a3": (1, 2, 64, 6, 2, 3, 1.0, 1.0),
    "C150_N4_w2_a4": (1, 1, 150, 4, 2, 4, 2.0, 1.0),
    "C256_N5_w2_a1": (1, 2, 256, 5, 2, 1, 1.0, 1.0),
    # chunks ending 24 rows past a 256-row tile, and chunks of 24 rows (the
    # short-tail pass with the anchor range)
    "C280_N6_w2_a1": (1, 2, 280, 6, 2, 1, 1.0, 0.5),
    "C280_N5_w1_a2_q4": (1, 2, 280, 5, 1, 2, 4.0, 0.5),
    "C280_N4_w0_a1": (1, 2, 280, 4, 0, 1, 1.0, 1.0),
    "C24_N8_w2_a3": (1, 2, 24, 8, 2, 3, 1.0, 1.0),
}


def _wl(name):
    B, H, C, N, w, a, qs, ks = CASES[name]
    return Workload(name, 1400 + sorted(CASES).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                    qscale=qs, kscale=ks), a


@pytest.mark.parametrize("name", sorted(CASES))
def test_anchor_against_oracle(name):
    wl, a = _wl(name)
    q, k, v = gen_qkv(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    S, z = rha.state_scan(kd, vd, wl.C, wl.w, anchors=a)
    out, lse = rha.hybrid_fwd(qd, kd, vd, S, z, wl.C, wl.w, return_lse=True, anchors=a)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    ref, den = oracle.hybrid_anchor_batched(q64, k64, v64, wl.C, wl.w, a, return_den=True)
    o = to64(out)
    g = rel_l2(o, ref)
    pc = per_chunk_rel_l2(o, ref, wl.C)
    assert g <= TOL["bf16"], f"rel-L2 {g:.3e}"
    assert pc.max() <= TOL["bf16"], f"worst chunk {pc.max():.3e}"
    assert np.abs(to64(lse) - np.log(den)).max() <= 1e-2
    Sref, zref = oracle.state_scan_anchor_batched(k64, v64, wl.C, wl.w, a)
    Sg, zg = to64(S), to64(z)
    empty = ~np.any(Sref.reshape(*Sref.shape[:3], -1) != 0, axis=-1)
    assert np.all(Sg.reshape(*Sg.shape[:3], -1)[empty] == 0) and np.all(zg[empty] == 0)
    if np.any(Sref != 0):
        assert rel_l2(Sg, Sref) <= TOL["bf16"] and rel_l2(zg, zref) <= TOL["bf16"]
    print(f"{name}: rel-L2 {g:.3e}, worst chunk {pc.max():.3e}")


@pytest.mark.timeout(600)
def test_anchor_wan13b_first_frame_sink():
    wl = CONFIGS["wan13b"]
    a = 1
    print(f"[parity] anchor wan13b: H{wl.H} C{wl.C} N{wl.N} w{wl.w} a{a}", flush=True)
    q, k, v = gen_qkv(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    S, z = rha.state_scan(kd, vd, wl.C, wl.w, anchors=a)
    out = rha.hybrid_fwd(qd, kd, vd, S, z, wl.C, wl.w, anchors=a)
    torch.cuda.synchronize()
    og = out.cpu()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    grouped = GroupedRows("anchor wan13b")
    for h in range(0, wl.H, 4):
        Sh, zh = oracle.state_scan_anchor(k64[0, h], v64[0, h], wl.C, wl.w, a)
        rows = sample_rows(wl.C, wl.N, 4 * wl.N, seed=13 + h)
        want = oracle.hybrid_anchor_rows(q64[0, h], k64[0, h], v64[0, h], wl.C, wl.w, a, rows, S=Sh, z=zh)
        grouped.add_by_chunk((0, h), og[0, h, rows].double().numpy(), want, rows, wl.C)
        assert rel_l2(to64(S[0, h]), Sh) <= TOL["bf16"]
    grouped.check(TOL["bf16"], ALARM["bf16"])
