"""GPU parity of the block-sparse window (rha_hybrid_fwd_sparse) against the
fp64 oracle's pruned definition (explainer page of "Long-Horizon Streaming
Video Generation via Hybrid Attention with Decoupled Distillation", section
2.A: blocks of the local window judged unimportant are pruned; the page gives
no criterion, so the kept blocks are a seeded random mask here).

* every block kept: bitwise equal to rha_hybrid_fwd (also at the Wan-1.3B shape);
* random masks (dense, half, sparse) at mid sizes: rel-L2 <= 1e-2 globally and
  per (b, h, chunk), lse within 1e-2 where the denominator is positive, and
  out = 0, lse = -inf where every weight was pruned;
* every block pruned: the linear term alone;
* Wan-1.3B shape with half the blocks kept: sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, Workload, gen_block_mask, gen_qkv
import linear_attention_video_chunked_amd as rha
from parity_utils import TOL, per_chunk_rel_l2, rel_l2, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rha.lib()


def _run(wl, mask, q=None, k=None, v=None):
    if q is None:
        q, k, v = gen_qkv(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    S, z = rha.state_scan(kd, vd, wl.C, wl.w)
    out, lse = rha.hybrid_fwd_sparse(qd, kd, vd, S, z, wl.C, wl.w, mask.to(DEV), return_lse=True)
    torch.cuda.synchronize()
    return (q, k, v), out, lse, (qd, kd, vd, S, z)


# name: (B, H, C, N, w, qscale, kscale)
CASES = {
    "C200_N5_w2": (2, 2, 200, 5, 2, 1.0, 0.5),
    "C300_N4_w3": (1, 2, 300, 4, 3, 1.0, 1.0),
    "C300_N4_w3_q4": (1, 2, 300, 4, 3, 4.0, 0.5),
    "C520_N3_w9": (1, 1, 520, 3, 9, 2.0, 1.0),
    "C64_N6_w4": (1, 2, 64, 6, 4, 1.0, 1.0),
    "C280_N5_w2": (1, 2, 280, 5, 2, 1.0, 0.5),  # 24-row chunk tails
}


def _wl(name):
    B, H, C, N, w, qs, ks = CASES[name]
    return Workload(name, 1200 + sorted(CASES).index(name), B=B, H=H, d=128, C=C, N=N, w=w, dtype="bf16",
                    qscale=qs, kscale=ks)


@pytest.mark.parametrize("name", sorted(CASES))
def test_all_kept_is_bitwise_dense(name):
    wl = _wl(name)
    ones = torch.ones(rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w), dtype=torch.uint8)
    _, out, lse, (qd, kd, vd, S, z) = _run(wl, ones)
    ref, ref_lse = rha.hybrid_fwd(qd, kd, vd, S, z, wl.C, wl.w, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


@pytest.mark.parametrize("density", [0.85, 0.5, 0.15])
@pytest.mark.parametrize("name", sorted(CASES))
def test_random_mask_against_oracle(name, density):
    wl = _wl(name)
    shape = rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w)
    mask = gen_block_mask(shape, density, seed=wl.wid * 10 + int(density * 100))
    (q, k, v), out, lse, _ = _run(wl, mask)
    ref, den = oracle.hybrid_block_sparse_batched(to64(q), to64(k), to64(v), wl.C, wl.w, mask.numpy(),
                                                  return_den=True)
    o = to64(out)
    g = rel_l2(o, ref)
    assert g <= TOL["bf16"], f"rel-L2 {g:.3e}"
    empty = den == 0
    full = ~empty
    # per (b, h, chunk) over rows with weight
    pc = per_chunk_rel_l2(np.where(empty[..., None], 0.0, o), ref, wl.C)
    assert np.nanmax(pc) <= TOL["bf16"], f"worst chunk {np.nanmax(pc):.3e}"
    assert np.all(o[empty] == 0)
    lg = to64(lse)
    assert np.all(np.isneginf(lg[empty]))
    assert np.abs(lg[full] - np.log(den[full])).max() <= 1e-2
    print(f"{name} density {density}: rel-L2 {g:.3e}, {empty.sum()} rows without weight")


@pytest.mark.parametrize("name", ["C200_N5_w2", "C300_N4_w3"])
def test_all_pruned_is_linear_only(name):
    wl = _wl(name)
    zeros = torch.zeros(rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w), dtype=torch.uint8)
    (q, k, v), out, lse, _ = _run(wl, zeros)
    ref = oracle.hybrid_block_sparse_batched(to64(q), to64(k), to64(v), wl.C, wl.w, zeros.numpy())
    o = to64(out)
    assert np.all(o[:, :, : wl.w * wl.C] == 0)
    assert rel_l2(o, ref) <= TOL["bf16"]


@pytest.mark.timeout(600)
def test_wan13b_all_kept_bitwise_and_half_kept_sampled():
    wl = CONFIGS["wan13b"]
    print(f"[parity] sparse wan13b: B{wl.B} H{wl.H} C{wl.C} N{wl.N} w{wl.w}", flush=True)
    q, k, v = gen_qkv(wl)
    shape = rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w)
    ones = torch.ones(shape, dtype=torch.uint8)
    _, out1, _, (qd, kd, vd, S, z) = _run(wl, ones, q, k, v)
    dense = rha.hybrid_fwd(qd, kd, vd, S, z, wl.C, wl.w)
    torch.cuda.synchronize()
    assert torch.equal(out1, dense)
    mask = gen_block_mask(shape, 0.5, seed=31)
    out = rha.hybrid_fwd_sparse(qd, kd, vd, S, z, wl.C, wl.w, mask.to(DEV))
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    rng = np.random.default_rng(5)
    got, want = [], []
    og = out.cpu()
    for h in range(0, wl.H, 3):
        Sh, zh = oracle.state_scan(k64[0, h], v64[0, h], wl.C, wl.w)
        rows = np.unique(np.concatenate([[0, 255, 256, 1559, 1560, wl.L - 1], rng.integers(0, wl.L, 24)]))
        want.append(oracle.hybrid_block_sparse_rows(q64[0, h], k64[0, h], v64[0, h], wl.C, wl.w, mask[0, h].numpy(),
                                                    rows, S=Sh, z=zh))
        got.append(og[0, h, rows].double().numpy())
    g = rel_l2(np.concatenate(got), np.concatenate(want))
    print(f"[parity] sparse wan13b half kept: sampled rel-L2 {g:.3e}", flush=True)
    assert g <= TOL["bf16"]
