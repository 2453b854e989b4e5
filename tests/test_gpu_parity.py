"""GPU parity: librha (through its C ABI) against the fp64 oracle.

Mid-size problems are compared element by element over the whole output;
full-size workloads (Wan 2.1 1.3B / 14B shapes, the 6x horizon, its 21-chunk
limit slices) on sampled rows plus the complete state tensors.  Bars: rel-L2
<= 1e-2 for bf16 and <= 1e-4 for float32, globally and per (b, h, chunk);
lse within 1e-2 (bf16) / 1e-4 (float32) absolute of ln(denominator).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, Workload, gen_qkv
import linear_attention_video_chunked_amd as rha
from parity_utils import ALARM, TOL, GroupedRows, per_chunk_rel_l2, rel_l2, sample_rows, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
LSE_TOL = {"bf16": 1e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rha.lib()  # raises LibraryNotBuilt if librha.so is missing


def run_lib(q, k, v, C, w):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    S, z = rha.state_scan(kd, vd, C, w)
    out, lse = rha.hybrid_fwd(qd, kd, vd, S, z, C, w, return_lse=True)
    torch.cuda.synchronize()
    return out, lse, S, z


# name: (B, H, d, C, N, w, dtype, qscale, kscale)
MID = {
    "bf16_d128_C200_N5_w2": (2, 3, 128, 200, 5, 2, "bf16", 1.0, 0.5),
    "bf16_d128_C200_N5_w2_q4": (2, 3, 128, 200, 5, 2, "bf16", 4.0, 0.5),
    "bf16_d128_C40_N7_w3": (1, 2, 128, 40, 7, 3, "bf16", 1.0, 1.0),
    "bf16_d128_C300_N4_w1": (1, 2, 128, 300, 4, 1, "bf16", 1.0, 1.0),
    "bf16_d128_C300_N4_w1_q4": (1, 2, 128, 300, 4, 1, "bf16", 4.0, 0.5),
    "bf16_d128_C130_N4_w0": (1, 2, 128, 130, 4, 0, "bf16", 1.0, 1.0),
    # chunks of at least one 256-row tile: tiles run over the flat sequence and
    # span chunk edges (aligned, ragged, pure linear, window past the start)
    "bf16_d128_C256_N5_w2": (1, 2, 128, 256, 5, 2, "bf16", 1.0, 1.0),
    "bf16_d128_C333_N6_w3": (2, 2, 128, 333, 6, 3, "bf16", 1.0, 0.5),
    "bf16_d128_C333_N6_w3_q4": (1, 2, 128, 333, 6, 3, "bf16", 4.0, 0.5),
    "bf16_d128_C300_N4_w0": (1, 2, 128, 300, 4, 0, "bf16", 1.0, 1.0),
    "bf16_d128_C270_N5_w9": (1, 1, 128, 270, 5, 9, "bf16", 2.0, 1.0),
    "bf16_d128_C130_N4_w4": (1, 2, 128, 130, 4, 4, "bf16", 1.0, 1.0),
    "bf16_d128_C130_N4_w9": (1, 2, 128, 130, 4, 9, "bf16", 2.0, 1.0),
    "bf16_d128_C1_N300_w3": (1, 2, 128, 1, 300, 3, "bf16", 1.0, 1.0),
    "bf16_d128_C64_N3_w2": (1, 1, 128, 64, 3, 2, "bf16", 1.0, 1.0),
    # chunks ending 1..32 rows past a 256-row tile (the short-tail workgroups),
    # and chunks of at most 32 rows (tails only)
    "bf16_d128_C280_N6_w3": (1, 2, 128, 280, 6, 3, "bf16", 1.0, 0.5),
    "bf16_d128_C280_N5_w2_q4": (1, 2, 128, 280, 5, 2, "bf16", 4.0, 0.5),
    "bf16_d128_C513_N4_w2": (2, 1, 128, 513, 4, 2, "bf16", 1.0, 1.0),
    "bf16_d128_C288_N4_w0": (1, 2, 128, 288, 4, 0, "bf16", 1.0, 1.0),
    "bf16_d128_C24_N9_w2": (1, 3, 128, 24, 9, 2, "bf16", 1.0, 1.0),
    "bf16_d128_C32_N6_w1_q4": (1, 2, 128, 32, 6, 1, "bf16", 4.0, 1.0),
    "bf16_d64_C100_N5_w2": (1, 3, 64, 100, 5, 2, "bf16", 1.0, 1.0),
    "bf16_d64_C100_N5_w2_q4": (1, 3, 64, 100, 5, 2, "bf16", 4.0, 0.5),
    "f32_d64_C70_N5_w2": (1, 2, 64, 70, 5, 2, "f32", 1.0, 1.0),
    "f32_d128_C70_N5_w2": (1, 2, 128, 70, 5, 2, "f32", 2.0, 1.0),
    "f32_d64_C1_N100_w0": (1, 2, 64, 1, 100, 0, "f32", 1.0, 1.0),
    "f32_d64_C33_N4_w9": (1, 1, 64, 33, 4, 9, "f32", 1.0, 1.0),
}


def mid_workload(name):
    B, H, d, C, N, w, dt, qs, ks = MID[name]
    wid = 100 + sorted(MID).index(name)
    return Workload(name, wid, B=B, H=H, d=d, C=C, N=N, w=w, dtype=dt, qscale=qs, kscale=ks)


def check_full(wl: Workload, out, lse, S, z, q64, k64, v64):
    ref, den = oracle.hybrid_batched(q64, k64, v64, wl.C, wl.w, return_den=True)
    Sref, zref = oracle.state_scan_batched(k64, v64, wl.C, wl.w)
    tol = TOL[wl.dtype]
    o = to64(out)
    g = rel_l2(o, ref)
    pc = per_chunk_rel_l2(o, ref, wl.C)
    assert g <= tol, f"{wl.name}: rel-L2 {g:.3e}"
    assert pc.max() <= tol, f"{wl.name}: worst chunk rel-L2 {pc.max():.3e} at {np.unravel_index(pc.argmax(), pc.shape)}"
    assert np.abs(to64(lse) - np.log(den)).max() <= LSE_TOL[wl.dtype]
    Sg, zg = to64(S), to64(z)
    if wl.w > 0:
        assert (Sg[:, :, : wl.w] == 0).all() and (zg[:, :, : wl.w] == 0).all()
    if (Sref != 0).any():
        assert rel_l2(Sg, Sref) <= tol
        assert rel_l2(zg, zref) <= tol
    return g, pc.max()


@pytest.mark.parametrize("name", sorted(MID))
def test_mid_size_against_oracle(name):
    wl = mid_workload(name)
    q, k, v = gen_qkv(wl)
    out, lse, S, z = run_lib(q, k, v, wl.C, wl.w)
    g, worst = check_full(wl, out, lse, S, z, to64(q), to64(k), to64(v))
    print(f"{name}: rel-L2 {g:.3e}, worst chunk {worst:.3e}")


def test_tiny_config_against_oracle_and_brute_force():
    wl = CONFIGS["tiny"]
    q, k, v = gen_qkv(wl)
    out, lse, S, z = run_lib(q, k, v, wl.C, wl.w)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    check_full(wl, out, lse, S, z, q64, k64, v64)
    for b in range(wl.B):
        for h in range(wl.H):
            ref = oracle.brute_masked(q64[b, h], k64[b, h], v64[b, h], wl.C, wl.w)
            assert rel_l2(to64(out)[b, h], ref) <= TOL["f32"]


# layout cases: a windowed one and one with no window (w = 0 has its own kernel)
LAYOUT = {
    "w2": lambda: mid_workload("bf16_d128_C200_N5_w2"),
    "w0_B2": lambda: Workload("layout_w0_B2", 190, B=2, H=3, d=128, C=200, N=5, w=0, dtype="bf16"),
}


@pytest.mark.parametrize("name", sorted(LAYOUT))
def test_strided_sequence_major_layout_matches_contiguous(name):
    # [B, L, H, d] storage viewed as [B, H, L, d]
    wl = LAYOUT[name]()
    q, k, v = gen_qkv(wl)
    a_out, a_lse, a_S, a_z = run_lib(q, k, v, wl.C, wl.w)
    check_full(wl, a_out, a_lse, a_S, a_z, to64(q), to64(k), to64(v))
    qs, ks, vs = (t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (q, k, v))
    S, z = rha.state_scan(ks, vs, wl.C, wl.w)
    out = torch.empty_like(qs)
    rha.hybrid_fwd(qs, ks, vs, S, z, wl.C, wl.w, out=out)
    torch.cuda.synchronize()
    assert torch.equal(S, a_S) and torch.equal(z, a_z)
    assert torch.equal(out.contiguous(), a_out)


@pytest.mark.parametrize("name", ["bf16_d128_C300_N4_w1", "bf16_d128_C300_N4_w0"])
def test_output_guard_bands_untouched(name):
    wl = mid_workload(name)
    q0, k0, v0 = gen_qkv(wl)
    ref_out, _, ref_S, ref_z = run_lib(q0, k0, v0, wl.C, wl.w)

    def padded(x, fill):
        big = torch.full((wl.B, wl.H, wl.L + 256, wl.d), fill, dtype=x.dtype, device=DEV)
        view = big[:, :, 128: 128 + wl.L]
        view.copy_(x)
        return big, view

    _, q = padded(q0, 0.0)
    _, k = padded(k0, 0.0)
    _, v = padded(v0, 0.0)
    big, out = padded(torch.zeros_like(q0), 7.0)
    Sbig = torch.full((ref_S.numel() + 2048,), 5.0, device=DEV)
    S = Sbig[1024: 1024 + ref_S.numel()].view(ref_S.shape)
    zbig = torch.full((ref_z.numel() + 128,), 5.0, device=DEV)
    z = zbig[64: 64 + ref_z.numel()].view(ref_z.shape)
    rha.state_scan(k, v, wl.C, wl.w, S=S, z=z)
    rha.hybrid_fwd(q, k, v, S, z, wl.C, wl.w, out=out)
    torch.cuda.synchronize()
    assert (big[:, :, :128] == 7.0).all() and (big[:, :, 128 + wl.L:] == 7.0).all()
    assert (Sbig[:1024] == 5.0).all() and (Sbig[1024 + S.numel():] == 5.0).all()
    assert (zbig[:64] == 5.0).all() and (zbig[64 + z.numel():] == 5.0).all()
    assert torch.equal(S, ref_S) and torch.equal(z, ref_z)
    assert torch.equal(out, ref_out)


def test_empty_problems():
    for shape in ((0, 2, 128, 128), (1, 0, 128, 128)):
        q = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
        S, z = rha.state_scan(q, q, 64, 1)
        out = rha.hybrid_fwd(q, q, q, S, z, 64, 1)
        assert out.shape == shape
    q = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    S, z = rha.state_scan(q, q, 64, 1)
    assert rha.hybrid_fwd(q, q, q, S, z, 64, 1).shape == q.shape
    torch.cuda.synchronize()


@pytest.mark.parametrize("C", [100, 300, 280])
@pytest.mark.parametrize("alpha", [40.0, 170.0, -170.0])
def test_score_growth_within_window(alpha, C):
    # Every query shares a component along feature 0; the last key of every
    # chunk is alpha along that feature, so windows see ordinary scores first
    # and then one key scoring about 0.35 * alpha (natural log units) above
    # them.  alpha = 40 stays inside the kernels' tolerance for a stale
    # reference maximum; alpha = 170 (a ~60-nat jump, 2^86) forces reference
    # moves after accumulation, both where the linear state seeds the
    # accumulators and where it does not; -170 makes those keys vanish.
    # C = 300: query tiles that span two chunks; C = 280: a 24-row tail per
    # chunk (the short-tail workgroups, plain online maximum).
    wl = Workload("growth", 950, B=1, H=2, d=128, C=C, N=4, w=2, dtype="bf16", qscale=1.0, kscale=0.5)
    q, k, v = gen_qkv(wl)
    q = q.clone()
    k = k.clone()
    q[..., 0] += 4.0
    k[:, :, wl.C - 1:: wl.C, 0] = alpha
    out, lse, S, z = run_lib(q, k, v, wl.C, wl.w)
    check_full(wl, out, lse, S, z, to64(q), to64(k), to64(v))


def test_bitwise_deterministic():
    wl = mid_workload("bf16_d128_C200_N5_w2_q4")
    q, k, v = gen_qkv(wl)
    a = run_lib(q, k, v, wl.C, wl.w)
    b = run_lib(q, k, v, wl.C, wl.w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------------------------ full-size workloads

FULL = {
    "wan13b": CONFIGS["wan13b"],
    "wan13b_q4": CONFIGS["wan13b"].replace(name="wan13b_q4", qscale=4.0),
    "wan14b": CONFIGS["wan14b"],
    "wan14b_q4": CONFIGS["wan14b"].replace(name="wan14b_q4", qscale=4.0),
    "long": CONFIGS["long"],
    "long_q4": CONFIGS["long"].replace(name="long_q4", qscale=4.0),
    "long_slice_w0": CONFIGS["long"].replace(name="long_slice_w0", N=21, w=0),
    "long_slice_wall": CONFIGS["long"].replace(name="long_slice_wall", N=21, w=21),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_rows(name):
    wl = FULL[name]
    print(f"[parity] {name}: B{wl.B} H{wl.H} d{wl.d} C{wl.C} N{wl.N} w{wl.w}", flush=True)
    q, k, v = gen_qkv(wl)
    out, lse, S, z = run_lib(q, k, v, wl.C, wl.w)
    out2 = rha.hybrid_fwd(*(t.to(DEV) for t in (q, k, v)), S, z, wl.C, wl.w)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "run-to-run difference"
    # rows at chunk edges, 256-row tile edges, the short tail, plus random ones
    rows = sample_rows(wl.C, wl.N, 4 * wl.N, seed=wl.wid)
    Sg, zg = S.cpu(), z.cpu()
    og, lg = out.cpu(), lse.cpu()
    errs_s, worst_lse = [], 0.0
    grouped = GroupedRows(name)
    for b in range(wl.B):
        for h in range(wl.H):
            k64 = k[b, h].double().numpy()
            v64 = v[b, h].double().numpy()
            Sref, zref = oracle.state_scan(k64, v64, wl.C, wl.w)
            if wl.w > 0:
                assert (Sg[b, h, : wl.w] == 0).all()
            if (Sref != 0).any():
                errs_s.append(max(rel_l2(Sg[b, h].double().numpy(), Sref), rel_l2(zg[b, h].double().numpy(), zref)))
            ref, den = oracle.hybrid_rows(q[b, h].double().numpy(), k64, v64, wl.C, wl.w, rows, S=Sref, z=zref,
                                          return_den=True)
            got = og[b, h, rows].double().numpy()
            grouped.add_by_chunk((b, h), got, ref, rows, wl.C)
            worst_lse = max(worst_lse, float(np.abs(lg[b, h, rows].double().numpy() - np.log(den)).max()))
    print(f"[parity] {name}: state rel-L2 max {max(errs_s, default=0):.3e}, lse max abs {worst_lse:.2e}", flush=True)
    grouped.check(TOL[wl.dtype], ALARM[wl.dtype] if wl.qscale == 1.0 else None)
    assert max(errs_s, default=0.0) <= TOL[wl.dtype]
    assert worst_lse <= LSE_TOL[wl.dtype]
