"""rha_stream_step_noalloc against rha_stream_step with a caller workspace,
through the C ABI: two calls in a row on one GPU, the second with a smaller
problem, each equal bitwise to the workspace call (the same kernels, split
the same way) -- output, and S, z after the commit."""
import pytest
import torch

import linear_attention_video_chunked_amd as rha
from synth import CONFIGS, Workload, gen_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _chunk(x, t, C):
    return x[:, :, t * C:(t + 1) * C].contiguous()


def _pair(wl, q, k, v, t_call):
    """Two stream states fed the same chunks 0 .. t_call-1 with the workspace
    step; chunk t_call then goes through each entry point."""
    ref = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV, split=True)
    got = rha.StreamState(wl.B, wl.H, wl.d, wl.C, wl.w, device=DEV, split=True)
    for t in range(t_call):
        for st in (ref, got):
            rha.stream_step(st, _chunk(q, t, wl.C), _chunk(k, t, wl.C), _chunk(v, t, wl.C))
    qt, kt, vt = (_chunk(x, t_call, wl.C) for x in (q, k, v))
    o_ref = rha.stream_step(ref, qt, kt, vt)
    o_got = torch.empty_like(qt)
    lse = torch.empty((wl.B, wl.H, wl.C), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rha.stream_step_noalloc(got, qt, kt, vt, out=o_got, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return ref, got, o_ref, o_got


def test_noalloc_step_equals_workspace_step_twice_then_smaller():
    big = CONFIGS["stream"].replace(N=11)  # 12 heads, 1560-token chunks, 9-chunk window
    small = Workload("noalloc_small", 960, B=1, H=2, d=128, C=200, N=5, w=3, dtype="bf16", kscale=0.5)
    need_big = None
    for wl, t_call in ((big, 10), (small, 4)):
        print(f"[noalloc] H{wl.H} C{wl.C} w{wl.w}: chunk {t_call}", flush=True)
        q, k, v = (x.to(DEV) for x in gen_qkv(wl))
        ref, got, o_ref, o_got = _pair(wl, q, k, v, t_call)
        assert torch.equal(o_got, o_ref)
        assert torch.equal(got.S, ref.S) and torch.equal(got.z, ref.z)
        assert got.t == ref.t == t_call + 1
        assert torch.equal(got.k_cache, ref.k_cache) and torch.equal(got.v_cache, ref.v_cache)
        if need_big is None:  # the first problem does use the scratch (a split step)
            need_big = ref.workspace.numel() if ref.workspace is not None else 0
            assert 0 < need_big <= rha._rha.NOALLOC_SCRATCH_BYTES
