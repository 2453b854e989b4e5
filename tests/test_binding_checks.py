"""The Python binding refuses tensors the kernels cannot take -- host tensors,
tensors on another device, state or lse buffers of the wrong dtype or shape --
with a ValueError raised before any call into the library.

The host-tensor cases run without a GPU: each raises before librha.so is
asked to do anything.  The dtype, shape and device cases need GPU tensors.
"""
import pytest
import torch

import linear_attention_video_chunked_amd as rha

B, H, C, N, d = 1, 2, 64, 3, 128


def host_qkv(dtype=torch.bfloat16):
    return tuple(torch.zeros((B, H, C * N, d), dtype=dtype) for _ in range(3))


def host_state():
    return torch.zeros((B, H, N, d, d)), torch.zeros((B, H, N, d))


def test_state_scan_refuses_host_tensors():
    _, k, v = host_qkv()
    with pytest.raises(ValueError, match="GPU tensor"):
        rha.state_scan(k, v, C, 2)


def test_hybrid_fwd_refuses_host_tensors():
    q, k, v = host_qkv()
    S, z = host_state()
    with pytest.raises(ValueError, match="GPU tensor"):
        rha.hybrid_fwd(q, k, v, S, z, C, 2)


def test_sparse_bidir_bwd_refuse_host_tensors():
    q, k, v = host_qkv()
    S, z = host_state()
    mask = torch.ones(rha.sparse_mask_shape(B, H, C, N, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        rha.hybrid_fwd_sparse(q, k, v, S, z, C, 2, mask)
    with pytest.raises(ValueError, match="GPU tensor"):
        rha.state_scan_bidir(k, v, C, 2)
    with pytest.raises(ValueError, match="GPU tensor"):
        rha.hybrid_fwd_bidir(q, k, v, (S, z, S, z), C, 2)
    lse = torch.zeros((B, H, C * N))
    with pytest.raises(ValueError, match="GPU tensor"):
        rha.hybrid_bwd(q, k, v, S, z, q, lse, q, C, 2)


def test_stream_step_refuses_host_tensors():
    st = rha.StreamState(B, H, d, C, 2, device="cpu", split=False)
    q = torch.zeros((B, H, C, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        rha.stream_step(st, q, q, q)
    assert st.t == 0


gpu = pytest.mark.gpu


def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@gpu
def test_wrong_state_dtype_shape_and_device_refused():
    _gpu_or_skip()
    q, k, v = (t.cuda() for t in host_qkv())
    S, z = (t.cuda() for t in host_state())
    with pytest.raises(ValueError, match="float32"):
        rha.hybrid_fwd(q, k, v, S.double(), z, C, 2)
    with pytest.raises(ValueError, match="shape"):
        rha.hybrid_fwd(q, k, v, S[:, :, :2].contiguous(), z, C, 2)
    with pytest.raises(ValueError, match="on"):
        rha.hybrid_fwd(q, k, v, S.cpu(), z, C, 2)
    with pytest.raises(ValueError, match="float32"):
        rha.hybrid_fwd(q, k, v, S, z, C, 2, lse=torch.zeros((B, H, C * N), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="float32"):
        rha.state_scan(k, v, C, 2, S=S.half(), z=z)
    lse = torch.zeros((B, H, C * N), device="cuda")
    with pytest.raises(ValueError, match="float32"):
        rha.hybrid_bwd(q, k, v, S.half(), z, q, lse, q, C, 2)


@gpu
def test_stream_state_on_another_device_refused():
    _gpu_or_skip()
    st = rha.StreamState(B, H, d, C, 2, device="cpu", split=False)
    q = torch.zeros((B, H, C, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="stream state"):
        rha.stream_step(st, q, q, q)
    assert st.t == 0
