"""The binding refuses host tensors (and tensors of another shape, dtype or layout) for every
pointer it hands to the library, before any C call: a host pointer would reach a kernel as an
unmapped device address.  Nothing here launches a kernel."""

import pytest

pytestmark = pytest.mark.gpu


def _dev_qkv(B=1, H=2, N=64, d=64, dtype=None):
    import torch

    dtype = dtype or torch.bfloat16
    return tuple(torch.zeros(B, H, N, d, dtype=dtype, device="cuda") for _ in range(3))


def test_forward_outputs_on_the_host_are_refused(gpu_lib):
    import torch

    q, k, v = _dev_qkv()
    with pytest.raises(ValueError, match="o must be a device tensor"):
        gpu_lib.fa_fwd(q, k, v, o=torch.empty_like(q, device="cpu"))
    with pytest.raises(ValueError, match="lse must be a device tensor"):
        gpu_lib.fa_fwd(q, k, v, lse=torch.empty(1, 2, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="not contiguous"):
        gpu_lib.fa_fwd(q, k, v, o=torch.empty(1, 2, 64, 128, dtype=q.dtype, device="cuda")[..., ::2])
    with pytest.raises(ValueError, match="v must be a device tensor"):
        gpu_lib.fa_fwd(q, k, v.cpu())


def test_splitkv_and_noalloc_buffers_on_the_host_are_refused(gpu_lib):
    import torch

    q, k, v = _dev_qkv(N=1000)
    with pytest.raises(ValueError, match="workspace must be a device tensor"):
        gpu_lib.fa_fwd_splitkv(q, k, v, splits=4, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="lse must be a device tensor"):
        gpu_lib.fa_fwd_splitkv(q[:, :, :1].contiguous(), k, v, lse=torch.empty(1, 2, 1))
    with pytest.raises(ValueError, match="o must be a device tensor"):
        gpu_lib.fa_fwd_splitkv_noalloc(q[:, :, :1].contiguous(), k, v, o=torch.empty(1, 2, 1, 64, dtype=q.dtype))


def test_backward_buffers_on_the_host_are_refused(gpu_lib):
    import torch

    q, k, v = _dev_qkv()
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 2, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="lse must be a device tensor"):
        gpu_lib.fa_bwd(q, k, v, o, lse.cpu(), o)
    with pytest.raises(ValueError, match="dk must be a device tensor"):
        gpu_lib.fa_bwd(q, k, v, o, lse, o, dk=torch.empty(q.shape, dtype=q.dtype))
    with pytest.raises(ValueError, match="workspace must be a device tensor"):
        gpu_lib.fa_bwd(q, k, v, o, lse, o, workspace=torch.empty(4096, dtype=torch.uint8))


def test_fp8_buffers_on_the_host_are_refused(gpu_lib):
    import torch

    x = torch.zeros(1, 2, 100, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="x8 must be a device tensor"):
        gpu_lib.fa_quantize_fp8(x, x8=torch.empty(1, 2, 100, 128, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales must be a device tensor"):
        gpu_lib.fa_quantize_fp8(x, scales=torch.empty(1, 2, 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="not contiguous"):
        gpu_lib.fa_quantize_fp8(x, scales=torch.empty(1, 2, 4, dtype=torch.float32, device="cuda")[..., ::2])
    c = torch.zeros(1, 2, 100, 128, dtype=torch.uint8, device="cuda")
    vt = torch.zeros(1, 2, 128, 128, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, 2, 2, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="v_scale must be a device tensor"):
        gpu_lib.fa_fwd_fp8(c, c, vt, s, s, s.cpu())
    with pytest.raises(ValueError, match="lse must be a device tensor"):
        gpu_lib.fa_fwd_fp8(c, c, vt, s, s, s, lse=torch.empty(1, 2, 100))
