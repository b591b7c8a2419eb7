"""The allocation-free split-KV entry point (fa_fwd_splitkv_qk_noalloc) against the split-KV
entry point with a caller workspace (fa_fwd_splitkv_qk), through the C ABI.

Both run the same kernels with the same split count, so their outputs must agree bit for
bit; the second call of each pair runs a smaller problem on the static scratch that the
first one left dirty, and is also held to the oracle's tolerances.
"""

import ctypes

import numpy as np
import pytest

import workloads as wl
from gpu_util import compare, scale_of, to_device, to_host
from oracle import attention_forward

pytestmark = pytest.mark.gpu


def _inputs(B, H, Nq, Nk, d, dtype, seed):
    q = wl.random_tensor((B, H, Nq, d), dtype, [seed, 1])
    k = wl.random_tensor((B, H, Nk, d), dtype, [seed, 2])
    v = wl.random_tensor((B, H, Nk, d), dtype, [seed, 3])
    return q, k, v


def _call_c(lib, fn, tq, tk, tv, o, lse, splits, extra=()):
    """One call straight through the C entry point (no binding logic in between)."""
    import torch

    B, H, Nq, d = tq.shape
    Nk = tk.shape[2]
    dt = 2 if tq.dtype == torch.bfloat16 else 1
    st = torch.cuda.current_stream().cuda_stream
    args = [tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(), *extra,
            B, H, Nq, Nk, d, ctypes.c_float(1.0 / d ** 0.5), dt, splits, ctypes.c_void_p(st)]
    return fn(*args)


# (B, H, Nq, Nk, d, dtype, splits): each pair's second problem is smaller than its first
PAIRS = [
    ((4, 16, 1, 16384, 128, "bf16", 0), (2, 4, 1, 5000, 128, "bf16", 0)),          # decode shapes
    ((1, 8, 512, 8192, 128, "fp16", 6), (1, 2, 100, 3000, 64, "fp16", 3)),         # chunks of queries
    ((1, 4, 2048, 2048, 64, "bf16", 0), (1, 1, 700, 700, 128, "bf16", 4)),         # square, ragged tail
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_entry_point_on_two_calls(gpu_lib, first, second):
    import torch

    lib = gpu_lib.load()
    for i, (B, H, Nq, Nk, d, dtype, splits) in enumerate((first, second)):
        q, k, v = _inputs(B, H, Nq, Nk, d, dtype, seed=1000 * i + Nk)
        tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
        tdt = tq.dtype
        code = 2 if tdt == torch.bfloat16 else 1
        used = splits if splits else lib.fa_fwd_splitkv_qk_splits(B, H, Nq, Nk, d, code)
        need = lib.fa_fwd_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, code, used)
        assert used > 1 and 0 < need <= gpu_lib.NOALLOC_SCRATCH_BYTES, (used, need)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o_ws, o_na = torch.empty_like(tq), torch.full_like(tq, float("nan"))
        l_ws = torch.empty(B, H, Nq, dtype=torch.float32, device="cuda")
        l_na = torch.full_like(l_ws, float("nan"))
        assert _call_c(lib, lib.fa_fwd_splitkv_qk, tq, tk, tv, o_ws, l_ws, used, (ws.data_ptr(), need)) == 0
        assert _call_c(lib, lib.fa_fwd_splitkv_qk_noalloc, tq, tk, tv, o_na, l_na, used) == 0
        torch.cuda.synchronize()
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), f"call {i}: O differs"
        assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32)), f"call {i}: LSE differs"
        if i == 1:   # the call after a larger one, on the scratch it left behind: oracle parity
            O_ref = np.empty_like(q)
            L_ref = np.empty(q.shape[:3])
            for b in range(B):
                for h in range(H):
                    O_ref[b, h], L_ref[b, h] = attention_forward(q[b, h], k[b, h], v[b, h], scale_of(d))
            compare(to_host(o_na), l_na.cpu().numpy().astype(np.float64), O_ref, L_ref, dtype,
                    f"noalloc second call {second}")


def test_noalloc_too_large_is_rejected_before_launch(gpu_lib):
    import torch

    lib = gpu_lib.load()
    # 8 splits of 8192 query rows at d = 128 need more than the static scratch
    B, H, Nq, Nk, d = 1, 8, 1024, 8192, 128
    t = torch.zeros(B, H, Nq, d, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(B, H, Nk, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, H, Nq, dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.FaError) as e:
        gpu_lib.fa_fwd_splitkv_noalloc(t, kv, kv, torch.empty_like(t), lse, splits=8)
    assert e.value.status == 9
