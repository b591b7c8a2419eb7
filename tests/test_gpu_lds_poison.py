"""Forward parity on the LDS-poison debug build (libfa_poison.so): every K/V tile buffer is
filled with NaN right before its copy is issued, so a read that races a copy -- a missing
wait or barrier, a stage reused too early -- produces NaN outputs, which the comparison
rejects.  Every compiled forward kernel is forced through FA_TILE, causal and not, at
ragged lengths, plus the split-KV path."""

import ctypes
import os

import numpy as np
import pytest

import workloads as wl
from gpu_util import compare, scale_of, to_device, to_host
from oracle import attention_forward

pytestmark = pytest.mark.gpu

# (tile, d, dtype): every compiled bf16/fp16 kernel, and the fp32 one
VARIANTS = [("256,128,8", 128, "bf16"), ("128,64,4", 128, "bf16"), ("128,32,4", 128, "fp16"),
            ("256,128,8", 64, "bf16"), ("128,128,4", 64, "fp16"), ("128,64,4", 64, "bf16"),
            ("32,32,4", 64, "fp32")]


@pytest.fixture(scope="module")
def poison_lib(gpu_lib):
    return gpu_lib.load_variant(gpu_lib.POISON_LIB_PATH)


def _oracle(q, k, v, d, causal):
    O = np.empty_like(q)
    L = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            O[b, h], L[b, h] = attention_forward(q[b, h], k[b, h], v[b, h], scale_of(d), causal=causal)
    return O, L


def _fwd(lib, tq, tk, tv, causal):
    import torch

    B, H, N, d = tq.shape
    code = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[tq.dtype]
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=tq.device)
    fn = lib.fa_fwd_causal if causal else lib.fa_fwd
    st = fn(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
            ctypes.c_float(scale_of(d)), code, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    torch.cuda.synchronize()
    return to_host(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("tile,d,dtype", VARIANTS, ids=[f"{t}-d{d}-{dt}" for t, d, dt in VARIANTS])
def test_poisoned_forward_parity(poison_lib, monkeypatch, tile, d, dtype, causal):
    monkeypatch.setenv("FA_TILE", tile)
    # one key; ragged tails over several tiles; on the non-causal 4-wave plans, a one-row last
    # block with at least 32 key tiles, whose waves split the keys (their V copies poisoned too)
    Ns = (1, 300, 1031) + ((4097,) if not causal and tile.endswith(",4") and dtype != "fp32" else ())
    for N in Ns:
        B, H = 1, 2
        q, k, v = (wl.random_tensor((B, H, N, d), dtype, [N, d, 31, t]) for t in (1, 2, 3))
        O, L = _fwd(poison_lib, *(to_device(x, dtype) for x in (q, k, v)), causal)
        O_ref, L_ref = _oracle(q, k, v, d, causal)
        compare(O, L, O_ref, L_ref, dtype, f"poison FA_TILE={tile} d={d} {dtype} N={N} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_poisoned_tail_first_parity(gpu_lib, poison_lib, d):
    # the last row of every head computed ahead of the 8-wave launch (split-KV workgroups
    # over the head's key ranges, partials parked in O, merged), every stage poisoned
    B, H, N, dtype = 2, 8, 4097, "bf16"
    assert gpu_lib.fa_fwd_plan(B, H, N, d, gpu_lib.FA_BF16)["tail_kv_splits"] > 1
    q, k, v = (wl.random_tensor((B, H, N, d), dtype, [N, d, 41, t]) for t in (1, 2, 3))
    O, L = _fwd(poison_lib, *(to_device(x, dtype) for x in (q, k, v)), False)
    O_ref, L_ref = _oracle(q, k, v, d, False)
    compare(O, L, O_ref, L_ref, dtype, f"poison tail first d={d}")


def test_poisoned_splitkv_parity(poison_lib):
    import torch

    B, H, Nq, Nk, d, dtype = 2, 2, 5, 3000, 128, "bf16"
    q = wl.random_tensor((B, H, Nq, d), dtype, [Nq, Nk, 1])
    k = wl.random_tensor((B, H, Nk, d), dtype, [Nq, Nk, 2])
    v = wl.random_tensor((B, H, Nk, d), dtype, [Nq, Nk, 3])
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    splits = 7
    need = poison_lib.fa_fwd_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, 2, splits)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    st = poison_lib.fa_fwd_splitkv_qk(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      ws.data_ptr(), need, B, H, Nq, Nk, d, ctypes.c_float(scale_of(d)), 2, splits,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    torch.cuda.synchronize()
    O_ref, L_ref = _oracle(q, k, v, d, False)
    compare(to_host(o), lse.cpu().numpy().astype(np.float64), O_ref, L_ref, dtype, "poison split-KV")


def test_poison_build_is_a_different_library(gpu_lib, poison_lib):
    assert os.path.exists(gpu_lib.POISON_LIB_PATH)
    assert os.path.getsize(gpu_lib.POISON_LIB_PATH) != os.path.getsize(gpu_lib.LIB_PATH)
    assert poison_lib.fa_version() == gpu_lib.load().fa_version()
