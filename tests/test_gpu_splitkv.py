"""GPU parity of the split-KV forward (key ranges computed separately, merged by their
LSE) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

import workloads as wl
from gpu_util import compare, scale_of, to_device, to_host
from oracle import attention_forward, attention_rows

pytestmark = pytest.mark.gpu


def _qkv(B, H, N, d, dtype, seed):
    return tuple(wl.random_tensor((B, H, N, d), dtype, [seed, t]) for t in (1, 2, 3))


def _oracle_full(q, k, v, scale):
    O = np.empty_like(q)
    L = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            O[b, h], L[b, h] = attention_forward(q[b, h], k[b, h], v[b, h], scale)
    return O, L


@pytest.mark.parametrize("B,H,N,d,dtype,splits", [
    (1, 2, 1000, 128, "bf16", 4),
    (1, 1, 4097, 128, "fp16", 7),
    (2, 3, 777, 64, "bf16", 3),
    (1, 4, 2048, 64, "fp16", 0),
    (1, 1, 300, 128, "bf16", 64),     # clamped to the 5 key tiles
    (1, 1, 129, 128, "bf16", 2),      # the second split holds one tile with one key
    (1, 2, 576, 128, "bf16", 4),      # 9 tiles in splits of 3: the last split is empty
])
def test_splitkv_parity(gpu_lib, B, H, N, d, dtype, splits):
    import torch

    q, k, v = _qkv(B, H, N, d, dtype, seed=N + 13 * splits)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd_splitkv(tq, tk, tv, splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    compare(to_host(o), lse.cpu().numpy().astype(np.float64), O_ref, L_ref, dtype, f"splits={splits} N={N}")


def test_one_split_is_the_plain_forward_bitwise(gpu_lib):
    import torch

    q, k, v = _qkv(2, 4, 1500, 128, "bf16", seed=3)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = gpu_lib.fa_fwd(tq, tk, tv)
    o2, l2 = gpu_lib.fa_fwd_splitkv(tq, tk, tv, splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_splitkv_deterministic(gpu_lib):
    import torch

    q, k, v = _qkv(1, 2, 3000, 64, "bf16", seed=5)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = gpu_lib.fa_fwd_splitkv(tq, tk, tv, splits=5)
    o2, l2 = gpu_lib.fa_fwd_splitkv(tq, tk, tv, splits=5)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_splitkv_long_single_head_sampled(gpu_lib):
    # One head of 16384 keys: the plain grid has 128 workgroups for 256 CUs; the chooser
    # splits it.  Checked on sampled rows; timing against the plain forward is printed.
    import torch

    N, d, dtype = 16384, 128, "bf16"
    splits = gpu_lib.fa_fwd_splitkv_splits(1, 1, N, d, torch.bfloat16)
    assert splits > 1
    q, k, v = _qkv(1, 1, N, d, dtype, seed=77)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd_splitkv(tq, tk, tv)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 127, 128, 8191, N - 1} | set(np.random.default_rng(1).choice(N, 59, replace=False).tolist())))
    rr = torch.from_numpy(rows).cuda()
    O_ref, L_ref = attention_rows(q[0, 0], k[0, 0], v[0, 0], scale_of(d), rows)
    compare(to_host(o[0, 0].index_select(0, rr)), lse[0, 0].index_select(0, rr).cpu().numpy().astype(np.float64),
            O_ref, L_ref, dtype, f"N={N} splits={splits}")

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ws = torch.empty(gpu_lib.fa_fwd_splitkv_workspace_bytes(1, 1, N, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    t_plain = timed(lambda: gpu_lib.fa_fwd(tq, tk, tv, o, lse))
    t_split = timed(lambda: gpu_lib.fa_fwd_splitkv(tq, tk, tv, o, lse, workspace=ws))
    print(f"B=1 H=1 N={N}: plain {t_plain:.3f} ms, split-KV x{splits} {t_split:.3f} ms")


@pytest.mark.parametrize("B,H,Nq,Nk,d,dtype,splits", [
    (2, 4, 1, 5000, 128, "bf16", 0),      # decode: one query per head
    (1, 3, 1, 777, 64, "fp16", 5),
    (1, 2, 7, 3000, 128, "fp16", 0),      # a few new queries against a long history
    (2, 2, 300, 100, 128, "bf16", 1),     # more queries than keys, no split
    (1, 2, 130, 4097, 64, "bf16", 9),
    (2, 4, 1, 5000, 128, "bf16", 1),      # decode unsplit: the block's waves split the keys
    (1, 2, 20, 3000, 64, "fp16", 1),
])
def test_splitkv_unequal_lengths(gpu_lib, B, H, Nq, Nk, d, dtype, splits):
    import torch

    q = wl.random_tensor((B, H, Nq, d), dtype, [Nq, Nk, 1])
    k = wl.random_tensor((B, H, Nk, d), dtype, [Nq, Nk, 2])
    v = wl.random_tensor((B, H, Nk, d), dtype, [Nq, Nk, 3])
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd_splitkv(tq, tk, tv, splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    compare(to_host(o), lse.cpu().numpy().astype(np.float64), O_ref, L_ref, dtype, f"Nq={Nq} Nk={Nk} splits={splits}")
