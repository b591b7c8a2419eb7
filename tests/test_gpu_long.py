"""GPU parity at the longest sequences the pages speak of.

"从零理解Flash Attention中的online softmax" (section 10) reports sequences up to 128K supported.
Here N = 131072 keys per head: 1024 key tiles of 128, so the running maximum, the two row
sums and the unnormalised accumulator are carried through a thousand tile updates.  The
oracle computes sampled rows exactly (fp64, all keys); the rows include the first and last
ones, the rows at tile and workgroup edges and seeded random rows.
"""

import numpy as np
import pytest

import workloads as wl
from gpu_util import compare, scale_of, to_device, to_host
from oracle import attention_rows

pytestmark = pytest.mark.gpu

LONG_N = 131072


def _rows(N, seed, count=32):
    fixed = [0, 1, 127, 128, 255, 256, N // 2, N - 257, N - 256, N - 2, N - 1]
    rng = np.random.default_rng([seed, 6])
    extra = rng.choice(N, size=count - len(fixed), replace=False)
    return np.unique(np.concatenate([np.array(fixed), extra])).astype(np.int64)


def _check_rows(o, lse, q, k, v, scale, dtype, causal, seed, what):
    import torch

    worst = {}
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            rows = _rows(q.shape[2], seed + 7 * h + 1000 * b)
            rr = torch.from_numpy(rows).cuda()
            Og = to_host(o[b, h].index_select(0, rr))
            Lg = lse[b, h].index_select(0, rr).cpu().numpy().astype(np.float64)
            O_ref, L_ref = attention_rows(q[b, h], k[b, h], v[b, h], scale, rows, causal=causal)
            s = compare(Og, Lg, O_ref, L_ref, dtype, f"{what} b{b} h{h}")
            worst = {key: max(worst.get(key, 0), val) for key, val in s.items()}
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()
    print(f"{what}: worst over heads {worst}")


@pytest.mark.parametrize("dtype,d,causal", [
    ("bf16", 128, False),
    ("bf16", 128, True),
    ("fp16", 128, False),
    ("bf16", 64, False),
])
def test_long_sequence_sampled_rows(gpu_lib, dtype, d, causal):
    import torch

    B, H, N = 1, 2, LONG_N
    seed = 131 + d + (1 if causal else 0)
    q, k, v = (wl.random_tensor((B, H, N, d), dtype, [seed, t]) for t in (1, 2, 3))
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv, causal=causal)
    torch.cuda.synchronize()
    _check_rows(o, lse, q, k, v, scale_of(d), dtype, causal, seed,
                f"N={N} d={d} {dtype}{' causal' if causal else ''}")


def test_long_single_head_splitkv(gpu_lib):
    """One 128K head with its key range cut into 4 parts of 32768 keys, each computed on its
    own and merged by LSE.  (The chooser would not split it: its 1024 query blocks already
    fill the chip.)"""
    import torch

    B, H, N, d, dtype = 1, 1, LONG_N, 128, "bf16"
    seed = 4242
    q, k, v = (wl.random_tensor((B, H, N, d), dtype, [seed, t]) for t in (1, 2, 3))
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    assert gpu_lib.fa_fwd_splitkv_splits(B, H, N, d, torch.bfloat16) == 1
    o, lse = gpu_lib.fa_fwd_splitkv(tq, tk, tv, splits=4)
    torch.cuda.synchronize()
    _check_rows(o, lse, q, k, v, scale_of(d), dtype, False, seed, f"N={N} split-KV x4")
