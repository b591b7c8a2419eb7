"""Seeded random shapes through every forward entry point, against the oracle: sequence
lengths that land anywhere relative to the query and key tiles, small and odd B and H,
both head dims and both 16-bit types, causal or not, and split counts the chooser would
not pick.  The shapes are drawn once from a fixed seed, so the cases are the same on
every run."""

import numpy as np
import pytest

import workloads as wl
from gpu_util import compare, run_fwd, scale_of, to_device, to_host
from oracle import attention_forward

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)
CASES = []
for i in range(24):
    CASES.append(dict(
        B=int(_rng.integers(1, 4)), H=int(_rng.integers(1, 5)), N=int(_rng.integers(1, 700)),
        d=int(_rng.choice([64, 128])), dtype=str(_rng.choice(["bf16", "fp16"])),
        causal=bool(_rng.integers(0, 2)), splits=int(_rng.integers(2, 9)),
        scale=float(_rng.choice([0.0, 0.05, 0.3])), seed=i))


def _inputs(c):
    return tuple(wl.random_tensor((c["B"], c["H"], c["N"], c["d"]), c["dtype"], [c["seed"], 900 + t])
                 for t in (1, 2, 3))


def _oracle(q, k, v, scale, causal):
    B, H = q.shape[:2]
    O = np.empty_like(q)
    L = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = attention_forward(q[b, h], k[b, h], v[b, h], scale, causal=causal)
    return O, L


def _name(c):
    return "B{B}H{H}N{N}d{d}-{dtype}-{}-s{scale}".format("causal" if c["causal"] else "full", **c)


@pytest.mark.parametrize("c", CASES, ids=_name)
def test_random_shape_forward(gpu_lib, c):
    q, k, v = _inputs(c)
    scale = c["scale"] or scale_of(c["d"])
    O, L = run_fwd(gpu_lib, q, k, v, c["dtype"], causal=c["causal"], scale=scale)
    O_ref, L_ref = _oracle(q, k, v, scale, c["causal"])
    compare(O, L, O_ref, L_ref, c["dtype"], _name(c))


@pytest.mark.parametrize("c", [c for c in CASES if not c["causal"]], ids=_name)
def test_random_shape_splitkv(gpu_lib, c):
    import torch

    q, k, v = _inputs(c)
    scale = c["scale"] or scale_of(c["d"])
    tq, tk, tv = (to_device(x, c["dtype"]) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd_splitkv(tq, tk, tv, splits=c["splits"], scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = _oracle(q, k, v, scale, False)
    compare(to_host(o), lse.cpu().numpy().astype(np.float64), O_ref, L_ref, c["dtype"],
            _name(c) + f"-splits{c['splits']}")


# Tail first: seeded grids of whole rounds of 256-row blocks plus 1..128 last rows per head
# (the chooser computes those rows ahead of the 8-wave launch); checked on sampled rows that
# include every last row and the first 256 rows of the head, where the partials are parked.
_trng = np.random.default_rng(20261203)
TAIL_CASES = []
for i in range(8):
    bh = int(_trng.choice([8, 16, 32]))
    k = int(_trng.choice([256 // bh, 512 // bh]))   # whole rounds of 256 blocks
    B = int(_trng.choice([1, 2]))
    TAIL_CASES.append(dict(B=B, H=bh // B, N=256 * k + int(_trng.integers(1, 129)),
                           d=int(_trng.choice([64, 128])), dtype=str(_trng.choice(["bf16", "fp16"])), seed=100 + i))


@pytest.mark.parametrize("c", TAIL_CASES, ids=lambda c: "B{B}H{H}N{N}d{d}-{dtype}".format(**c))
def test_random_tail_first(gpu_lib, c):
    import torch

    from oracle import attention_rows

    B, H, N, d, dtype = c["B"], c["H"], c["N"], c["d"], c["dtype"]
    code = {"bf16": gpu_lib.FA_BF16, "fp16": gpu_lib.FA_F16}[dtype]
    plan = gpu_lib.fa_fwd_plan(B, H, N, d, code)
    assert plan["waves"] == 8 and plan["tail_kv_splits"] > 1, plan
    q, k, v = (wl.random_tensor((B, H, N, d), dtype, [c["seed"], 910 + t]) for t in (1, 2, 3))
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(c["seed"])
    n_main = N // 256 * 256
    for b, h in ((0, 0), (B - 1, H - 1), (0, H // 2)):
        rows = np.unique(np.concatenate([np.arange(0, 256, 7), np.arange(n_main, N), rng.choice(N, 24, replace=False)]))
        rr = torch.from_numpy(rows).cuda()
        Og = to_host(o[b, h].index_select(0, rr))
        Lg = lse[b, h].index_select(0, rr).cpu().numpy().astype(np.float64)
        O_ref, L_ref = attention_rows(q[b, h], k[b, h], v[b, h], scale_of(d), rows)
        compare(Og, Lg, O_ref, L_ref, dtype, "tail first B{B}H{H}N{N}d{d}-{dtype} b{b} h{h}".format(b=b, h=h, **c))
