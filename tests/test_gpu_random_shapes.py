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
