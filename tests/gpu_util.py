"""Helpers for the GPU parity tests: upload exact inputs, run through the C ABI,
and compare with the oracle under the stated tolerances."""

from __future__ import annotations

import math

import numpy as np

import workloads as wl

# Max-abs tolerances on O by input dtype, and on LSE.
O_TOL = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 1e-2}
LSE_TOL = {"fp32": 1e-5, "fp16": 1e-3, "bf16": 1e-3}
MANTISSA_BITS = {"fp32": 23, "fp16": 10, "bf16": 7}


def torch_dtype(dtype: str):
    import torch

    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(x: np.ndarray, dtype: str):
    """float64 array of exactly representable values -> contiguous device tensor."""
    import torch

    arr = wl.storage_array(x, dtype)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.cuda().contiguous()


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of |x| in the output dtype (normal range)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, {"fp32": -126, "fp16": -14, "bf16": -126}[dtype])
    return 0.5 * np.exp2(e - MANTISSA_BITS[dtype])


def compare(O, L, O_ref, L_ref, dtype: str, what: str = ""):
    """Pass iff every |O - O_ref| <= tol + half an output ulp of O_ref (the output is stored
    in the input dtype, so rounding it alone costs up to half an ulp) and every
    |LSE - LSE_ref| <= LSE tol; no NaN/Inf anywhere.  Returns the error summary."""
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    assert np.all(np.isfinite(L)), f"{what}: non-finite LSE"
    err = np.abs(O - O_ref)
    bound = O_TOL[dtype] + half_ulp(O_ref, dtype)
    bad = err > bound
    lerr = np.abs(L - L_ref)
    summary = dict(max_err_o=float(err.max()) if err.size else 0.0,
                   n_above_bare_tol=int((err > O_TOL[dtype]).sum()),
                   max_err_lse=float(lerr.max()) if lerr.size else 0.0)
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: O error {err[idx]:.3e} > bound {bound[idx]:.3e} at {idx} "
                             f"(got {O[idx]}, ref {O_ref[idx]}); {int(bad.sum())} elements out; {summary}")
    assert lerr.max(initial=0) <= LSE_TOL[dtype], f"{what}: LSE error {lerr.max():.3e}; {summary}"
    return summary


def run_fwd(fa, q, k, v, dtype, causal=False, scale=None, stream=None):
    """Upload (float64 [B,H,N,d]) inputs, run fa_fwd, return (O, LSE) as float64 host arrays."""
    tq, tk, tv = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    o, lse = fa.fa_fwd(tq, tk, tv, scale=scale, causal=causal, stream=stream)
    import torch

    torch.cuda.synchronize()
    return to_host(o), lse.cpu().numpy().astype(np.float64)


def scale_of(d):
    return 1.0 / math.sqrt(d)
