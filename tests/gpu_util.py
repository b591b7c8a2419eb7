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


# Gradients.  The backward rebuilds P in fp32, rounds P and dS = P * (dP - D) to the
# input type before the second products, and forms D from O as stored (rounded, and
# carrying the forward's own error, whose size is that of rounding P).  With u the unit
# roundoff of the input type (2^-8 bf16, 2^-11 fp16), first-order error analysis gives,
# elementwise,
#     |d dV| <= u (P^T |dO|),
#     |d dK| <= u scale (|dS|^T |Q| + (P * E)^T |Q|),
#     |d dQ| <= u scale (|dS| |K| + E * (P |K|)),
# with E_i = 2 sum_k |dO_ik| (P |V|)_ik bounding the error of D_i.  Values that round into
# the subnormal range carry an absolute error of up to eta (half the smallest subnormal
# spacing: 2^-25 fp16, 2^-134 bf16) instead, adding eta times the other operand's absolute
# column sums.  The test allows twice these (fp32 accumulation and exp2 rounding are
# second order) plus half an output ulp, and separately bounds the normwise relative
# error.
UNIT_ROUNDOFF = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
SUBNORMAL_HALF_STEP = {"fp16": 2.0 ** -25, "bf16": 2.0 ** -134}
GRAD_REL_FRO = {"fp16": 2e-3, "bf16": 1e-2}


def _d_error_weight(V, dO, P):
    """E_i = 2 sum_k |dO_ik| (P |V|)_ik: bound on the error of D_i (O rounded and carrying
    the forward's error)."""
    return 2.0 * (np.abs(dO) * (P @ np.abs(V))).sum(axis=-1)


def mass_dq(K, V, dO, scale, P, dS, dtype):
    """Error mass of dQ for query rows r: P, dS [r, N]; dO [r, d]; K, V all keys."""
    E = _d_error_weight(V, dO, P)
    aK = np.abs(K)
    floor = SUBNORMAL_HALF_STEP[dtype] / UNIT_ROUNDOFF[dtype] * aK.sum(axis=0)
    return scale * (np.abs(dS) @ aK + E[:, None] * (P @ aK) + floor[None, :])


def mass_dkdv(Q, V, dO, scale, P, dS, dtype, cols=None):
    """Error masses of dK, dV for key columns ``cols`` (all if None), summed over the query
    rows r given: P, dS [r, N]; Q, dO [r, d].  Row blocks add up."""
    E = _d_error_weight(V, dO, P)
    if cols is not None:
        P, dS = P[:, cols], dS[:, cols]
    aQ, adO = np.abs(Q), np.abs(dO)
    f = SUBNORMAL_HALF_STEP[dtype] / UNIT_ROUNDOFF[dtype]
    m_dk = scale * (np.abs(dS).T @ aQ + (P * E[:, None]).T @ aQ + f * aQ.sum(axis=0)[None, :])
    m_dv = P.T @ adO + f * adO.sum(axis=0)[None, :]
    return m_dk, m_dv


def compare_grad(G, G_ref, dtype: str, what: str = "", mass=None, check_fro: bool = True):
    """Pass iff |G - G_ref| <= 2 u mass + half an output ulp elementwise, the relative
    Frobenius error is within GRAD_REL_FRO (unless ``check_fro`` is off: there the
    gradient is a small difference of large terms and only the elementwise bound, which
    accounts for that, is asserted), and nothing is NaN/Inf."""
    assert np.all(np.isfinite(G)), f"{what}: non-finite gradient"
    err = np.abs(G - G_ref)
    bound = 2.0 * UNIT_ROUNDOFF[dtype] * mass + half_ulp(G_ref, dtype)
    bad = err > bound
    den = np.linalg.norm(G_ref)
    rel = float(np.linalg.norm(G - G_ref) / den) if den > 0 else float(np.linalg.norm(G))
    ratio = err / bound
    # the O rule (tolerance + half an output ulp), reported beside the derived bound
    o_rule = O_TOL[dtype] + half_ulp(G_ref, dtype)
    summary = dict(max_err=float(err.max()) if err.size else 0.0, rel_fro=rel,
                   max_err_over_bound=float(ratio.max()) if ratio.size else 0.0,
                   max_ref=float(np.abs(G_ref).max()) if G_ref.size else 0.0,
                   max_err_over_o_rule=float((err / o_rule).max()) if err.size else 0.0,
                   n_above_o_rule=int((err > o_rule).sum()))
    if bad.any():
        idx = np.unravel_index(np.argmax(ratio), err.shape)
        raise AssertionError(f"{what}: error {err[idx]:.3e} > bound {bound[idx]:.3e} at {idx} "
                             f"(got {G[idx]}, ref {G_ref[idx]}); {int(bad.sum())} elements out; {summary}")
    if check_fro:
        assert rel <= GRAD_REL_FRO[dtype], f"{what}: relative Frobenius error {rel:.3e}; {summary}"
    return summary
