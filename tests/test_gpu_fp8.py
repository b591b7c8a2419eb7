"""GPU parity of the block-scaled fp8 mode (quantiser and forward) against the fp8 oracle.

The quantiser is integer work: its codes and scales must equal the oracle's bit for bit.

The forward is attention of the dequantised tensors (the oracle's ``attention_fp8``) up to
the kernel's own rounding of P to E4M3.  With P = 2^(s c - m + 1) formed in fp32, P' = P
times the V block factor 2^(e_v - e_vmax) <= 1 rounded to E4M3 (relative error <= 2^-4 in
the normal range, absolute <= 2^-10 in the subnormal one), O = 2^(e_vmax) sum P'~ v~ / l with
l = sum P in fp32, and l >= 2 Z where Z = sum_j e^(S_j - max S) (the running maximum m never
exceeds the row maximum), first-order error analysis gives, elementwise,

    |O - O_ref| <= 2^-4 (W |V^|) + 2^-11 2^(e_vmax) / Z * sum_j |v~_j|
                   + 2 dS (W |V^|) + 1e-5 (W |V^|) + 1e-6

(W the oracle's softmax weights, V^ the dequantised V, v~ its codes' values; the last two
terms cover fp32 accumulation and the exp2 approximation), plus half an output ulp.

dS bounds the error of the scores themselves.  The fp8 MFMA does not sum its 64 products
in full fp32: over 262144 dot products of four input families (uniform codes,
block-quantised normal data, heavy cancellation, one large value among small ones) the
error of one 32x32x64 step reached 2^-10.8 of its largest |product| (and was unbiased).
The tests take eps = 2^-9 per step, so with Q^_i and K^_j the dequantised rows,

    dS_i = eps * (d / 64) * scale * max_k |Q^_ik| * max_jk |K^_jk|,

and a score error moves LSE by at most its own size and O by at most 2 dS (W |V^|).  LSE
is formed from the unrounded fp32 sum, so |LSE - LSE_ref| <= dS_i + 1e-5 + 2^-20 |LSE|.
The edge workload's all-zero-Q and one-hot heads give P exactly representable, and there O
must match closed forms to fp32 accuracy.
"""

import numpy as np
import pytest

import workloads as wl
from gpu_util import half_ulp, scale_of, to_device, to_host
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu

MFMA_EPS = 2.0 ** -9      # error of one fp8 32x32x64 MFMA step / its largest |product|


def _quantize_gpu(fa, x, dtype, transpose):
    import torch

    codes, scales = fa.fa_quantize_fp8(to_device(x, dtype), transpose=transpose)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy().astype(np.float64)


def _outlier_input(B, H, N, d, dtype, seed):
    x = wl.random_tensor((B, H, N, d), dtype, [seed, 1])
    x[0, 0, : min(N, 3)] *= 64.0                      # an outlier block
    if N > 64:
        x[0, -1, 64: min(N, 128)] = 0.0                # an all-zero block
    return wl.round_to_dtype(x, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 200, 1000])
def test_quantize_matches_oracle(gpu_lib, dtype, d, N):
    x = _outlier_input(2, 3, N, d, dtype, seed=N + d)
    codes_ref, scales_ref = ofp8.quantize_blocks(x)
    c, s = _quantize_gpu(gpu_lib, x, dtype, transpose=False)
    np.testing.assert_array_equal(s, scales_ref)
    np.testing.assert_array_equal(c, codes_ref)
    ct, st = _quantize_gpu(gpu_lib, x, dtype, transpose=True)
    Np = gpu_lib.fa_fp8_padded_len(N)
    assert ct.shape == (2, 3, d, Np)
    np.testing.assert_array_equal(st, scales_ref)
    np.testing.assert_array_equal(ct[..., :N], np.swapaxes(codes_ref, -1, -2))
    assert (ct[..., N:] == 0).all()


# ------------------------------------------------------------------ forward ---

def _fp8_bound(Qd, Kd, Vd, vcodes, vscales, scale, rows, causal=False):
    """The elementwise O error bound and the per-row LSE bound of the module docstring,
    for query rows ``rows`` (W and Z of the masked scores when ``causal``)."""
    S = scale * (Qd[rows] @ Kd.T)
    if causal:
        S = np.where(np.arange(Kd.shape[0])[None, :] <= np.asarray(rows)[:, None], S, -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    Z = E.sum(axis=1, keepdims=True)
    W = E / Z
    wv = W @ np.abs(Vd)
    vabs = np.abs(ofp8.e4m3_decode(vcodes)).sum(axis=0, keepdims=True)
    dS = MFMA_EPS * (Qd.shape[1] / 64) * scale * np.abs(Qd[rows]).max(axis=1, keepdims=True) * np.abs(Kd).max()
    o_bound = 2.0 ** -4 * wv + 2.0 ** -11 * vscales.max() / Z * vabs + 2 * dS * wv + 1e-5 * wv + 1e-6
    return o_bound, dS[:, 0]


def _run_fp8(fa, q, k, v, in_dtype, out_dtype, scale=None, causal=False):
    import torch

    tq, tk, tv = (to_device(x, in_dtype) for x in (q, k, v))
    q8, qs = fa.fa_quantize_fp8(tq)
    k8, ks = fa.fa_quantize_fp8(tk)
    vt8, vs = fa.fa_quantize_fp8(tv, transpose=True)
    o, lse = fa.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, scale=scale, causal=causal,
                           out_dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float16)
    torch.cuda.synchronize()
    return to_host(o), lse.cpu().numpy().astype(np.float64)


def _check_head(O, L, q, k, v, scale, out_dtype, rows, what, causal=False):
    """Oracle for one head (on the requested rows) and the bound check."""
    qc, qs = ofp8.quantize_blocks(q)
    kc, ks = ofp8.quantize_blocks(k)
    vc, vs = ofp8.quantize_blocks(v)
    O_ref, L_ref = ofp8.attention_fp8_rows(qc, qs, kc, ks, vc, vs, scale, rows, causal=causal)
    Qd, Kd, Vd = (ofp8.dequantize_blocks(c, s) for c, s in ((qc, qs), (kc, ks), (vc, vs)))
    o_bound, dS = _fp8_bound(Qd, Kd, Vd, vc, vs, scale, rows, causal)
    bound = o_bound + half_ulp(O_ref, out_dtype)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    if (err > bound).any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: O error {err[i]:.3e} > bound {bound[i]:.3e} at {i}")
    lerr = np.abs(L - L_ref)
    lbound = dS + 1e-5 + 2.0 ** -20 * np.abs(L_ref)
    assert (lerr <= lbound).all(), f"{what}: LSE error {lerr.max():.3e} (bound {lbound[np.argmax(lerr)]:.3e})"
    return float(err.max()), float((err / bound).max()), float(lerr.max())


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 63, 65, 129, 300, 1000])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp16"])
def test_fp8_forward_parity(gpu_lib, in_dtype, out_dtype, d, N):
    B, H = 1, 3
    q, k, v = (wl.random_tensor((B, H, N, d), in_dtype, [N, d, t]) for t in (1, 2, 3))
    v[0, 1, : min(N, 40)] *= 16.0          # V blocks of different scales within one head
    v = wl.round_to_dtype(v, in_dtype)
    O, L = _run_fp8(gpu_lib, q, k, v, in_dtype, out_dtype)
    worst = 0.0
    for h in range(H):
        e, frac, le = _check_head(O[0, h], L[0, h], q[0, h], k[0, h], v[0, h], scale_of(d), out_dtype,
                                  np.arange(N), f"N={N} d={d} h={h}")
        worst = max(worst, frac)
    print(f"N={N} d={d} {out_dtype}: worst error / bound = {worst:.3f}")


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 65, 127, 128, 129, 300, 1000])
def test_fp8_causal_parity(gpu_lib, out_dtype, d, N):
    """fa_fwd_fp8_causal against causal attention of the dequantised tensors: query blocks
    of 128 rows and key tiles of 64 put the diagonal inside, at and across tile edges."""
    B, H = 2, 2
    in_dtype = "bf16"
    q, k, v = (wl.random_tensor((B, H, N, d), in_dtype, [N, d, t, 7]) for t in (1, 2, 3))
    v[1, 0, : min(N, 40)] *= 16.0
    v = wl.round_to_dtype(v, in_dtype)
    O, L = _run_fp8(gpu_lib, q, k, v, in_dtype, out_dtype, causal=True)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            e, frac, le = _check_head(O[b, h], L[b, h], q[b, h], k[b, h], v[b, h], scale_of(d), out_dtype,
                                      np.arange(N), f"causal N={N} d={d} b={b} h={h}", causal=True)
            worst = max(worst, frac)
    # row 0 attends to key 0 alone: P = 2^1 is exact in E4M3, so O_0 is V^_0 rounded once
    vc, vs = ofp8.quantize_blocks(v[0, 0])
    v0 = ofp8.dequantize_blocks(vc, vs)[0]
    assert (np.abs(O[0, 0, 0] - v0) <= 1e-6 * np.abs(v0) + half_ulp(v0, out_dtype)).all()
    print(f"causal N={N} d={d} {out_dtype}: worst error / bound = {worst:.3f}")


def test_fp8_edge_workload_closed_forms(gpu_lib):
    """B2 H8 N4097 d128: zero-Q heads give O = mean of V^ and LSE = ln N exactly in P; one-hot
    heads give O = V^ of the boosted key; the x10 heads are held to the bound."""
    w = wl.WORKLOADS[4]
    q, k, v = wl.make_inputs(w)
    O, L = _run_fp8(gpu_lib, q, k, v, w.dtype, "bf16")
    rows = wl.sampled_rows(w, 0, 0)
    for b in range(w.B):
        for h in range(w.H):
            vc, vs = ofp8.quantize_blocks(v[b, h])
            Vd = ofp8.dequantize_blocks(vc, vs)
            cat = wl.edge_category(b, h, w.H)
            if cat == 0:
                ref = np.broadcast_to(Vd.mean(0), Vd.shape)
                np.testing.assert_allclose(O[b, h], ref, rtol=0, atol=1e-5 + half_ulp(ref, "bf16").max())
                np.testing.assert_allclose(L[b, h], np.log(w.N), atol=1e-5)
            elif cat == 2:
                ref = Vd[wl.boost_targets(w, b, h)]
                assert (np.abs(O[b, h] - ref) <= 1e-6 + half_ulp(ref, "bf16")).all()
            else:
                _check_head(O[b, h][rows], L[b, h][rows], q[b, h], k[b, h], v[b, h], w.scale, "bf16", rows,
                            f"edge b={b} h={h}")


@pytest.mark.parametrize("B,H,N", [(4, 16, 2049), (4, 32, 16384)])
def test_fp8_large_sampled(gpu_lib, B, H, N):
    """Large grids, launched as the benchmark launches them, on sampled rows of three heads."""
    import torch

    d = 128
    gen = torch.Generator(device="cuda").manual_seed(N)
    q, k, v = (torch.randn(B, H, N, d, device="cuda", dtype=torch.bfloat16, generator=gen) for _ in range(3))
    q8, qs = gpu_lib.fa_quantize_fp8(q)
    k8, ks = gpu_lib.fa_quantize_fp8(k)
    vt8, vs = gpu_lib.fa_quantize_fp8(v, transpose=True)
    o, lse = gpu_lib.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    rows = np.array(sorted({0, 63, 64, 255, 256, N - 1} | set(rng.choice(N, 26, replace=False).tolist())))
    for (b, h) in ((0, 0), (B // 2, H - 1), (B - 1, H // 2)):
        qh, kh, vh = (to_host(t[b, h]) for t in (q, k, v))
        e, frac, le = _check_head(to_host(o[b, h])[rows], lse[b, h].cpu().numpy().astype(np.float64)[rows],
                                  qh, kh, vh, scale_of(d), "bf16", rows, f"B={B} H={H} N={N} b={b} h={h}")
        print(f"N={N} b={b} h={h}: max err {e:.2e}, worst error / bound {frac:.3f}, LSE err {le:.1e}")


def test_fp8_causal_large_sampled(gpu_lib):
    """The causal kernel on the long-sequence grid, sampled rows near the start, at block
    and tile edges and at the end."""
    import torch

    B, H, N, d = 2, 16, 16384, 128
    gen = torch.Generator(device="cuda").manual_seed(77)
    q, k, v = (torch.randn(B, H, N, d, device="cuda", dtype=torch.bfloat16, generator=gen) for _ in range(3))
    q8, qs = gpu_lib.fa_quantize_fp8(q)
    k8, ks = gpu_lib.fa_quantize_fp8(k)
    vt8, vs = gpu_lib.fa_quantize_fp8(v, transpose=True)
    o, lse = gpu_lib.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, 8191, N - 1} | set(rng.choice(N, 24, replace=False).tolist())))
    for (b, h) in ((0, 0), (B - 1, H - 1)):
        qh, kh, vh = (to_host(t[b, h]) for t in (q, k, v))
        e, frac, le = _check_head(to_host(o[b, h])[rows], lse[b, h].cpu().numpy().astype(np.float64)[rows],
                                  qh, kh, vh, scale_of(d), "bf16", rows, f"causal N={N} b={b} h={h}", causal=True)
        print(f"causal N={N} b={b} h={h}: max err {e:.2e}, worst error / bound {frac:.3f}, LSE err {le:.1e}")


def test_fp8_deterministic_and_empty(gpu_lib):
    import torch

    q, k, v = (torch.randn(1, 2, 700, 64, device="cuda", dtype=torch.float16) for _ in range(3))
    outs = []
    for _ in range(2):
        q8, qs = gpu_lib.fa_quantize_fp8(q)
        k8, ks = gpu_lib.fa_quantize_fp8(k)
        vt8, vs = gpu_lib.fa_quantize_fp8(v, transpose=True)
        outs.append(gpu_lib.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, out_dtype=torch.float16))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    e = torch.empty(2, 3, 0, 128, device="cuda", dtype=torch.bfloat16)
    e8, es = gpu_lib.fa_quantize_fp8(e)
    et8, ets = gpu_lib.fa_quantize_fp8(e, transpose=True)
    o, lse = gpu_lib.fa_fwd_fp8(e8, e8, et8, es, es, ets)
    assert o.shape == (2, 3, 0, 128) and lse.shape == (2, 3, 0)
