"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-backward] [--copy-calibration BYTES] [--sweep]

Workload: B=4, H=32, N=16384, d=128, bf16 Q/K/V, scale 1/sqrt(d), non-causal, one
forward per step through the C ABI (fa_fwd) with inputs resident in HBM.  Prints
ONE JSON line on stdout (everything else goes to stderr):

  value      forward TFLOP/s = 4*B*H*N^2*d / (time per step)
  roofline   the kernel against the dense bf16 MFMA peak; `achieved` is the same
             algorithmic FLOPs over the kernel's average duration measured with HIP
             events on the launch stream; `traffic` is HBM bytes per launch from the
             committed rocprofv3 counter summary when it was taken on the current
             kernel source, else null
  backward   the recompute-based backward (fa_bwd) on the same tensors with seeded dO,
             timed separately after the forward; TFLOP/s counted as 10*B*H*N^2*d
             (2.5x the forward: S, dP, dV, dK, dQ), not part of `value`
  fp8        the opt-in block-scaled fp8 forward (fa_fwd_fp8) on the same inputs quantised
             once by fa_quantize_fp8 (codes resident in HBM, like a cached K/V); TFLOP/s
             counted as 4*B*H*N^2*d against the dense fp8 MFMA peak; the quantiser's time is
             reported beside it, not inside it
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload (whole heads
             in row chunks, all keys, about 15 s of host time), timed on the host
             cores, with the GPU output checked on the same rows
  mfma_busy  the forward's MFMA-busy fraction (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES per SIMD cycle)
             and clock from the committed counter summary, when it was taken on the current
             kernel source, else null
  power      socket power and GFX clock (amd-smi) sampled while the forward runs back to back
             for --power-seconds after the timed steps, with the board's power cap; the
             kernel is power-bound on this workload, so these numbers bound its rate
  configs    forward time of the four other workloads at their real sizes: fp32 B1 H1 N256
             d64 (latency-bound), bf16 B4 H16 N2048 d64, fp16 B1 H32 N16384 d128 and the edge
             workload bf16 B2 H8 N4097 d128 (zero, x10 and one-hot heads), each after 0.2 s
             of warm-up launches: the mean of 50 launches queued back to back (TFLOP/s and
             % of the MFMA peak of the input type are taken from it), and the median and min
             of per-launch events, whose intervals also hold each event's own gap
  causal     the causal forward (fa_fwd_causal) on the same tensors, TFLOP/s counted on the
             computed half (2*B*H*N^2*d)
  hbm_small_n  short sequences at B*H = 1024, d = 128, bf16, N in {128, 256, 512}, where the
             forward is bounded by HBM: algorithmic bytes (Q, K, V read once, O and LSE
             written once) per launch (back-to-back mean, as for configs), as GB/s and % of
             the 8 TB/s HBM peak
  sweep      (--sweep only) forward time of the smaller workloads (fp32 B1 H1 N256 d64,
             bf16 B4 H16 N2048 d64, fp16 B1 H32 N16384 d128, bf16 B2 H8 N4097 d128), the
             causal and split-KV variants, the fp8 forward causal at d=128 and at d=64,
             short sequences at B*H=1024 d=128 where the kernel is bounded by HBM
             bandwidth, and a decode shape; min and median of per-launch events
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) and % of MI355X bf16 MFMA peak, d=128"
PEAK_BF16_TFLOPS = 2516.6          # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2           # MI355X dense fp8 MFMA: 256 CU x 8192 FLOP/clk x 2.4 GHz
PEAK_FP32_TFLOPS = 157.3           # MI355X fp32 (vector and matrix)
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E
B, H, N, D = 4, 32, 16384, 128
KERNEL_SOURCES = ("online_softmax_attention_fa_amd/csrc/fa_fwd_kernel.hip",
                  "online_softmax_attention_fa_amd/csrc/fa_device.h",
                  "online_softmax_attention_fa_amd/csrc/fa_internal.h")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fa_fwd_bf16_B4_H32_N16384_d128_counters.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the forward kernel's sources with comments and blank space removed, so that
    an edit to a comment does not invalidate the recorded counters."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    if not os.path.exists(PMC_SUMMARY):
        return None, "no counter summary"
    text = open(PMC_SUMMARY).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes):
        return None, "summary lacks hash or bytes"
    if m_hash.group(1) != kernel_source_hash():
        return None, "kernel changed since counters were taken"
    return float(m_bytes.group(1)), "ok"


def mfma_busy_from_profile():
    """The forward's MFMA-busy fraction and clock from the committed counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE / 8), if it matches this
    source: the share of the matrix cores' cycles the kernel keeps them working, the peak
    fraction at the clock the chip actually ran."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_busy = re.search(r"\| MFMA busy per SIMD \| ([0-9.]+) %", text)
    m_clk = re.search(r"MFMA peak at ([0-9.]+) GHz", text)
    if not (m_hash and m_busy and m_clk) or m_hash.group(1) != kernel_source_hash():
        return None
    return {"frac": round(float(m_busy.group(1)) / 100, 4), "clock_ghz": float(m_clk.group(1)),
            "source": "profiles/fa_fwd_bf16_B4_H32_N16384_d128_counters.md: SQ_VALU_MFMA_BUSY_CYCLES / "
                      "(1024 SIMDs x GRBM_GUI_ACTIVE / 8), rocprofv3 counter run of this kernel source"}


def cpu_baseline(q, k, v, o, lse, scale, budget_s=15.0, chunk=2048):
    """The oracle (fp64 numpy, as it stands) on a bounded sample of the workload: whole heads,
    taken in a fixed order and evaluated in row chunks of ``chunk`` query rows against all
    keys, until about ``budget_s`` seconds of oracle time are spent.  The GPU output on the
    covered rows is checked against it."""
    import numpy as np

    from oracle import attention_rows

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    order = np.random.default_rng(1234).permutation(B * H)
    spent, rows_done, heads_done = 0.0, 0, []
    err_o = err_l = 0.0
    for bh in order:
        b, h = divmod(int(bh), H)
        qh = q[b, h].float().cpu().numpy().astype(np.float64)
        kh = k[b, h].float().cpu().numpy().astype(np.float64)
        vh = v[b, h].float().cpu().numpy().astype(np.float64)
        og = o[b, h].float().cpu().numpy().astype(np.float64)
        lg = lse[b, h].cpu().numpy().astype(np.float64)
        heads_done.append((b, h))
        for r0 in range(0, N, chunk):
            rows = np.arange(r0, min(N, r0 + chunk))
            t0 = time.perf_counter()
            O_ref, L_ref = attention_rows(qh, kh, vh, scale, rows)
            spent += time.perf_counter() - t0
            rows_done += len(rows)
            err_o = max(err_o, float(np.abs(og[rows] - O_ref).max()))
            err_l = max(err_l, float(np.abs(lg[rows] - L_ref).max()))
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    flops = 4.0 * rows_done * N * D
    full_s = 4.0 * B * H * N * N * D / (flops / spent)
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows_done} query rows ({len(heads_done)} heads, whole heads first) of the "
                  f"workload against all {N} keys: 4*rows*N*d = {flops:.3e} FLOP of fp64 numpy "
                  f"three-pass attention in {spent:.1f} s",
        "seconds": round(spent, 2),
        "extrapolated_full_workload_s": round(full_s, 1),
        "gpu_rows_max_err_o": err_o,
        "gpu_rows_max_err_lse": err_l,
    }


def backward_sample_check(q, k, v, do, dq, dk, dv, scale, heads=1, nrows=64, ncols=32):
    """The oracle's gradients on sampled rows (dQ) and columns (dK, dV) of ``heads`` seeded
    heads of the workload, against the GPU's: bare max-abs error per gradient, and the count
    of elements above 1e-2 + half a bf16 ulp of the reference (the rule that holds O's
    tolerance up to the rounding of the stored output)."""
    import numpy as np

    from oracle import backward_cols_dkdv, backward_rows_dq

    rng = np.random.default_rng(20240603)
    out = {"heads": [], "rows_per_head": nrows, "cols_per_head": ncols}
    worst = {"dq": [0.0, 0, 0.0], "dk": [0.0, 0, 0.0], "dv": [0.0, 0, 0.0]}   # max err, count over, max |ref|
    t0 = time.perf_counter()

    def half_ulp_bf16(x):
        ax = np.abs(x)
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
        return 0.5 * np.exp2(np.maximum(e, -126) - 7)

    def upd(key, got, ref):
        err = np.abs(got - ref)
        w = worst[key]
        w[0] = max(w[0], float(err.max()))
        w[1] += int((err > 1e-2 + half_ulp_bf16(ref)).sum())
        w[2] = max(w[2], float(np.abs(ref).max()))

    for bh in rng.choice(B * H, size=heads, replace=False):
        b, hh = divmod(int(bh), H)
        f64 = lambda t: t[b, hh].float().cpu().numpy().astype(np.float64)
        Q, K, V, dO = f64(q), f64(k), f64(v), f64(do)
        rows = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.choice(N, nrows - 4, replace=False)]))
        cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, ncols - 2, replace=False)]))
        upd("dq", f64(dq)[rows], backward_rows_dq(Q, K, V, dO, scale, rows))
        dk_ref, dv_ref = backward_cols_dkdv(Q, K, V, dO, scale, cols)
        upd("dk", f64(dk)[cols], dk_ref)
        upd("dv", f64(dv)[cols], dv_ref)
        out["heads"].append([b, hh])
    for key, (e, n, r) in worst.items():
        out[key] = {"max_abs_err": e, "n_above_1e-2_plus_half_ulp": n, "max_abs_ref": r}
    out["seconds"] = round(time.perf_counter() - t0, 2)
    log(f"backward sample check: {out}")
    return out


def time_backward(fa, q, k, v, o, lse, scale, stream, steps):
    """fa_bwd on the forward's O and LSE with seeded dO; events on the launch stream."""
    import torch

    gen = torch.Generator(device=q.device).manual_seed(20240602)
    do = torch.randn(q.shape, device=q.device, dtype=q.dtype, generator=gen)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, D, q.dtype), dtype=torch.uint8, device=q.device)
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale=scale, stream=stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale=scale, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = 10.0 * B * H * N * N * D
    tflops = flops / (ms * 1e-3) / 1e12
    ok = all(torch.isfinite(t).all().item() for t in (dq, dk, dv))
    log(f"backward {ms:.3f} ms/step, {tflops:.1f} TFLOP/s (10*B*H*N^2*d), finite={ok}")
    return {"ms_per_step": round(ms, 4), "tflops": round(tflops, 2), "steps": steps,
            "flops_per_step": flops, "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
            "outputs_finite": ok}, (do, dq, dk, dv)


def time_fp8(fa, q, k, v, o_ref, scale, stream, steps):
    """fa_quantize_fp8 of Q, K, V once, then fa_fwd_fp8 timed with events on the stream."""
    import torch

    def quantize():
        return (fa.fa_quantize_fp8(q, stream=stream), fa.fa_quantize_fp8(k, stream=stream),
                fa.fa_quantize_fp8(v, transpose=True, stream=stream))

    (q8, qs), (k8, ks), (vt8, vs) = quantize()
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=q.device, dtype=torch.float32)
    fwd = lambda: fa.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, o, lse, scale=scale, stream=stream)
    fwd()
    torch.cuda.synchronize()
    t_q = launch_times(quantize, stream, 3, warmup=1)
    t = launch_times(fwd, stream, steps, warmup=2)
    ms = sum(t) / len(t)
    flops = 4.0 * B * H * N * N * D
    tflops = flops / (ms * 1e-3) / 1e12
    diff = (o.float() - o_ref.float()).abs().max().item()
    ok = bool(torch.isfinite(o).all().item() and torch.isfinite(lse).all().item())
    log(f"fp8 forward {ms:.3f} ms/launch, {tflops:.1f} TFLOP/s = {100 * tflops / PEAK_FP8_TFLOPS:.1f}% of the fp8 "
        f"peak; quantise Q, K, V {sum(t_q) / len(t_q):.3f} ms; max |O_fp8 - O_bf16| = {diff:.3e}")
    return {"ms_per_launch": round(ms, 4), "min_ms": round(min(t), 4), "tflops": round(tflops, 2),
            "peak": PEAK_FP8_TFLOPS, "frac_of_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
            "quantize_qkv_ms": round(sum(t_q) / len(t_q), 4), "max_abs_diff_vs_bf16_o": diff,
            "outputs_finite": ok, "steps": steps}


def _smi(cmd):
    import subprocess

    try:
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=20)
        return r.stdout
    except (OSError, subprocess.SubprocessError):
        return ""


def parse_smi_metric(txt):
    """(socket watts, mean GFX MHz over the XCDs) from `amd-smi metric -p -c` text, or None."""
    w = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
    clk = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", txt)]
    if not w or not clk:
        return None
    return float(w[0]), sum(clk) / len(clk)


def power_while_running(fn, seconds, settle=1.0, period=0.25):
    """Socket power (W) and per-XCD GFX clocks (MHz) from `amd-smi metric -p -c`, sampled in a
    child process while `fn` (one forward launch) runs back to back for `seconds`.  Samples in
    the first `settle` seconds are dropped (clocks and power ramp up).  None if amd-smi is absent."""
    import threading

    import torch

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            t = time.perf_counter()
            got = parse_smi_metric(_smi(["amd-smi", "metric", "-g", "0", "-p", "-c"]))
            if got is not None:
                samples.append((t, *got))
            stop.wait(period)

    cap_txt = _smi(["rocm-smi", "--showmaxpower"])
    cap = re.findall(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", cap_txt)
    fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stop.set()
    th.join()
    kept = [s for s in samples if s[0] - t0 >= settle]
    if not kept:
        return None
    watts = [s[1] for s in kept]
    mhz = [s[2] for s in kept]
    return {"socket_w_mean": round(sum(watts) / len(watts), 1), "socket_w_max": round(max(watts), 1),
            "power_cap_w": float(cap[0]) if cap else None,
            "gfx_mhz_mean": round(sum(mhz) / len(mhz), 1), "samples": len(kept),
            "seconds": round(wall, 2), "launches": n, "ms_per_launch": round(wall * 1e3 / n, 4),
            "source": "amd-smi metric -p -c (socket power, mean GFX clock of the 8 XCDs); rocm-smi --showmaxpower"}


def launch_times(fn, stream, steps, warmup=5, warm_seconds=0.2):
    """Per-launch durations (ms) from events recorded between back-to-back launches, after at
    least `warmup` launches and `warm_seconds` of back-to-back launches.  A short kernel timed
    straight after an idle spell runs before the clocks have settled under load: 10-12%
    slower at B4 H16 N2048 d64 (85.7 against 77.1 us) and at the edge workload."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def back_to_back_ms(fn, stream, n):
    """Mean time (ms) of n launches queued back to back between two events, nothing between
    them: the rate of a stream of calls, without the per-launch event records."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _timed_case(fa, stream, q, k, v, scale, steps):
    """(min, median) per-launch ms, back-to-back mean ms over 50 launches, outputs finite."""
    import statistics

    import torch

    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=q.device, dtype=torch.float32)
    fn = lambda: fa.fa_fwd(q, k, v, o, lse, scale=scale, stream=stream)
    t = launch_times(fn, stream, steps)
    mean = back_to_back_ms(fn, stream, 50)
    ok = bool(torch.isfinite(o).all().item() and torch.isfinite(lse).all().item())
    return min(t), statistics.median(t), mean, ok


def _upload(x, dtype, dev):
    """Exactly representable float64 values -> device tensor of the storage dtype."""
    import torch

    import workloads as wl

    arr = wl.storage_array(x, dtype)
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(arr).to(dev)


def configs_leg(fa, stream, steps=20):
    """The forward at the other workloads' real sizes.  fp32 B1 H1 N256 d64 and the edge
    workload bf16 B2 H8 N4097 d128 take the seeded inputs of the workloads module (the edge
    one with its zero, x10 and one-hot heads); the two larger iid ones draw N(0,1) on the
    device (torch Philox), the same distribution without 200M host draws."""
    import torch

    import workloads as wl

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(20240604)
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
    rows = []
    for cid in (1, 2, 3, 4):
        w = wl.WORKLOADS[cid]
        dt = tdt[w.dtype]
        if cid in (1, 4):
            q, k, v = (_upload(x, w.dtype, dev) for x in wl.make_inputs(w, threads=8))
            source = "workloads module (seeded numpy)"
        else:
            q, k, v = (torch.randn(w.B, w.H, w.N, w.d, device=dev, dtype=dt, generator=gen) for _ in range(3))
            source = "device N(0,1), torch Philox"
        tmin, tmed, tmean, ok = _timed_case(fa, stream, q, k, v, w.scale, steps)
        peak = PEAK_FP32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS
        tf = w.flops / (tmean * 1e-3) / 1e12
        nbytes = 4.0 * w.B * w.H * w.N * w.d * q.element_size() + 4.0 * w.B * w.H * w.N
        r = {"workload": f"{w.dtype} B{w.B} H{w.H} N{w.N} d{w.d}" + (" edge heads" if w.kind == "edge" else ""),
             "mean_us": round(1e3 * tmean, 2), "median_us": round(1e3 * tmed, 2), "min_us": round(1e3 * tmin, 2),
             "tflops": round(tf, 2), "pct_of_mfma_peak": round(100 * tf / peak, 2), "peak_tflops": peak,
             "gbps_algorithmic": round(nbytes / (tmean * 1e-3) / 1e9, 1),
             "plan": fa.fa_fwd_plan(w.B, w.H, w.N, w.d, dt), "outputs_finite": ok, "inputs": source}
        if cid == 1:
            r["note"] = "latency-bound (8 workgroups): microseconds and GB/s, no roofline claim"
        rows.append(r)
        log(f"config {r['workload']}: mean {r['mean_us']} us (per-launch median {r['median_us']}), {r['tflops']} TFLOP/s = "
            f"{r['pct_of_mfma_peak']}% of peak, finite={ok}")
        del q, k, v
    return rows


def hbm_small_n_leg(fa, stream, steps=20):
    """Short sequences at B*H = 1024, d = 128, bf16: algorithmic bytes over launch time."""
    import torch

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(20240605)
    b, h, d = 16, 64, 128
    rows = []
    for n in (128, 256, 512):
        q, k, v = (torch.randn(b, h, n, d, device=dev, dtype=torch.bfloat16, generator=gen) for _ in range(3))
        tmin, tmed, tmean, ok = _timed_case(fa, stream, q, k, v, 1.0 / math.sqrt(d), steps)
        nbytes = 4.0 * b * h * n * d * 2 + 4.0 * b * h * n
        gbps = nbytes / (tmean * 1e-3) / 1e9
        rows.append({"workload": f"bf16 B{b} H{h} N{n} d{d}", "mean_us": round(1e3 * tmean, 2),
                     "median_us": round(1e3 * tmed, 2), "min_us": round(1e3 * tmin, 2),
                     "algorithmic_bytes": nbytes, "gbps": round(gbps, 1),
                     "pct_of_hbm_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                     "flop_per_byte": round(4.0 * b * h * n * n * d / nbytes, 1),
                     "plan": fa.fa_fwd_plan(b, h, n, d, torch.bfloat16), "outputs_finite": ok})
        log(f"hbm small N={n}: mean {rows[-1]['mean_us']} us (per-launch median {rows[-1]['median_us']}), {rows[-1]['gbps']} GB/s = "
            f"{rows[-1]['pct_of_hbm_peak']}% of 8 TB/s")
        del q, k, v
    return rows


def causal_leg(fa, q, k, v, scale, stream, steps=10):
    """The causal forward (fa_fwd_causal) on the same tensors; TFLOP/s counted on the half of
    the score matrix that is computed, 2*B*H*N^2*d."""
    import statistics

    import torch

    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=q.device, dtype=torch.float32)
    t = launch_times(lambda: fa.fa_fwd_causal(q, k, v, o, lse, scale=scale, stream=stream), stream, steps, warmup=2)
    tmed = statistics.median(t)
    flops = 2.0 * B * H * N * N * D
    tf = flops / (tmed * 1e-3) / 1e12
    ok = bool(torch.isfinite(o).all().item() and torch.isfinite(lse).all().item())
    log(f"causal forward: median {tmed:.3f} ms, {tf:.1f} TFLOP/s on the computed half, finite={ok}")
    return {"median_ms": round(tmed, 4), "min_ms": round(min(t), 4), "tflops": round(tf, 2),
            "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "flops": flops,
            "plan": fa.fa_fwd_plan(B, H, N, D, q.dtype, causal=True), "outputs_finite": ok}


def sweep(fa, stream, steps=20):
    """Forward timings of the smaller workloads, the bandwidth-bound short sequences, a decode
    shape, and one small call replayed from a captured graph."""
    import statistics

    import torch

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(7)
    cases = [
        ("fp32 B1 H1 N256 d64", 1, 1, 256, 64, torch.float32, "plain"),
        ("fp32 B1 H1 N256 d64 graph replay", 1, 1, 256, 64, torch.float32, "graph"),
        ("bf16 B4 H16 N2048 d64", 4, 16, 2048, 64, torch.bfloat16, "plain"),
        ("fp16 B1 H32 N16384 d128", 1, 32, 16384, 128, torch.float16, "plain"),
        ("bf16 B2 H8 N4097 d128", 2, 8, 4097, 128, torch.bfloat16, "plain"),
        ("bf16 B4 H32 N16384 d128 causal", 4, 32, 16384, 128, torch.bfloat16, "causal"),
        ("fp8 B4 H32 N16384 d128 causal", 4, 32, 16384, 128, torch.bfloat16, "fp8causal"),
        ("fp8 B4 H32 N16384 d64", 4, 32, 16384, 64, torch.bfloat16, "fp8"),
        ("bf16 B1 H1 N16384 d128", 1, 1, 16384, 128, torch.bfloat16, "plain"),
        ("bf16 B1 H1 N16384 d128 split-KV", 1, 1, 16384, 128, torch.bfloat16, "split"),
        ("bf16 B1 H8 N4096 d128", 1, 8, 4096, 128, torch.bfloat16, "plain"),
        ("bf16 B1 H8 N4096 d128 split-KV", 1, 8, 4096, 128, torch.bfloat16, "split"),
    ] + [(f"bf16 B16 H64 N{n} d128", 16, 64, n, 128, torch.bfloat16, "plain") for n in (128, 256, 512)] + [
        ("bf16 B8 H32 decode Nq1 Nk16384 d128 split-KV", 8, 32, 16384, 128, torch.bfloat16, "decode"),
    ]
    rows = []
    for name, b, h, n, d, dt, mode in cases:
        nq = 1 if mode == "decode" else n
        q = torch.randn(b, h, nq, d, device=dev, dtype=dt, generator=gen)
        k, v = (torch.randn(b, h, n, d, device=dev, dtype=dt, generator=gen) for _ in range(2))
        o = torch.empty_like(q)
        lse = torch.empty(b, h, nq, device=dev, dtype=torch.float32)
        sc = 1.0 / math.sqrt(d)
        if mode == "decode":
            splits = fa.fa_fwd_splitkv_qk_splits(b, h, nq, n, d, dt)
            ws = torch.empty(max(1, fa.fa_fwd_splitkv_qk_workspace_bytes(b, h, nq, n, d, dt, splits)),
                             dtype=torch.uint8, device=dev)
            fn = lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, splits=splits, workspace=ws, scale=sc, stream=stream)
        elif mode == "graph":
            # the call captured once in a HIP graph and replayed: no per-call launch work
            s2 = torch.cuda.Stream()
            s2.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s2):
                fa.fa_fwd(q, k, v, o, lse, scale=sc)
            torch.cuda.current_stream().wait_stream(s2)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fa.fa_fwd(q, k, v, o, lse, scale=sc)
            fn = graph.replay
        elif mode in ("fp8", "fp8causal"):
            # codes and scales resident (quantised once, outside the timed launches)
            (q8, qs), (k8, ks), (vt8, vs) = (fa.fa_quantize_fp8(q), fa.fa_quantize_fp8(k),
                                             fa.fa_quantize_fp8(v, transpose=True))
            fn = lambda: fa.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, o, lse, scale=sc, stream=stream,
                                       causal=(mode == "fp8causal"))
        elif mode == "split":
            splits = fa.fa_fwd_splitkv_splits(b, h, n, d, dt)
            ws = torch.empty(max(1, fa.fa_fwd_splitkv_workspace_bytes(b, h, n, d, dt, splits)),
                             dtype=torch.uint8, device=dev)
            fn = lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, splits=splits, workspace=ws, scale=sc, stream=stream)
        else:
            fn = lambda: fa.fa_fwd(q, k, v, o, lse, scale=sc, stream=stream, causal=(mode == "causal"))
        t = launch_times(fn, stream, steps)
        tmin, tmed = min(t), statistics.median(t)
        flops = 4.0 * b * h * nq * n * d * (0.5 if mode in ("causal", "fp8causal") else 1.0)
        in_bytes = 1 if mode.startswith("fp8") else q.element_size()
        nbytes = (nq + 2.0 * n) * b * h * d * in_bytes + nq * b * h * d * q.element_size() + 4.0 * b * h * nq
        peak = 157.3 if dt == torch.float32 else PEAK_FP8_TFLOPS if mode.startswith("fp8") else PEAK_BF16_TFLOPS
        r = {"case": name, "min_ms": round(tmin, 4), "median_ms": round(tmed, 4),
             "tflops": round(flops / (tmed * 1e-3) / 1e12, 2),
             "pct_of_mfma_peak": round(100 * flops / (tmed * 1e-3) / 1e12 / peak, 2),
             "gbps": round(nbytes / (tmed * 1e-3) / 1e9, 1)}
        if mode in ("split", "decode"):
            r["splits"] = splits
        rows.append(r)
        log(f"sweep {name}: median {tmed * 1e3:.1f} us, min {tmin * 1e3:.1f} us, {r['tflops']} TFLOP/s "
            f"({r['pct_of_mfma_peak']}% of MFMA peak), {r['gbps']} GB/s algorithmic")
        del q, k, v, o, lse, fn
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--sweep", action="store_true", help="also time the smaller workloads")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' forward timings")
    ap.add_argument("--no-hbm-small-n", action="store_true", help="skip the short-sequence HBM leg")
    ap.add_argument("--no-causal", action="store_true", help="skip the causal forward leg")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--fp8-steps", type=int, default=10)
    ap.add_argument("--power-seconds", type=float, default=4.0,
                    help="run the forward this long while sampling socket power and clock (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many bytes (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}). The kernel's per-GPU share is the same "
              f"workload with B*H divided across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch

    import online_softmax_attention_fa_amd as fa

    fa.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scale = 1.0 / math.sqrt(D)

    gen = torch.Generator(device=dev).manual_seed(20240601)
    q = torch.randn(B, H, N, D, device=dev, dtype=torch.bfloat16, generator=gen)
    k = torch.randn(B, H, N, D, device=dev, dtype=torch.bfloat16, generator=gen)
    v = torch.randn(B, H, N, D, device=dev, dtype=torch.bfloat16, generator=gen)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    plan = fa.fa_fwd_plan(B, H, N, D, torch.bfloat16)
    log(f"plan: {plan}")

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration // 2, dtype=torch.bfloat16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration} bytes read + written")

    for _ in range(args.warmup):
        fa.fa_fwd(q, k, v, o, lse, scale=scale, stream=stream)
    torch.cuda.synchronize()

    # one event between consecutive launches: the sum is the bracketed time, the
    # differences give per-launch min and median
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        fa.fa_fwd(q, k, v, o, lse, scale=scale, stream=stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_launch = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms_per_step = max(kernel_ms, wall * 1e3 / args.steps)

    flops = 4.0 * B * H * N * N * D
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    traffic, traffic_note = traffic_from_profile()
    log(f"kernel {kernel_ms:.3f} ms/launch (events), wall {wall * 1e3 / args.steps:.3f} ms/step; "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / PEAK_BF16_TFLOPS:.1f}% of peak; traffic: {traffic_note}")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V drawn on the device (torch Philox), rounded to bf16",
        "config": {"workload": "attention forward, B=4 H=32 N=16384 d=128 bf16, non-causal, "
                               "scale=1/sqrt(d), LSE saved", "B": B, "H": H, "N": N, "d": D,
                   "causal": False, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * achieved / PEAK_BF16_TFLOPS, 2),
        "launch_ms": {"mean": round(kernel_ms, 4), "min": round(per_launch[0], 4),
                      "median": round(per_launch[len(per_launch) // 2], 4)},
        "plan": plan,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "mfma_busy": mfma_busy_from_profile(),
    }
    # the shorter legs run first, before the sustained power, backward and fp8 legs heat the chip
    if not args.no_configs:
        out["configs"] = configs_leg(fa, stream)
    if not args.no_hbm_small_n:
        out["hbm_small_n"] = hbm_small_n_leg(fa, stream)
    if not args.no_causal:
        out["causal"] = causal_leg(fa, q, k, v, scale, stream)
    if args.power_seconds > 0:
        pw = power_while_running(lambda: fa.fa_fwd(q, k, v, o, lse, scale=scale, stream=stream), args.power_seconds)
        if pw is not None:
            # the same FLOPs against the MFMA peak at the clock the chip actually ran
            pw["frac_of_peak_at_measured_clock"] = round(
                achieved / (PEAK_BF16_TFLOPS * pw["gfx_mhz_mean"] / 2400.0), 4)
        out["power"] = pw
        log(f"power: {pw}")
    grads = None
    if not args.no_backward:
        out["backward"], grads = time_backward(fa, q, k, v, o, lse, scale, stream, args.backward_steps)
    if not args.no_fp8:
        out["fp8"] = time_fp8(fa, q, k, v, o, scale, stream, args.fp8_steps)
    if args.sweep:
        out["sweep"] = sweep(fa, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(q, k, v, o, lse, scale)
        if grads is not None:
            out["cpu_baseline"]["backward_sample_check"] = backward_sample_check(q, k, v, *grads, scale)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
