"""The entry points inside a captured HIP graph.

"从零理解Flash Attention中的online softmax" (section 6.2) captures the whole attention
computation in a graph so that replays skip the launch overhead.  The library's calls
queue kernels on the caller's stream and allocate nothing, so they can be captured: here
the forward, the split-KV forward (partial kernel + merge) and the backward (three
kernels) go into one graph, which is replayed several times with eager work and
synchronisations between replays; every replay must reproduce the eager results bit for
bit.
"""

import pytest

pytestmark = pytest.mark.gpu


def test_forward_splitkv_backward_in_one_graph(gpu_lib):
    import torch

    fa = gpu_lib
    B, H, N, d = 2, 3, 700, 128
    gen = torch.Generator(device="cuda").manual_seed(31)
    q, k, v, do = (torch.randn(B, H, N, d, device="cuda", dtype=torch.bfloat16, generator=gen) for _ in range(4))
    o, o2 = torch.empty_like(q), torch.empty_like(q)
    lse, lse2 = (torch.empty(B, H, N, device="cuda", dtype=torch.float32) for _ in range(2))
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    splits = 3
    ws_fwd = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(B, H, N, d, torch.bfloat16, splits),
                         dtype=torch.uint8, device="cuda")
    ws_bwd = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d, torch.bfloat16), dtype=torch.uint8, device="cuda")

    def work(stream):
        fa.fa_fwd(q, k, v, o, lse, stream=stream)
        fa.fa_fwd_splitkv(q, k, v, o2, lse2, splits=splits, workspace=ws_fwd, stream=stream)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws_bwd, stream=stream)

    # eager reference
    work(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, o2, lse2, dq, dk, dv)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):       # warm-up on the capture stream
        work(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(torch.cuda.current_stream())

    outs = (o, lse, o2, lse2, dq, dk, dv)
    for rep in range(4):
        for t in outs:                # eager work between replays; outputs must be rewritten
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("o", "lse", "o_split", "lse_split", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(t.view(torch.int8), r.view(torch.int8)), f"replay {rep}: {name} differs"


def test_fp8_and_causal_in_one_graph(gpu_lib):
    """The fp8 quantiser (including V^T's zero padding) and the fp8 and 16-bit causal
    forwards, captured together and replayed with the outputs poisoned in between."""
    import torch

    fa = gpu_lib
    B, H, N, d = 2, 3, 333, 64
    gen = torch.Generator(device="cuda").manual_seed(32)
    q, k, v = (torch.randn(B, H, N, d, device="cuda", dtype=torch.bfloat16, generator=gen) for _ in range(3))
    Np, nb = fa.fa_fp8_padded_len(N), fa.fa_fp8_scale_blocks(N)
    q8, k8 = (torch.empty(B, H, N, d, dtype=torch.uint8, device="cuda") for _ in range(2))
    vt8 = torch.empty(B, H, d, Np, dtype=torch.uint8, device="cuda")
    qs, ks, vs = (torch.empty(B, H, nb, dtype=torch.float32, device="cuda") for _ in range(3))
    o8, o8c, oc = (torch.empty_like(q) for _ in range(3))
    l8, l8c, lc = (torch.empty(B, H, N, device="cuda", dtype=torch.float32) for _ in range(3))

    def work(stream):
        fa.fa_quantize_fp8(q, x8=q8, scales=qs, stream=stream)
        fa.fa_quantize_fp8(k, x8=k8, scales=ks, stream=stream)
        fa.fa_quantize_fp8(v, transpose=True, x8=vt8, scales=vs, stream=stream)
        fa.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, o8, l8, stream=stream)
        fa.fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, o8c, l8c, stream=stream, causal=True)
        fa.fa_fwd(q, k, v, oc, lc, causal=True, stream=stream)

    work(torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = (q8, k8, vt8, qs, ks, vs, o8, l8, o8c, l8c, oc, lc)
    ref = [t.clone() for t in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(torch.cuda.current_stream())

    names = ("q8", "k8", "vt8", "qs", "ks", "vs", "o_fp8", "lse_fp8", "o_fp8_causal", "lse_fp8_causal",
             "o_causal", "lse_causal")
    for rep in range(4):
        for t in outs:
            if t.dtype == torch.uint8:
                t.fill_(0x7F)          # a NaN code, and non-zero in V^T's padding
            else:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(names, outs, ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: {name} differs"


def test_ping_pong_and_short_head_forwards_in_one_graph(gpu_lib, monkeypatch):
    """The d = 64 ping-pong schedule (8-wave plan, three stages; pinned through FA_TILE), the
    three-per-CU short-head plans (d = 64 and d = 128) and a tail-first forward (its split-KV
    and merge launches ahead of the 8-wave one, partials parked in O) captured together;
    every replay must reproduce the eager results bit for bit, with O and the LSE filled with
    NaN before each."""
    import os

    import torch

    fa = gpu_lib
    gen = torch.Generator(device="cuda").manual_seed(37)
    shapes = ((4, 16, 2100, 64), (16, 32, 300, 64), (16, 32, 300, 128), (2, 8, 4097, 128))
    tiles = ("256,128,8", "", "", "")     # the library reads FA_TILE at each call
    plans = []
    for sh, tile in zip(shapes, tiles):
        monkeypatch.setenv("FA_TILE", tile)
        plans.append(fa.fa_fwd_plan(*sh, torch.bfloat16))
    assert (plans[0]["waves"], plans[0]["block_k"]) == (8, 128)
    assert (plans[1]["waves"], plans[1]["block_k"]) == (4, 64)
    assert (plans[2]["waves"], plans[2]["block_k"]) == (4, 32)
    assert (plans[3]["waves"], plans[3]["block_k"], plans[3]["tail_kv_splits"]) == (8, 128, 16)
    ins = [tuple(torch.randn(*sh, device="cuda", dtype=torch.bfloat16, generator=gen) for _ in range(3))
           for sh in shapes]
    outs = [(torch.empty_like(q), torch.empty(q.shape[:3], device="cuda", dtype=torch.float32)) for q, _, _ in ins]

    def work(stream):
        for (q, k, v), (o, lse), tile in zip(ins, outs, tiles):
            os.environ["FA_TILE"] = tile
            fa.fa_fwd(q, k, v, o, lse, stream=stream)

    work(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [(o.clone(), lse.clone()) for o, lse in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(torch.cuda.current_stream())

    for rep in range(3):
        for o, lse in outs:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((o, lse), (ro, rl)) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.int16), ro.view(torch.int16)), f"replay {rep}: O of shape {shapes[i]}"
            assert torch.equal(lse.view(torch.int32), rl.view(torch.int32)), f"replay {rep}: LSE of shape {shapes[i]}"
