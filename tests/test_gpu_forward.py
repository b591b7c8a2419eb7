"""GPU parity of the forward pass (through the C ABI) against the fp64 oracle.

Full outputs where the oracle finishes in seconds; sampled rows (every column of O
and LSE for 64 rows per head: tile-boundary rows plus seeded random ones) at the
large sizes, launched exactly as the benchmark launches them.
"""

import numpy as np
import pytest

import workloads as wl
from gpu_util import compare, run_fwd, scale_of, to_device, to_host
from oracle import attention_forward, attention_rows

pytestmark = pytest.mark.gpu


def _oracle_full(q, k, v, scale, causal=False):
    B, H = q.shape[:2]
    O = np.empty_like(q)
    L = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = attention_forward(q[b, h], k[b, h], v[b, h], scale, causal=causal)
    return O, L


def _random_qkv(B, H, N, d, dtype, seed, sigma=1.0):
    return tuple(wl.random_tensor((B, H, N, d), dtype, [seed, t], sigma) for t in (1, 2, 3))


# ---------------------------------------------------------------- workloads ---

@pytest.mark.parametrize("cid", [1, 2, 4])
def test_workload_full_parity(gpu_lib, cid):
    w = wl.WORKLOADS[cid]
    q, k, v = wl.make_inputs(w)
    O, L = run_fwd(gpu_lib, q, k, v, w.dtype)
    O_ref, L_ref = _oracle_full(q, k, v, w.scale)
    s = compare(O, L, O_ref, L_ref, w.dtype, w.name)
    print(f"{w.name}: {s}")
    if w.kind == "edge":
        # closed forms on the structured heads
        for b in range(w.B):
            for h in range(w.H):
                cat = wl.edge_category(b, h, w.H)
                if cat == 0:      # all-zero Q: LSE = ln N, O = column mean of V
                    np.testing.assert_allclose(L[b, h], np.log(w.N), atol=1e-4)
                    np.testing.assert_allclose(O[b, h], np.broadcast_to(v[b, h].mean(0), (w.N, w.d)),
                                               atol=1e-2)
                elif cat == 2:    # one-hot: O_i = V_{j*(i)} (up to the output rounding)
                    t = wl.boost_targets(w, b, h)
                    np.testing.assert_allclose(O[b, h], v[b, h][t], rtol=2 ** -8, atol=1e-6)


@pytest.mark.parametrize("cid", [3, 5])
def test_workload_sampled_rows(gpu_lib, cid):
    import torch

    w = wl.WORKLOADS[cid]
    q, k, v = wl.make_inputs(w, threads=16)
    tq, tk, tv = (to_device(x, w.dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    worst = {}
    for b in range(w.B):
        for h in range(w.H):
            rows = wl.sampled_rows(w, b, h)
            rr = torch.from_numpy(rows).cuda()
            Og = to_host(o[b, h].index_select(0, rr))
            Lg = lse[b, h].index_select(0, rr).cpu().numpy().astype(np.float64)
            O_ref, L_ref = attention_rows(q[b, h], k[b, h], v[b, h], w.scale, rows)
            s = compare(Og, Lg, O_ref, L_ref, w.dtype, f"{w.name} b{b} h{h}")
            worst = {key: max(worst.get(key, 0), val) for key, val in s.items()}
    # nothing anywhere is NaN/Inf
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()
    print(f"{w.name}: worst over heads {worst}")


# ------------------------------------------------------------- ragged tails ---

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 31, 33, 63, 64, 65, 127, 129, 255, 257, 700])
def test_tail_sweep(gpu_lib, dtype, d, N):
    q, k, v = _random_qkv(1, 2, N, d, dtype, seed=N * 1000 + d)
    O, L = run_fwd(gpu_lib, q, k, v, dtype)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    compare(O, L, O_ref, L_ref, dtype, f"N={N} d={d} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 5, 64, 129, 300, 1024])
def test_causal(gpu_lib, dtype, d, N):
    q, k, v = _random_qkv(2, 1, N, d, dtype, seed=7 * N + d)
    O, L = run_fwd(gpu_lib, q, k, v, dtype, causal=True)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d), causal=True)
    compare(O, L, O_ref, L_ref, dtype, f"causal N={N} d={d} {dtype}")


# ------------------------------------- one-wave last blocks: the keys split four ways ---

# (FA_TILE, d): every non-causal 4-wave kernel
TAIL_PLANS = [("128,32,4", 128), ("128,64,4", 128), ("128,64,4", 64), ("128,128,4", 64)]


@pytest.mark.parametrize("tile,d", TAIL_PLANS, ids=[f"{t}-d{d}" for t, d in TAIL_PLANS])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rows", [1, 17, 32])
def test_one_wave_last_block(gpu_lib, monkeypatch, tile, d, dtype, rows):
    # A last query block of `rows` <= 32 rows on a grid resident at once: its four waves all
    # take those rows and a quarter of the key tiles each (34 to 38 tiles: the last wave
    # holds fewer than the others), and merge through LDS.
    monkeypatch.setenv("FA_TILE", tile)
    bc = int(tile.split(",")[1])
    N = 128 * (32 * bc // 128 + 1) + rows
    plan = gpu_lib.fa_fwd_plan(1, 2, N, d, wl_dtype_code(dtype))
    assert plan["tail_kv_splits"] == 4, plan
    q, k, v = _random_qkv(1, 2, N, d, dtype, seed=N * 10 + d + rows)
    O, L = run_fwd(gpu_lib, q, k, v, dtype)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    compare(O, L, O_ref, L_ref, dtype, f"FA_TILE={tile} d={d} {dtype} N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_one_wave_last_block_large_scores(gpu_lib, monkeypatch, dtype):
    # Scores of several hundred: each wave's running maximum differs widely, so the merge
    # rescales the partials by factors that underflow to zero for some rows.
    monkeypatch.setenv("FA_TILE", "128,32,4")
    N, d = 1281, 128
    assert gpu_lib.fa_fwd_plan(1, 2, N, d, wl_dtype_code(dtype))["tail_kv_splits"] == 4
    sigma = 10.0 if dtype == "bf16" else 4.0
    q, k, v = _random_qkv(1, 2, N, d, dtype, seed=4242, sigma=sigma)
    v = wl.random_tensor(v.shape, dtype, [4242, 9])
    O, L = run_fwd(gpu_lib, q, k, v, dtype)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    compare(O, L, O_ref, L_ref, dtype, f"large scores N={N} {dtype}")


# ------------------------------------------------------------ extreme inputs ---

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_large_magnitude_scores(gpu_lib, dtype):
    # scores of several hundred (fp16 range limits the input scale)
    sigma = 10.0 if dtype == "bf16" else 4.0
    q, k, v = _random_qkv(1, 2, 1000, 128, dtype, seed=99, sigma=sigma)
    v = wl.random_tensor(v.shape, dtype, [99, 9])
    O, L = run_fwd(gpu_lib, q, k, v, dtype)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(128))
    compare(O, L, O_ref, L_ref, dtype, f"x{sigma} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_large_magnitude_scores_eight_wave_plans(gpu_lib, monkeypatch, dtype, d, causal):
    # Scores of several hundred on the long-sequence plans (8 waves; at d = 64 non-causal the
    # ping-pong schedule; causal d = 128 the 32-key plan): the running maximum jumps on later
    # tiles too, so tiles are redone with their own maximum, next to the diagonal masks.  The
    # plan is pinned through FA_TILE (the chooser picks by grid size).
    import torch

    B, H, N = 4, 16, 2100
    monkeypatch.setenv("FA_TILE", "128,32,4" if causal and d == 128 else "256,128,8")
    plan = gpu_lib.fa_fwd_plan(B, H, N, d, wl_dtype_code(dtype), causal=causal)
    assert plan["waves"] == (4 if causal and d == 128 else 8)
    sigma = 10.0 if dtype == "bf16" else 4.0
    q, k, _ = _random_qkv(B, H, N, d, dtype, seed=77 + d, sigma=sigma)
    v = wl.random_tensor((B, H, N, d), dtype, [77 + d, 9])
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv, causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng([77, d])
    for b in range(B):
        for h in range(0, H, 3):
            rows = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.choice(N, 12, replace=False)]))
            rr = torch.from_numpy(rows).cuda()
            Og = to_host(o[b, h].index_select(0, rr))
            Lg = lse[b, h].index_select(0, rr).cpu().numpy().astype(np.float64)
            O_ref, L_ref = attention_rows(q[b, h], k[b, h], v[b, h], scale_of(d), rows, causal=causal)
            compare(Og, Lg, O_ref, L_ref, dtype, f"x{sigma} {dtype} d{d} causal={causal} b{b} h{h}")
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_short_heads_three_per_cu_plan(gpu_lib, dtype, d):
    # Many short heads (N = 300: four full 64-key tiles and a ragged one) take the
    # three-workgroups-per-CU plan: 64-key tiles at d = 64, 32-key tiles at d = 128.
    import torch

    B, H, N = 16, 32, 300
    plan = gpu_lib.fa_fwd_plan(B, H, N, d, wl_dtype_code(dtype))
    assert plan["waves"] == 4 and plan["block_k"] == (64 if d == 64 else 32)
    q, k, v = _random_qkv(B, H, N, d, dtype, seed=300 + d)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    for b in range(0, B, 5):
        for h in range(0, H, 7):
            O_ref, L_ref = attention_forward(q[b, h], k[b, h], v[b, h], scale_of(d))
            compare(to_host(o[b, h]), lse[b, h].cpu().numpy().astype(np.float64), O_ref, L_ref, dtype,
                    f"short heads {dtype} d{d} b{b} h{h}")
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()


def test_custom_scale_and_stream(gpu_lib):
    import torch

    q, k, v = _random_qkv(2, 3, 333, 64, "bf16", seed=5)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        O, L = run_fwd(gpu_lib, q, k, v, "bf16", scale=0.05, stream=s)
    O_ref, L_ref = _oracle_full(q, k, v, 0.05)
    compare(O, L, O_ref, L_ref, "bf16", "scale=0.05 side stream")


def test_deterministic_bitwise(gpu_lib):
    import torch

    q, k, v = _random_qkv(2, 4, 1500, 128, "bf16", seed=3)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = gpu_lib.fa_fwd(tq, tk, tv)
    o2, l2 = gpu_lib.fa_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_key_value_permutation_invariance(gpu_lib):
    # Jointly permuting K and V rows leaves the exact result unchanged; the GPU result
    # changes only by rounding.
    q, k, v = _random_qkv(1, 2, 777, 128, "bf16", seed=11)
    perm = np.random.default_rng(0).permutation(777)
    O1, L1 = run_fwd(gpu_lib, q, k, v, "bf16")
    O2, L2 = run_fwd(gpu_lib, q, k[:, :, perm], v[:, :, perm], "bf16")
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(128))
    compare(O1, L1, O_ref, L_ref, "bf16", "original order")
    compare(O2, L2, O_ref, L_ref, "bf16", "permuted keys")


def test_empty_problem_is_a_no_op(gpu_lib):
    import torch

    z = torch.zeros(2, 3, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = gpu_lib.fa_fwd(z, z, z)
    assert o.shape == z.shape and lse.shape == (2, 3, 0)


# ------------------------------------------- 8-wave plan: long rows, ragged tails ---

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,causal", [(2049, False), (3000, False), (8191, False), (2500, True), (4099, True)])
def test_eight_wave_plan_sampled(gpu_lib, monkeypatch, dtype, d, N, causal):
    # The 8-wave, 128-key-tile plan (causal at d = 128: the 4-wave, 32-key-tile plan at three
    # waves per SIMD), pinned through FA_TILE; rows past the last full query block and keys
    # past the last full tile exercise the masks.
    import torch

    B, H = 4, 16
    monkeypatch.setenv("FA_TILE", "128,32,4" if causal and d == 128 else "256,128,8")
    plan = gpu_lib.fa_fwd_plan(B, H, N, d, wl_dtype_code(dtype), causal=causal)
    if causal and d == 128:
        assert plan["waves"] == 4 and plan["block_k"] == 32
    else:
        assert plan["waves"] == 8 and plan["block_k"] == 128
    q, k, v = _random_qkv(B, H, N, d, dtype, seed=N * 7 + d + int(causal))
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv, causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng([N, d])
    for b, h in ((0, 0), (1, 7), (3, 15)):
        rows = np.unique(np.concatenate([[0, 255, 256, N - 257, N - 256, N - 1], rng.choice(N, 40, replace=False)]))
        rows = rows[(rows >= 0) & (rows < N)]
        rr = torch.from_numpy(rows).cuda()
        Og = to_host(o[b, h].index_select(0, rr))
        Lg = lse[b, h].index_select(0, rr).cpu().numpy().astype(np.float64)
        O_ref, L_ref = attention_rows(q[b, h], k[b, h], v[b, h], scale_of(d), rows, causal=causal)
        compare(Og, Lg, O_ref, L_ref, dtype, f"N={N} d={d} {dtype} causal={causal} b{b} h{h}")
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("B,H,N", [(5, 8, 2001), (2, 8, 4300)])
def test_three_per_cu_plan_sampled(gpu_lib, dtype, B, H, N):
    # grids just over one round of two 128-row workgroups per CU run on the 32-key-tile
    # kernel at three per CU (non-causal); ragged last query block and key tile
    import torch

    d = 128
    plan = gpu_lib.fa_fwd_plan(B, H, N, d, wl_dtype_code(dtype))
    assert plan["waves"] == 4 and plan["block_k"] == 32
    q, k, v = _random_qkv(B, H, N, d, dtype, seed=N + B)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    rng = np.random.default_rng([N, B])
    for b, h in ((0, 0), (B - 1, H - 1), (B // 2, 3)):
        rows = np.unique(np.concatenate([[0, 31, 32, 127, 128, N - 129, N - 128, N - 1], rng.choice(N, 40, replace=False)]))
        rows = rows[(rows >= 0) & (rows < N)]
        rr = torch.from_numpy(rows).cuda()
        Og = to_host(o[b, h].index_select(0, rr))
        Lg = lse[b, h].index_select(0, rr).cpu().numpy().astype(np.float64)
        O_ref, L_ref = attention_rows(q[b, h], k[b, h], v[b, h], scale_of(d), rows)
        compare(Og, Lg, O_ref, L_ref, dtype, f"B{B} H{H} N={N} {dtype} b{b} h{h}")


TAIL_FIRST = [
    # (B, H, N, d, dtype): 8-wave plans whose last N % 256 rows run ahead of the main launch
    (2, 8, 4097, 128, "bf16"),    # one round of 256 full blocks, one last row per head
    (2, 8, 4097, 64, "fp16"),     # d = 64: the ping-pong main launch
    (2, 4, 8193, 128, "fp16"),
    (2, 8, 4128, 128, "bf16"),    # 32 last rows
    (2, 8, 4113, 64, "bf16"),     # 17 last rows
    (2, 8, 4160, 128, "bf16"),    # 64 last rows: two waves of the split-KV block
    (2, 8, 4224, 128, "fp16"),    # 128 last rows: the whole split-KV block
    (2, 8, 4196, 64, "bf16"),     # 100 last rows
]


@pytest.mark.parametrize("B,H,N,d,dtype", TAIL_FIRST, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{c[4]}" for c in TAIL_FIRST])
def test_tail_first(gpu_lib, B, H, N, d, dtype):
    # The split-KV launch computes the last rows of every head into partials parked in the
    # head's first O rows, the merge writes those rows' O and LSE, and the 8-wave launch then
    # overwrites the parked partials with the full blocks' outputs: every row equals the oracle.
    plan = gpu_lib.fa_fwd_plan(B, H, N, d, wl_dtype_code(dtype))
    assert plan["waves"] == 8 and plan["tail_kv_splits"] > 1 and plan["grid"] == B * H * (N // 256), plan
    q, k, v = _random_qkv(B, H, N, d, dtype, seed=N * 7 + d)
    O, L = run_fwd(gpu_lib, q, k, v, dtype)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    compare(O, L, O_ref, L_ref, dtype, f"tail first B{B} H{H} N{N} d{d} {dtype}")


def test_tail_first_non_finite(gpu_lib):
    # NaN in a last row's query stays in that row; a NaN key in the last split's range reaches
    # every row, the last rows through the merge; a NaN value row reaches every output row but
    # no LSE.
    B, H, N, d, dtype = 2, 8, 4097, 128, "bf16"
    assert gpu_lib.fa_fwd_plan(B, H, N, d, wl_dtype_code(dtype))["tail_kv_splits"] > 1
    q, k, v = _random_qkv(B, H, N, d, dtype, seed=99)
    qn = q.copy(); qn[1, 5, N - 1, 7] = np.nan
    O, L = run_fwd(gpu_lib, qn, k, v, dtype)
    bad_o, bad_l = ~np.isfinite(O), ~np.isfinite(L)
    assert bad_o[1, 5, N - 1].all() and bad_l[1, 5, N - 1]
    bad_o[1, 5, N - 1] = False; bad_l[1, 5, N - 1] = False
    assert not bad_o.any() and not bad_l.any(), "a NaN query row leaked"
    kn = k.copy(); kn[0, 2, N - 2, 3] = np.nan
    O, L = run_fwd(gpu_lib, q, kn, v, dtype)
    assert (~np.isfinite(O[0, 2])).all(axis=1).all() and (~np.isfinite(L[0, 2])).all()
    assert np.isfinite(O[0, 3]).all() and np.isfinite(L[1]).all(), "a NaN key leaked to another head"
    vn = v.copy(); vn[1, 1, 10, 4] = np.nan
    O, L = run_fwd(gpu_lib, q, k, vn, dtype)
    assert (~np.isfinite(O[1, 1, :, 4])).all() and np.isfinite(L).all()


def test_tail_first_not_taken_when_o_overlaps_an_input(gpu_lib, capfd, monkeypatch):
    # O written over Q (each block reads its own Q rows before it writes them): the parked
    # partials would overwrite queries not read yet, so the call takes the 8-wave grid with
    # its short last block instead, and the result still equals the oracle.
    import torch

    B, H, N, d, dtype = 2, 8, 4097, 128, "bf16"
    q, k, v = _random_qkv(B, H, N, d, dtype, seed=5)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    monkeypatch.setenv("FA_LOG", "1")
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    assert "rows first" in capfd.readouterr().err
    compare(to_host(o), lse.cpu().numpy().astype(np.float64), O_ref, L_ref, dtype, "separate O")
    o2, lse2 = gpu_lib.fa_fwd(tq, tk, tv, o=tq)
    torch.cuda.synchronize()
    assert "rows first" not in capfd.readouterr().err
    compare(to_host(o2), lse2.cpu().numpy().astype(np.float64), O_ref, L_ref, dtype, "O over Q")


IN_PLACE = [
    # (B, H, N, d, dtype, causal, FA_TILE): O written over Q on each kind of plan
    (2, 8, 4300, 128, "bf16", False, ""),           # 4 waves, 32-key tiles, three per CU
    (1, 2, 1153, 128, "bf16", False, "128,32,4"),   # the last block's waves split its keys
    (2, 4, 2100, 64, "fp16", False, "256,128,8"),   # ping-pong
    (1, 4, 1500, 128, "bf16", True, ""),            # causal
    (1, 2, 300, 64, "fp32", False, ""),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal,tile", IN_PLACE,
                         ids=[f"{c[4]}-N{c[2]}-d{c[3]}{'-causal' if c[5] else ''}{'-' + c[6] if c[6] else ''}" for c in IN_PLACE])
def test_in_place_over_q(gpu_lib, monkeypatch, B, H, N, d, dtype, causal, tile):
    # Every workgroup reads its own query rows before it writes their outputs, so O may be
    # Q's memory (fa.h); the result equals the oracle's on the original queries.
    import torch

    if tile:
        monkeypatch.setenv("FA_TILE", tile)
    q, k, v = _random_qkv(B, H, N, d, dtype, seed=N + d + 3)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d), causal=causal)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = gpu_lib.fa_fwd(tq, tk, tv, o=tq, causal=causal)
    torch.cuda.synchronize()
    assert o.data_ptr() == tq.data_ptr()
    compare(to_host(o), lse.cpu().numpy().astype(np.float64), O_ref, L_ref, dtype, f"in place {dtype} N={N}")


def wl_dtype_code(dtype):
    import online_softmax_attention_fa_amd as fa

    return {"fp32": fa.FA_F32, "fp16": fa.FA_F16, "bf16": fa.FA_BF16}[dtype]


# ------------------------------------------------------------ non-finite inputs ---

NON_FINITE_CASES = [
    # (dtype, N, d, FA_TILE, query rows poisoned, key row poisoned, value row poisoned)
    ("bf16", 300, 64, "", 77, 140, 200, 31),
    ("fp16", 300, 64, "", 77, 140, 200, 31),
    ("fp32", 300, 64, "", 77, 140, 200, 31),
    # one-row last block whose waves split the keys (37 tiles): the NaN key lies in the last
    # wave's quarter, so it must survive the merge into wave 0; the Inf row is that block's
    ("bf16", 1153, 128, "128,32,4", 77, 1152, 1000, 31),
    ("fp16", 1153, 128, "128,32,4", 77, 1152, 1000, 31),
]


@pytest.mark.parametrize("dtype,N,d,tile,qnan,qinf,knan,vnan", NON_FINITE_CASES,
                         ids=[f"{c[0]}-N{c[1]}-d{c[2]}" for c in NON_FINITE_CASES])
def test_non_finite_inputs_propagate(gpu_lib, monkeypatch, dtype, N, d, tile, qnan, qinf, knan, vnan):
    """A NaN or Inf in query row i reaches row i's output and LSE only; a NaN in key row j
    reaches every row (each score row contains key j); a NaN in value row j reaches every
    output row but no LSE.  Rows not touched stay equal to the oracle."""
    import torch

    if tile:
        monkeypatch.setenv("FA_TILE", tile)
        assert gpu_lib.fa_fwd_plan(1, 1, N, d, wl_dtype_code(dtype))["tail_kv_splits"] == 4
    q, k, v = _random_qkv(1, 1, N, d, dtype, seed=7)
    O_ref, L_ref = _oracle_full(q, k, v, scale_of(d))
    cases = {
        "q row NaN": (q.copy(), k, v, "q"),
        "q row Inf": (q.copy(), k, v, "qinf"),
        "k row NaN": (q, k.copy(), v, "k"),
        "v row NaN": (q, k, v.copy(), "v"),
    }
    cases["q row NaN"][0][0, 0, qnan, 5] = np.nan
    cases["q row Inf"][0][0, 0, qinf, 3] = np.inf
    cases["k row NaN"][1][0, 0, knan, 9] = np.nan
    cases["v row NaN"][2][0, 0, vnan, 2] = np.nan
    for name, (qq, kk, vv, kind) in cases.items():
        O, L = run_fwd(gpu_lib, qq, kk, vv, dtype)
        bad_o = ~np.isfinite(O[0, 0])
        bad_l = ~np.isfinite(L[0, 0])
        if kind in ("q", "qinf"):
            row = qnan if kind == "q" else qinf
            assert bad_o[row].all() or bad_l[row], f"{name}: row {row} stayed finite"
            others = np.arange(N) != row
            assert not bad_o[others].any() and not bad_l[others].any(), f"{name}: leaked to other rows"
            compare(O[:, :, others], L[:, :, others], O_ref[:, :, others], L_ref[:, :, others], dtype, name)
        elif kind == "k":
            assert bad_o.all(axis=1).all() and bad_l.all(), f"{name}: some row stayed finite"
        else:
            assert bad_o[:, 2].all(), f"{name}: the poisoned column stayed finite in some row"
            assert not bad_l.any(), f"{name}: a NaN value leaked into the LSE"
