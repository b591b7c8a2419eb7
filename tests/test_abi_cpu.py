"""The C ABI on the CPU: libfa.so loads, exports every symbol include/fa.h declares,
validates arguments before touching a device, and reports its launch plan.

No compute call is made here.  Pointers passed to the validating calls are fake
(never dereferenced); with valid arguments and no GPU the call must stop at the
device check with FA_ERR_DEVICE.
"""

import ctypes
import functools
import os
import re

import pytest

import online_softmax_attention_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M)))


def exported_symbols():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(fa.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    syms = exported_symbols()
    for name in declared_functions():
        assert name in syms, f"{name} declared in fa.h but not exported"
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.fa_version() >= 100
    for code, name in fa.STATUS.items():
        assert lib.fa_status_str(code).decode().startswith(name)
    assert lib.fa_status_str(99).decode() == "FA_ERR_UNKNOWN"


FAKE = 0x10000  # 16-byte aligned, never dereferenced


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=64, d=64, scale=0.125,
         dtype=fa.FA_BF16, causal=False):
    fn = lib.fa_fwd_causal if causal else lib.fa_fwd
    return fn(q, k, v, o, lse, B, H, N, d, scale, dtype, None)


@pytest.mark.parametrize("causal", [False, True])
def test_validation_order_and_codes(lib, causal):
    assert _fwd(lib, q=None, causal=causal) == 1
    assert _fwd(lib, q=None, N=-1, causal=causal) == 2        # shape before pointers
    assert _fwd(lib, q=None, d=80, causal=causal) == 3
    assert _fwd(lib, q=None, N=0, causal=causal) == 0         # empty: NULL allowed
    assert _fwd(lib, lse=None, causal=causal) == 1
    assert _fwd(lib, N=-1, causal=causal) == 2
    assert _fwd(lib, B=-2, causal=causal) == 2
    assert _fwd(lib, d=96, causal=causal) == 3
    assert _fwd(lib, d=256, causal=causal) == 3
    assert _fwd(lib, dtype=7, causal=causal) == 3
    assert _fwd(lib, q=FAKE + 8, causal=causal) == 4
    assert _fwd(lib, o=FAKE + 4, causal=causal) == 4
    assert _fwd(lib, lse=FAKE + 2, causal=causal) == 4
    assert _fwd(lib, lse=FAKE + 4, causal=causal) != 4       # LSE needs only 4-byte alignment
    assert _fwd(lib, scale=0.0, causal=causal) == 5
    assert _fwd(lib, scale=-1.0, causal=causal) == 5
    assert _fwd(lib, scale=float("inf"), causal=causal) == 5
    assert _fwd(lib, scale=float("nan"), causal=causal) == 5
    # shape overflow of the 32-bit per-head index math
    assert _fwd(lib, N=1 << 25, d=128, causal=causal) == 2
    # empty problems succeed without touching a device
    assert _fwd(lib, B=0, causal=causal) == 0
    assert _fwd(lib, N=0, causal=causal) == 0


def test_valid_call_without_gpu_stops_at_device_check(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the device check passes")
    assert _fwd(lib) == 6
    assert _fwd(lib, causal=True) == 6


WS = 0x20000  # 256-byte aligned fake workspace


def _bwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=WS,
         ws_bytes=None, B=1, H=2, N=64, d=64, scale=0.125, dtype=fa.FA_BF16, causal=False):
    if ws_bytes is None:
        ws_bytes = 2 * 4 * B * H * N + 512
    fn = lib.fa_bwd_causal if causal else lib.fa_bwd
    return fn(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, N, d, scale, dtype, None)


def test_bwd_workspace_size(lib):
    # two fp32 arrays of B*H*N, each rounded up to 256 bytes
    assert lib.fa_bwd_workspace_bytes(1, 1, 64, 64, fa.FA_BF16) == 512
    assert lib.fa_bwd_workspace_bytes(1, 1, 65, 64, fa.FA_BF16) == 1024
    assert lib.fa_bwd_workspace_bytes(4, 32, 16384, 128, fa.FA_BF16) == 2 * 4 * 4 * 32 * 16384
    assert lib.fa_bwd_workspace_bytes(1, 1, 64, 80, fa.FA_BF16) == 0
    assert lib.fa_bwd_workspace_bytes(1, -1, 64, 64, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_bytes(2, 8, 4097, 128, fa.FA_F16) == 2 * (-(-2 * 8 * 4097 * 4 // 256) * 256)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_validation_order_and_codes(lib, causal):
    assert _bwd(lib, q=None, causal=causal) == 1
    assert _bwd(lib, dv=None, causal=causal) == 1
    assert _bwd(lib, do=None, N=-1, causal=causal) == 2
    assert _bwd(lib, d=96, causal=causal) == 3
    assert _bwd(lib, dtype=fa.FA_F32, causal=causal) == 3     # backward: 16-bit inputs only
    assert _bwd(lib, q=None, N=0, causal=causal) == 0         # empty: NULLs allowed
    assert _bwd(lib, ws=None, N=0, causal=causal) == 0
    assert _bwd(lib, dk=FAKE + 8, causal=causal) == 4
    assert _bwd(lib, do=FAKE + 2, causal=causal) == 4
    assert _bwd(lib, lse=FAKE + 2, causal=causal) == 4
    assert _bwd(lib, scale=0.0, causal=causal) == 5
    assert _bwd(lib, scale=float("nan"), causal=causal) == 5
    assert _bwd(lib, ws=None, causal=causal) == 8
    assert _bwd(lib, ws=WS + 16, causal=causal) == 8          # 256-byte alignment
    assert _bwd(lib, ws_bytes=511, causal=causal) == 8
    assert _bwd(lib, N=1 << 25, d=128, causal=causal) == 2


def test_bwd_valid_call_without_gpu_stops_at_device_check(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the device check passes")
    assert _bwd(lib) == 6
    assert _bwd(lib, causal=True, dtype=fa.FA_F16, d=128) == 6


@pytest.mark.parametrize("dtype", [fa.FA_F32, fa.FA_F16, fa.FA_BF16])
@pytest.mark.parametrize("d", [64, 128])
def test_plan_respects_lds_and_covers_rows(lib, dtype, d):
    for (B, H, N) in [(1, 1, 1), (1, 1, 256), (4, 16, 2048), (2, 8, 4097), (4, 32, 16384)]:
        p = fa.fa_fwd_plan(B, H, N, d, dtype)
        assert p["lds_bytes"] <= 160 * 1024
        assert p["waves"] * 64 <= 1024
        assert p["block_q"] * p["wave_kv_splits"] == p["waves"] * p["rows_per_wave"]
        assert p["rows_per_wave"] % 32 == 0 and p["block_k"] % 32 == 0
        tail_first = p["waves"] == 8 and p["tail_kv_splits"] > 1
        assert p["grid"] == B * H * (N // p["block_q"] if tail_first else -(-N // p["block_q"]))
        assert not tail_first or 1 <= N % 256 <= 32
        assert p["kv_splits"] >= 1


def test_plan_splits_the_keys_of_a_short_last_block_only_on_grids_resident_at_once(lib, monkeypatch):
    # On the 4-wave plans (pinned here through FA_TILE) the last query block's waves share its
    # <= 32 rows and split the key tiles four ways when the grid fits in one round, with at
    # least 32 key tiles.
    def tail(B, H, N, d, dtype=fa.FA_BF16, causal=False):
        return fa.fa_fwd_plan(B, H, N, d, dtype, causal=causal)["tail_kv_splits"]

    monkeypatch.setenv("FA_TILE", "128,32,4")
    assert tail(2, 8, 4097, 128) == 4            # 528 workgroups at three per CU: one round
    assert tail(2, 8, 4097, 128, fa.FA_F16) == 4
    assert tail(2, 8, 4128, 128) == 4            # 32 rows in the last block
    assert tail(2, 4, 8193, 128) == 4
    assert tail(2, 8, 4129, 128) == 1            # 33 rows: two waves hold rows
    assert tail(4, 8, 4097, 128) == 1            # 1056 workgroups: more than one round
    assert tail(2, 8, 4097, 128, causal=True) == 1
    assert tail(1, 2, 257, 128) == 1             # 9 key tiles: too few to share
    monkeypatch.setenv("FA_TILE", "128,64,4")
    assert tail(2, 8, 4097, 64) == 4             # 64-key tiles at three per CU
    monkeypatch.delenv("FA_TILE")
    assert tail(1, 1, 4097, 64, fa.FA_F32) == 1
    assert tail(0, 8, 4097, 128) == 0            # empty problem: the plan is all zeros
    assert tail(2, 8, 4300, 128) == 1            # the chooser's 4-wave plan, 76 last rows


def test_plan_computes_the_last_rows_first_on_eight_wave_grids(lib):
    # N = 256 k + r, 1 <= r <= 128, where the 8-wave grid of full blocks costs less than the one
    # with the short last blocks: the r rows of every head go ahead of the main launch on
    # tail_kv_splits workgroups per head (about 256 in all, at most 16 key tiles per range),
    # and the main grid covers the full blocks only.
    def plan(B, H, N, d=128, dtype=fa.FA_BF16, causal=False):
        p = fa.fa_fwd_plan(B, H, N, d, dtype, causal=causal)
        return p["waves"], p["grid"], p["tail_kv_splits"]

    assert plan(2, 8, 4097) == (8, 256, 16)      # one round of 256 full blocks
    assert plan(2, 8, 4097, dtype=fa.FA_F16) == (8, 256, 16)
    assert plan(2, 8, 4097, d=64) == (8, 256, 16)
    assert plan(2, 8, 4128) == (8, 256, 16)      # 32 last rows
    assert plan(2, 4, 8193) == (8, 256, 32)      # 129 key tiles of 64: 16 per range at most
    assert plan(4, 8, 4097) == (8, 512, 8)       # two rounds
    assert plan(8, 8, 4097) == (8, 1024, 5)      # four rounds; 65 key tiles, at most 16 per range
    assert plan(2, 8, 16385) == (8, 1024, 17)
    assert plan(4, 16, 2049) == (8, 512, 4)
    assert plan(2, 8, 4129) == (8, 256, 16)      # 33 last rows
    assert plan(2, 8, 4224) == (8, 256, 15)      # 128 last rows: 15 ranges fill the room in O
    assert plan(2, 8, 4225)[0] == 4              # 129: more than one split-KV block per head
    assert plan(3, 8, 4097) == (8, 408, 1)       # the last round has room for the short blocks
    assert plan(1, 8, 4097) == (8, 136, 1)       # under one round: likewise
    assert plan(4, 32, 16384)[2] == 1            # no short block
    assert plan(16, 64, 2049)[0] == 4            # 1024 heads: the second pass over K and V costs more
    assert plan(8, 16, 2049)[0] == 4
    assert plan(2, 8, 4097, causal=True)[2] == 1
    assert plan(2, 8, 4097, dtype=fa.FA_F32)[2] == 1


def test_plan_takes_three_workgroups_per_cu_for_a_grid_just_over_one_round_or_short_heads(lib):
    # 528 workgroups of 128 rows: two per CU leave a nearly empty second round, three per
    # CU (32-key tiles) fit them in one; causal grids and full rounds keep 64-key tiles
    p = fa.fa_fwd_plan(2, 8, 4300, 128, fa.FA_BF16)
    assert (p["waves"], p["block_k"], p["grid"]) == (4, 32, 544)
    assert fa.fa_fwd_plan(5, 8, 2048, 128, fa.FA_F16)["block_k"] == 32
    assert fa.fa_fwd_plan(2, 8, 4300, 128, fa.FA_BF16, causal=True)["block_k"] == 64
    # short sequences with two or more 128-row workgroups per CU also take 32-key tiles
    # (latency-bound: a third resident workgroup overlaps copies with compute); a small
    # grid, or a causal one, keeps 64-key tiles
    assert fa.fa_fwd_plan(16, 16, 1024, 128, fa.FA_BF16)["block_k"] == 32
    assert fa.fa_fwd_plan(16, 64, 128, 128, fa.FA_BF16)["block_k"] == 32
    assert fa.fa_fwd_plan(1, 8, 1024, 128, fa.FA_BF16)["block_k"] == 64
    assert fa.fa_fwd_plan(16, 16, 1024, 128, fa.FA_BF16, causal=True)["block_k"] == 64
    # d = 64 short heads: 64-key tiles at three per CU; small grids and causal keep 128
    p = fa.fa_fwd_plan(16, 64, 512, 64, fa.FA_BF16)
    assert (p["waves"], p["block_k"], p["lds_bytes"]) == (4, 64, 32768)
    assert fa.fa_fwd_plan(1, 8, 512, 64, fa.FA_BF16)["block_k"] == 128
    assert fa.fa_fwd_plan(16, 64, 512, 64, fa.FA_BF16, causal=True)["block_k"] == 128
    # under one round of 256-row blocks: one 8-wave workgroup per CU on 216 CUs beats 432
    # four-wave ones at up to two per CU
    p = fa.fa_fwd_plan(3, 6, 3000, 128, fa.FA_BF16)
    assert (p["waves"], p["block_k"], p["grid"]) == (8, 128, 216)
    # d = 64, 544 blocks of 128 rows: three per CU in one round (as at d = 128)
    p = fa.fa_fwd_plan(2, 8, 4300, 64, fa.FA_BF16)
    assert (p["waves"], p["block_k"], p["grid"]) == (4, 64, 544)


@pytest.mark.parametrize("B,H,N,d,plan", [
    # (waves, Bc): the measured best plan of each grid (interleaved timings on one MI355X)
    (4, 32, 16384, 128, (8, 128)),   # 32 full rounds of 256-row blocks
    (3, 8, 4097, 128, (8, 128)),     # 408 blocks of 256: 218 us; 4 waves 233-238 us
    (2, 8, 2049, 128, (8, 128)),     # 144 blocks of 256: 58 us; 4 waves 62-63 us
    (2, 8, 4000, 128, (8, 128)),     # 256 blocks of 256: 125 us; 4 waves 133-134 us
    # last rows first, then 256 (512) full blocks of 256 rows: 139 us against 151 us for three
    # 4-wave workgroups per CU with the last block's key split (265 against 293 us; 139 against
    # 150 us; d = 64 163 against 183 us)
    (2, 8, 4097, 128, (8, 128)),
    (4, 8, 4097, 128, (8, 128)),
    (1, 16, 4097, 128, (8, 128)),
    (2, 16, 4097, 64, (8, 128)),
    (2, 8, 4129, 128, (8, 128)),     # 33 last rows first: 139 us; 4 waves at three per CU 172 us
    (2, 8, 4160, 128, (8, 128)),     # 64 last rows first: 142 us; 172 us
    (2, 8, 4300, 128, (4, 32)),      # 204 last rows: 544 blocks of 128 at three per CU
    (8, 8, 4097, 128, (8, 128)),     # last rows first: 505 us; 4 waves 527 us, 8 waves with short blocks 527 us
    (2, 8, 16385, 128, (8, 128)),    # last rows first: 1.88 ms; 2.05 and 2.07 ms
    (16, 64, 2049, 128, (4, 32)),    # 1024 heads: 2.13 ms; 8 waves 2.27 ms, last rows first 2.33 ms
    (8, 16, 2049, 128, (4, 32)),     # 273 us; last rows first 285 us, 8 waves 290 us
    (16, 16, 2049, 128, (4, 32)),    # 523 us; 8 waves (last rows first) 546 us
    (2, 32, 4097, 128, (8, 128)),    # last rows first: 496 us; 4 waves at three per CU 522 us
    (4, 32, 4097, 128, (4, 32)),     # 993 us; 8 waves (last rows first) 1002 us
    (1, 32, 8193, 128, (8, 128)),    # last rows first: 940 us; 1028 us
    (1, 8, 4096, 128, (4, 64)),      # 256 blocks of 128, one per CU: 80 us; 8 waves 100 us
    (4, 16, 2048, 64, (8, 128)),     # 512 blocks of 256 (ping-pong): 84 us; 4 waves 86-87 us
])
def test_plan_cost_model_picks_the_measured_best_plan(lib, B, H, N, d, plan):
    p = fa.fa_fwd_plan(B, H, N, d, fa.FA_BF16)
    assert (p["waves"], p["block_k"]) == plan


def test_plan_validates_like_fwd(lib):
    plan = fa.Plan()
    assert lib.fa_fwd_plan(1, 1, 10, 80, fa.FA_BF16, 0, ctypes.byref(plan)) == 3
    assert lib.fa_fwd_plan(1, -1, 10, 64, fa.FA_BF16, 0, ctypes.byref(plan)) == 2
    assert lib.fa_fwd_plan(1, 1, 10, 64, fa.FA_BF16, 0, None) == 1
    assert lib.fa_fwd_plan(0, 1, 10, 64, fa.FA_BF16, 0, ctypes.byref(plan)) == 0
    assert plan.grid == 0


def test_binding_refuses_host_tensors(lib):
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)


def test_library_has_no_torch_dependency():
    import subprocess

    out = subprocess.run(["ldd", fa.LIB_PATH], capture_output=True, text=True).stdout
    names = [line.split()[0] for line in out.splitlines() if line.strip()]   # not the load addresses
    assert names and not any("torch" in n or n.startswith("libc10") for n in names), names


def _skv(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=WS, ws_bytes=1 << 40, B=1, H=1, N=4096, d=128,
         scale=0.125, dtype=fa.FA_BF16, splits=4):
    return lib.fa_fwd_splitkv(q, k, v, o, lse, ws, ws_bytes, B, H, N, d, scale, dtype, splits, None)


def test_splitkv_workspace_and_split_choice(lib):
    # partial O (fp32, d per row) and partial LSE per split, each rounded up to 256 bytes
    rows = 2 * 3 * 1000
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 3, 1000, 64, fa.FA_BF16, 4) == \
        -(-4 * rows * 64 * 4 // 256) * 256 + -(-4 * rows * 4 // 256) * 256
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 3, 1000, 64, fa.FA_BF16, 1) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 3, 1000, 64, fa.FA_F32, 4) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 3, 1000, 64, fa.FA_BF16, 65) == 0
    # more splits than key tiles are clamped to the tiles (300 keys / 64 = 5 tiles at d=128)
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 1, 300, 128, fa.FA_BF16, 64) == \
        lib.fa_fwd_splitkv_workspace_bytes(1, 1, 300, 128, fa.FA_BF16, 5)
    # the chooser: a small grid is split, a full one is not; every split keeps >= 2 tiles
    assert lib.fa_fwd_splitkv_splits(1, 1, 16384, 128, fa.FA_BF16) > 1
    assert lib.fa_fwd_splitkv_splits(4, 32, 16384, 128, fa.FA_BF16) == 1
    for N in (128, 256, 1000, 4097, 16384):
        s = lib.fa_fwd_splitkv_splits(1, 1, N, 128, fa.FA_BF16)
        assert 1 <= s <= 64 and (s == 1 or -(-N // 64) >= 2 * s)
    # a full grid is split only when its last round of workgroups is nearly empty:
    # B=2 H=8 N=4097 d=128 has 528 blocks of 128 rows on 512 slots
    assert lib.fa_fwd_splitkv_splits(2, 8, 4097, 128, fa.FA_BF16) == 3
    assert lib.fa_fwd_splitkv_splits(4, 16, 2048, 64, fa.FA_BF16) == 1      # two full rounds
    assert lib.fa_fwd_splitkv_splits(2, 16, 8192, 128, fa.FA_BF16) == 1     # 1024 blocks
    assert lib.fa_fwd_splitkv_splits(8, 32, 4097, 128, fa.FA_BF16) == 1     # many rounds


def test_splitkv_validation(lib):
    assert _skv(lib, dtype=fa.FA_F32) == 3
    assert _skv(lib, d=80) == 3
    assert _skv(lib, splits=-1) == 2
    assert _skv(lib, splits=65) == 2
    assert _skv(lib, N=0, q=None, ws=None) == 0
    assert _skv(lib, q=None) == 1
    assert _skv(lib, o=FAKE + 8) == 4
    assert _skv(lib, scale=0.0) == 5
    assert _skv(lib, ws=None) == 8
    assert _skv(lib, ws=WS + 64) == 8
    assert _skv(lib, ws_bytes=16) == 8


def test_splitkv_valid_call_without_gpu_stops_at_device_check(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the device check passes")
    assert _skv(lib) == 6
    assert _skv(lib, splits=1, ws=None) == 6   # one split is fa_fwd: no workspace needed


def _q8(lib, x=FAKE, x8=FAKE, sc=FAKE, B=1, H=2, N=100, d=128, dtype=fa.FA_BF16, transpose=0):
    return lib.fa_quantize_fp8(x, x8, sc, B, H, N, d, dtype, transpose, None)


def _f8(lib, q=FAKE, k=FAKE, v=FAKE, qs=FAKE, ks=FAKE, vs=FAKE, o=FAKE, lse=FAKE, B=1, H=2, N=100, d=128,
        scale=0.125, dtype=fa.FA_BF16, causal=False):
    fn = lib.fa_fwd_fp8_causal if causal else lib.fa_fwd_fp8
    return fn(q, k, v, qs, ks, vs, o, lse, B, H, N, d, scale, dtype, None)


def test_fp8_sizes(lib):
    assert lib.fa_fp8_padded_len(1) == 128 and lib.fa_fp8_padded_len(128) == 128
    assert lib.fa_fp8_padded_len(129) == 256 and lib.fa_fp8_padded_len(0) == 0
    assert lib.fa_fp8_padded_len(-3) == 0
    assert lib.fa_fp8_scale_blocks(1) == 1 and lib.fa_fp8_scale_blocks(64) == 1
    assert lib.fa_fp8_scale_blocks(65) == 2 and lib.fa_fp8_scale_blocks(16384) == 256
    assert lib.fa_fp8_scale_blocks(0) == 0


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_validation_order_and_codes(lib, causal):
    f8 = functools.partial(_f8, causal=causal)
    assert _q8(lib, N=-1) == 2
    assert _q8(lib, d=96) == 3
    assert _q8(lib, dtype=fa.FA_F32) == 3
    assert _q8(lib, transpose=2) == 3
    assert _q8(lib, x=None, N=0) == 0
    assert _q8(lib, x8=None) == 1
    assert _q8(lib, sc=FAKE + 2) == 4
    assert _q8(lib, x8=FAKE + 8) == 4
    assert f8(lib, B=-1) == 2
    assert f8(lib, dtype=fa.FA_F32) == 3
    assert f8(lib, d=32) == 3
    assert f8(lib, q=None, N=0) == 0
    assert f8(lib, vs=None) == 1
    assert f8(lib, v=FAKE + 4) == 4
    assert f8(lib, ks=FAKE + 1) == 4
    assert f8(lib, scale=-1.0) == 5
    # the padded V^T head must fit 32-bit byte offsets
    assert f8(lib, N=(1 << 24) - 1, d=128) == 2


def test_fp8_valid_calls_without_gpu_stop_at_device_check(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the device check passes")
    assert _q8(lib) == 6
    assert _q8(lib, transpose=1) == 6
    assert _f8(lib) == 6
    assert _f8(lib, causal=True) == 6


def _skv_qk(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=WS, ws_bytes=1 << 40, B=2, H=4, Nq=1, Nk=5000,
            d=128, scale=0.125, dtype=fa.FA_BF16, splits=0):
    return lib.fa_fwd_splitkv_qk(q, k, v, o, lse, ws, ws_bytes, B, H, Nq, Nk, d, scale, dtype, splits, None)


def test_splitkv_qk_sizes_and_validation(lib):
    # the square case is the same call
    assert lib.fa_fwd_splitkv_qk_workspace_bytes(2, 3, 1000, 1000, 64, fa.FA_BF16, 4) == \
        lib.fa_fwd_splitkv_workspace_bytes(2, 3, 1000, 64, fa.FA_BF16, 4)
    assert lib.fa_fwd_splitkv_qk_splits(1, 1, 16384, 16384, 128, fa.FA_BF16) == \
        lib.fa_fwd_splitkv_splits(1, 1, 16384, 128, fa.FA_BF16)
    # decode: rows are Nq's, splits follow Nk's key tiles (5000 keys / 64 = 79 tiles)
    s = lib.fa_fwd_splitkv_qk_splits(2, 4, 1, 5000, 128, fa.FA_BF16)
    assert 2 <= s <= 39
    rows = 2 * 4 * 1
    assert lib.fa_fwd_splitkv_qk_workspace_bytes(2, 4, 1, 5000, 128, fa.FA_BF16, 8) == \
        -(-8 * rows * 128 * 4 // 256) * 256 + -(-8 * rows * 4 // 256) * 256
    assert lib.fa_fwd_splitkv_qk_workspace_bytes(2, 4, 1, 100, 128, fa.FA_BF16, 64) == \
        lib.fa_fwd_splitkv_qk_workspace_bytes(2, 4, 1, 100, 128, fa.FA_BF16, 2)   # 2 key tiles
    assert _skv_qk(lib, Nk=0) == 2            # queries with no keys
    assert _skv_qk(lib, Nq=0, Nk=0, q=None) == 0
    assert _skv_qk(lib, Nq=-1) == 2
    assert _skv_qk(lib, Nk=-5) == 2
    assert _skv_qk(lib, dtype=fa.FA_F32) == 3
    assert _skv_qk(lib, k=None) == 1
    assert _skv_qk(lib, ws=None, splits=8) == 8


def test_splitkv_qk_without_gpu_stops_at_device_check(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the device check passes")
    assert _skv_qk(lib, splits=8) == 6


def test_grids_beyond_32_bits_are_shape_errors(lib):
    # B*H*ceil(N/128) fits the index math, but a launch would need 2^31 workgroups or more
    B, H, N = 1 << 16, 1 << 8, 8192
    assert lib.fa_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, B, H, N, 64, 0.125, fa.FA_F32, None) == 2   # 32-row blocks
    plan = fa.Plan()
    assert lib.fa_fwd_plan(B, H, N, 64, fa.FA_F32, 0, ctypes.byref(plan)) == 2
    assert _skv(lib, B=B, H=H, N=N, d=64, splits=2) == 2
    assert _q8(lib, B=B, H=H, N=N, d=64) == 2
    assert _q8(lib, B=B, H=H, N=N, d=64, transpose=1) == 2


def test_heads_beyond_32_bit_byte_offsets_are_shape_errors(lib):
    # one head of 2^23 rows x 128 dims is 2 GiB of bf16: past the kernels' 32-bit offsets
    assert lib.fa_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1 << 23, 128, 0.125, fa.FA_BF16, None) == 2
    plan = fa.Plan()
    assert lib.fa_fwd_plan(1, 1, (1 << 23) - 1, 128, fa.FA_BF16, 0, ctypes.byref(plan)) == 0


def test_plan_reports_the_ping_pong_third_stage(lib):
    # non-causal d = 64 on 8 waves runs the ping-pong schedule: three 32 KiB K/V stages
    p = fa.fa_fwd_plan(4, 16, 2048, 64, fa.FA_BF16)
    assert (p["waves"], p["block_k"], p["lds_bytes"]) == (8, 128, 3 * 2 * 128 * 64 * 2)
    # the causal d = 64 plan on 8 waves and the d = 128 one keep two stages
    p = fa.fa_fwd_plan(4, 16, 2048, 64, fa.FA_BF16, causal=True)
    assert (p["waves"], p["lds_bytes"]) == (8, 2 * 2 * 128 * 64 * 2)
    p = fa.fa_fwd_plan(4, 32, 16384, 128, fa.FA_BF16)
    assert (p["waves"], p["lds_bytes"]) == (8, 2 * 2 * 128 * 128 * 2)


def _noalloc(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, H=4, Nq=1, Nk=5000, d=128, scale=0.125,
             dtype=fa.FA_BF16, splits=0):
    return lib.fa_fwd_splitkv_qk_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits, None)


def test_noalloc_validates_like_splitkv_qk(lib):
    assert lib.fa_status_str(9).decode().startswith("FA_ERR_SCRATCH")
    assert _noalloc(lib, Nk=0) == 2
    assert _noalloc(lib, Nq=-1) == 2
    assert _noalloc(lib, splits=65) == 2
    assert _noalloc(lib, d=96) == 3
    assert _noalloc(lib, dtype=fa.FA_F32) == 3
    assert _noalloc(lib, Nq=0, Nk=0, q=None) == 0
    assert _noalloc(lib, v=None) == 1
    assert _noalloc(lib, o=FAKE + 8) == 4
    assert _noalloc(lib, lse=FAKE + 2) == 4
    assert _noalloc(lib, scale=float("nan")) == 5


def test_noalloc_rejects_partials_beyond_the_static_scratch(lib):
    limit = fa.NOALLOC_SCRATCH_BYTES
    assert limit == 32 << 20
    # 8 splits of 8192 rows x 128 dims of fp32 partials: 32 MiB + the LSE partials > limit
    B, H, Nq, Nk, d, s = 1, 8, 1024, 8192, 128, 8
    need = lib.fa_fwd_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, fa.FA_BF16, s)
    assert need > limit
    assert _noalloc(lib, B=B, H=H, Nq=Nq, Nk=Nk, d=d, splits=s) == 9
    # the same rows in 7 splits fit
    assert lib.fa_fwd_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, fa.FA_BF16, 7) <= limit
    # the size check precedes the device check, so it holds without a GPU as well


def test_noalloc_valid_calls_without_gpu_stop_at_device_check(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the device check passes")
    assert _noalloc(lib) == 6                       # decode shape, several splits
    assert _noalloc(lib, B=1, H=8, Nq=1024, Nk=8192, splits=7) == 6
    assert _noalloc(lib, splits=1) == 6             # one split: the plain forward, no scratch


@pytest.fixture
def tile_env(monkeypatch):
    """Sets FA_TILE for one test (the library reads it on every call)."""
    def set_tile(value):
        monkeypatch.setenv("FA_TILE", value)
    yield set_tile
    monkeypatch.delenv("FA_TILE", raising=False)


def test_tile_override_replaces_the_plan(lib, tile_env):
    base = fa.fa_fwd_plan(4, 32, 16384, 128, fa.FA_BF16)
    assert (base["block_q"], base["block_k"], base["waves"]) == (256, 128, 8)
    tile_env("128,64,4")
    p = fa.fa_fwd_plan(4, 32, 16384, 128, fa.FA_BF16)
    assert (p["block_q"], p["block_k"], p["waves"], p["grid"], p["lds_bytes"]) == (128, 64, 4, 128 * 128, 65536)
    tile_env("128,32,4")
    assert fa.fa_fwd_plan(2, 8, 4097, 128, fa.FA_F16, causal=True)["block_k"] == 32
    tile_env("256,128,8")     # d = 64, non-causal: the ping-pong kernel with its third stage
    p = fa.fa_fwd_plan(1, 2, 300, 64, fa.FA_BF16)
    assert (p["block_q"], p["waves"], p["grid"], p["lds_bytes"]) == (256, 8, 4, 3 * 2 * 128 * 64 * 2)
    tile_env("32,32,4")
    p = fa.fa_fwd_plan(1, 1, 256, 64, fa.FA_F32)
    assert (p["block_q"], p["wave_kv_splits"]) == (32, 4)
    tile_env("")              # empty: the chooser decides
    assert fa.fa_fwd_plan(4, 32, 16384, 128, fa.FA_BF16) == base


@pytest.mark.parametrize("tile,d,dtype", [
    ("128,96,4", 128, fa.FA_BF16),      # no 96-key kernel
    ("256,64,4", 128, fa.FA_BF16),      # Br must be 32 rows per wave
    ("128,128,4", 128, fa.FA_BF16),     # 4 waves x 128 keys is compiled for d = 64 only
    ("128,32,4", 64, fa.FA_F16),        # 32-key tiles are compiled for d = 128 only
    ("128,64,4", 64, fa.FA_F32),        # fp32 has one variant
    ("abc", 128, fa.FA_BF16), ("128,64", 128, fa.FA_BF16), ("128,64,4,1", 128, fa.FA_BF16),
    ("128, 64, 4", 128, fa.FA_BF16), ("-128,64,4", 128, fa.FA_BF16), ("99999999,64,4", 128, fa.FA_BF16),
])
def test_tile_override_must_name_a_compiled_kernel(lib, tile_env, tile, d, dtype):
    tile_env(tile)
    plan = fa.Plan()
    assert lib.fa_fwd_plan(2, 4, 1000, d, dtype, 0, ctypes.byref(plan)) == 10
    assert _fwd(lib, B=2, H=4, N=1000, d=d, dtype=dtype) == 10      # before the device check
    assert _fwd(lib, B=2, H=4, N=1000, d=d, dtype=dtype, causal=True) == 10
    assert lib.fa_status_str(10).decode().startswith("FA_ERR_TILE")
    # calls that are not planned by the chooser ignore it
    assert _bwd(lib, d=d, dtype=fa.FA_BF16) in (0, 6)


def test_log_prints_the_plan_to_stderr(lib, monkeypatch, capfd):
    monkeypatch.setenv("FA_LOG", "1")
    _fwd(lib, B=4, H=32, N=16384, d=128)
    _skv(lib, splits=4)
    _bwd(lib)
    _f8(lib)
    monkeypatch.setenv("FA_TILE", "128,64,4")
    _fwd(lib, B=4, H=32, N=16384, d=128)
    monkeypatch.delenv("FA_TILE")
    # tail first (its partials go to O, so O must not overlap the inputs: distinct addresses)
    far = [ctypes.c_void_p(a << 32) for a in range(1, 6)]
    _fwd(lib, *far, B=2, H=8, N=4097, d=128)
    _fwd(lib, B=2, H=8, N=4097, d=128)   # O over Q: the 8-wave grid with its short blocks
    monkeypatch.setenv("FA_LOG", "0")
    _fwd(lib, B=1, H=1, N=77, d=64)
    err = capfd.readouterr().err
    assert "fa_fwd: B=4 H=32 N=16384 Nk=16384 d=128 bf16 -> Br=256 Bc=128 waves=8 grid=8192 lds=131072" in err
    assert "fa_fwd_splitkv: B=1 H=1 Nq=4096 Nk=4096 d=128 bf16 -> splits=4 of 64 key tiles" in err
    assert "the caller's workspace" in err
    assert "fa_bwd: B=1 H=2 N=64 d=64 bf16" in err
    assert "fa_fwd_fp8: B=1 H=2 N=100 d=128" in err
    assert "Br=128 Bc=64 waves=4 grid=16384 lds=65536 (FA_TILE)" in err
    assert ("fa_fwd: B=2 H=8 N=4097 Nk=4097 d=128 bf16 -> Br=256 Bc=128 waves=8 grid=256 lds=131072 "
            "(the last 1 rows first: 16 key ranges per head, merged)") in err
    assert "fa_fwd: B=2 H=8 N=4097 Nk=4097 d=128 bf16 -> Br=256 Bc=128 waves=8 grid=272 lds=131072\n" in err
    assert "N=77" not in err          # FA_LOG=0: silent


def test_huge_sizes_are_rejected_without_overflow(lib):
    # sizes near INT64_MAX: every check must reject them without forming an overflowing
    # product (the sanitized build of the library runs this file under UBSan)
    big = (1 << 63) - 1
    assert _fwd(lib, N=big, d=128) == 2
    assert _fwd(lib, N=1 << 60, d=64) == 2
    assert _fwd(lib, B=big, H=big) == 2
    assert _fwd(lib, B=1 << 40, H=1 << 40, N=1 << 40) == 2
    assert _bwd(lib, N=big, d=128) == 2
    assert lib.fa_bwd_workspace_bytes(big, big, big, 128, fa.FA_BF16) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 1, big, 128, fa.FA_BF16, 4) == 0
    assert lib.fa_fwd_splitkv_qk_workspace_bytes(1, 1, 1, big, 128, fa.FA_BF16, 0) == 0
    assert _skv_qk(lib, Nk=big) == 2
    assert lib.fa_fp8_padded_len(big) == 0 and lib.fa_fp8_padded_len(big - 127) == 0
    assert lib.fa_fp8_padded_len(big - 128) == big - 127   # (2^63 - 129) rounded up to 128
    assert lib.fa_fp8_scale_blocks(big) == big // 64 + 1
    assert _q8(lib, N=big) == 2
    assert _f8(lib, N=big) == 2
    plan = fa.Plan()
    assert lib.fa_fwd_plan(big, big, big, 128, fa.FA_BF16, 0, ctypes.byref(plan)) == 2


def test_header_builds_as_c_and_links(tmp_path):
    # A plain C11 caller: includes fa.h alone (it declares hipStream_t itself), links
    # libfa.so and calls the host-only entry points.
    import subprocess

    src = tmp_path / "caller.c"
    src.write_text(
        '#include "fa.h"\n#include <stdio.h>\n'
        "int main(void) {\n"
        "    fa_plan p;\n"
        "    hipStream_t s = 0;\n"
        "    (void)s;\n"
        "    if (fa_fwd_plan(4, 32, 16384, 128, FA_BF16, 0, &p) != FA_OK) return 1;\n"
        '    printf("%d %d %d %d\\n", fa_version() >= 100, p.block_q, p.block_k, p.waves);\n'
        "    return 0;\n}\n")
    exe = tmp_path / "caller"
    lib = os.path.join(os.path.dirname(os.path.abspath(fa.__file__)), "libfa.so")   # the in-tree build
    if not os.path.exists(lib):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    # the children run without the sanitizer runtime a parent run may preload
    env = {k: v for k, v in os.environ.items() if not k.startswith(("LD_PRELOAD", "ASAN_", "UBSAN_"))}
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    lib, f"-Wl,-rpath,{os.path.dirname(lib)}"], check=True, capture_output=True, text=True, env=env)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, env=env).stdout.split()
    assert out == ["1", "256", "128", "8"]


def test_header_typedef_agrees_with_hip():
    # C++ callers that include HIP's runtime header first see the same hipStream_t.
    import subprocess

    hip_inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(hip_inc, "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not installed")
    code = ('#include <hip/hip_runtime_api.h>\n#include "fa.h"\n'
            "static_assert(sizeof(hipStream_t) == sizeof(void*), \"handle\");\n"
            "int f(hipStream_t s) { return fa_fwd(0, 0, 0, 0, 0, 0, 0, 0, 64, 1.0f, FA_BF16, s); }\n")
    env = {k: v for k, v in os.environ.items() if not k.startswith(("LD_PRELOAD", "ASAN_", "UBSAN_"))}
    r = subprocess.run(["g++", "-std=c++17", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I", hip_inc,
                        "-I", os.path.join(ROOT, "include"), "-x", "c++", "-"], input=code, capture_output=True,
                       text=True, env=env)
    assert r.returncode == 0, r.stderr
