"""The seeded input generators: rounding, determinism, and the edge-case heads."""

import math

import numpy as np
import pytest

import workloads as wl
from oracle import attention_forward


def test_bf16_rounding_matches_torch_rne():
    import torch

    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    # include exact ties: values with the low 16 bits equal to 0x8000
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = wl.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_fp16_rounding_is_numpy_rne():
    x = np.random.default_rng(1).standard_normal(1000) * 3
    got = wl.round_to_dtype(x, "fp16")
    np.testing.assert_array_equal(got, x.astype(np.float32).astype(np.float16).astype(np.float64))


def test_per_head_seeding_is_deterministic_and_independent():
    w = wl.WORKLOADS[2]
    a = wl.make_head(w, 1, 3)
    b = wl.make_head(w, 1, 3)
    c = wl.make_head(w, 1, 4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])


def test_storage_array_roundtrip():
    import torch

    x = wl.random_tensor((3, 8), "bf16", [3])
    bits = wl.storage_array(x, "bf16")
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(t, x.astype(np.float32))


def test_edge_workload_categories():
    w = wl.WORKLOADS[4]
    cats = [wl.edge_category(b, h, w.H) for b in range(w.B) for h in range(w.H)]
    assert cats.count(0) == 6 and cats.count(1) == 5 and cats.count(2) == 5
    # zero-Q head
    q, k, v = wl.make_head(w, 0, 0)
    assert not q.any()
    # x10 head: scores reach +-100 and beyond
    q, k, v = wl.make_head(w, 0, 1)
    s = w.scale * (q[:64] @ k.T)
    assert np.abs(s).max() > 300
    # boosted head: every query's target scores ~ 100 after rounding, 50 above the rest
    q, k, v = wl.make_head(w, 0, 2)
    t = wl.boost_targets(w, 0, 2)
    rows = np.arange(0, w.N, 97)
    s = w.scale * (q[rows] @ k.T)
    st = s[np.arange(len(rows)), t[rows]]
    assert np.all(np.abs(st - 100) < 1.0)
    s[np.arange(len(rows)), t[rows]] = -np.inf
    assert np.all(st - s.max(1) > 40)


def test_sampled_rows_cover_tile_boundaries():
    w = wl.WORKLOADS[5]
    r = wl.sampled_rows(w, 0, 0)
    assert len(r) == 64 and len(set(r)) == 64
    for x in (0, 63, 64, 127, 128, 255, 256, w.N - 1):
        assert x in r


def test_flops_convention():
    w = wl.WORKLOADS[5]
    assert w.flops == 4 * 4 * 32 * 16384 ** 2 * 128
    assert abs(w.flops - 1.759e13) / 1.759e13 < 1e-3


def test_one_hot_head_oracle_selects_target_rows():
    # The oracle on a truncated boosted head: O_i is V_{j*(i)} to bf16-irrelevant precision.
    w = wl.WORKLOADS[4]
    q, k, v = wl.make_head(w, 0, 2)
    t = wl.boost_targets(w, 0, 2)
    rows = np.arange(0, 200)
    O, L = attention_forward(q[rows], k, v, w.scale)
    np.testing.assert_allclose(O, v[t[rows]], atol=1e-14)
    assert np.all(np.abs(L - 100) < 1.0)
