"""Seeded synthetic inputs for the attention forward/backward workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds only random-number generation, rounding of the drawn values
to the storage dtype, and the construction of the structured edge-case heads.  It
holds none of the attention arithmetic (no scores, softmax, or products with V).

Recipe (every tensor):
  * numpy ``default_rng(seed_words)`` draws fp64 N(0, 1) values,
  * they are rounded fp64 -> fp32 (numpy, round-to-nearest-even),
  * then fp32 -> storage dtype by round-to-nearest-even (bf16 by bit arithmetic,
    fp16 by numpy's cast).
The returned float64 arrays hold exactly the values the device sees, so the
oracle works on the same numbers.

Seed words are ``[config_id, tensor_id, b, h]`` so any single head can be
regenerated on its own (tensor ids: Q=1, K=2, V=3, dO=4, boost targets=5,
sampled rows=6).

The workloads follow the pages' problem statement (attention over tensors laid
out as [Batch, Heads, Seq_Len, Head_Dim], head dims 64/128, sequence lengths up
to 16K) -- see "FlashAttention 硬件感知计算剖析", section 五.1, and the 16K x 128
fp16 case of "从零理解Flash Attention中的online softmax", section 2.1.  The
pages benchmark on no public dataset for this path; dense attention cost does
not depend on values, so seeded N(0, 1) tensors stand in.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO, TENSOR_BOOST, TENSOR_ROWS = 1, 2, 3, 4, 5, 6

DTYPES = ("fp32", "fp16", "bf16")


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, dtype and how its inputs are drawn."""

    cid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    kind: str = "iid"  # "iid" or "edge" (the structured edge-case heads)
    backward: bool = False
    sampled: bool = False  # large: check sampled rows instead of the full output

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Forward FLOPs, 4*B*H*N^2*d (two N x N x d products, 2 FLOP per MAC)."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d


# The five workloads: a tiny fp32 head, a mid-size bf16 batch, the pages' 16K x 128
# fp16 case, structured edge cases at a ragged length, and the large bf16 case.
WORKLOADS = {
    1: Workload(1, "single_head_fp32", 1, 1, 256, 64, "fp32"),
    2: Workload(2, "batch_bf16_d64", 4, 16, 2048, 64, "bf16"),
    3: Workload(3, "long_fp16_d128", 1, 32, 16384, 128, "fp16", sampled=True),
    4: Workload(4, "edge_bf16_N4097", 2, 8, 4097, 128, "bf16", kind="edge"),
    5: Workload(5, "large_bf16_d128", 4, 32, 16384, 128, "bf16", backward=True, sampled=True),
}

BENCH_WORKLOAD = WORKLOADS[5]


# ---------------------------------------------------------------- rounding ---

def round_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> fp32 -> dtype (RNE both steps); returns the exact values as float64."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "fp32":
        return x32.astype(np.float64)
    if dtype == "fp16":
        return x32.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_float(round_to_bf16_bits(x32)).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_array(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exactly-representable float64 values -> the array to upload (bf16 as uint16 bits)."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x, dtype=np.float16)
    if dtype == "bf16":
        return round_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- drawing ---

def normal_head(seed_words, N: int, d: int, dtype: str, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(list(seed_words))
    x = rng.standard_normal((N, d))
    if sigma != 1.0:
        x = x * sigma
    return round_to_dtype(x, dtype)


def _head_iid(cid, tensor_id, b, h, N, d, dtype):
    return normal_head([cid, tensor_id, b, h], N, d, dtype)


def boosted_queries(q0: np.ndarray, k: np.ndarray, targets: np.ndarray, scale: float,
                    target_score: float, dtype: str) -> np.ndarray:
    """Query rows q_i = q0_i + c_i * k_{t(i)}, with c_i chosen so that scale * <q_i, k_t> hits
    ``target_score`` before rounding; then rounded to ``dtype``.  This builds the one-hot
    inputs of the edge-case workload; it is input construction, not attention."""
    kt = k[targets]                                   # [N, d]
    dots = np.einsum("nd,nd->n", q0, kt)
    norms = np.einsum("nd,nd->n", kt, kt)
    norms = np.where(norms > 0, norms, 1.0)
    c = (target_score - scale * dots) / (scale * norms)
    return round_to_dtype(q0 + c[:, None] * kt, dtype)


def edge_category(b: int, h: int, H: int) -> int:
    """0: all-zero Q; 1: Q and K scaled x10; 2: one key per query boosted to score +100."""
    return (b * H + h) % 3


def make_head(w: Workload, b: int, h: int, with_do: bool = False):
    """Inputs of one head as float64 arrays of exactly representable values.

    Returns (q, k, v) or (q, k, v, do) and, for edge heads of category 2, the boost
    targets are recoverable with :func:`boost_targets`.
    """
    N, d, dt = w.N, w.d, w.dtype
    if w.kind == "iid":
        q = _head_iid(w.cid, TENSOR_Q, b, h, N, d, dt)
        k = _head_iid(w.cid, TENSOR_K, b, h, N, d, dt)
    elif w.kind == "edge":
        cat = edge_category(b, h, w.H)
        if cat == 0:
            q = np.zeros((N, d))
            k = _head_iid(w.cid, TENSOR_K, b, h, N, d, dt)
        elif cat == 1:
            q = normal_head([w.cid, TENSOR_Q, b, h], N, d, dt, sigma=10.0)
            k = normal_head([w.cid, TENSOR_K, b, h], N, d, dt, sigma=10.0)
        else:
            q0 = _head_iid(w.cid, TENSOR_Q, b, h, N, d, dt)
            k = _head_iid(w.cid, TENSOR_K, b, h, N, d, dt)
            q = boosted_queries(q0, k, boost_targets(w, b, h), w.scale, 100.0, dt)
    else:
        raise ValueError(w.kind)
    v = _head_iid(w.cid, TENSOR_V, b, h, N, d, dt)
    if with_do:
        do = _head_iid(w.cid, TENSOR_DO, b, h, N, d, dt)
        return q, k, v, do
    return q, k, v


def boost_targets(w: Workload, b: int, h: int) -> np.ndarray:
    rng = np.random.default_rng([w.cid, TENSOR_BOOST, b, h])
    return rng.integers(0, w.N, size=w.N)


def make_inputs(w: Workload, with_do: bool = False, threads: int = 8):
    """All heads: float64 arrays [B, H, N, d] (exact values of the storage dtype)."""
    B, H, N, d = w.B, w.H, w.N, w.d
    nt = 4 if with_do else 3
    out = [np.empty((B, H, N, d), dtype=np.float64) for _ in range(nt)]

    def fill(bh):
        b, h = divmod(bh, H)
        t = make_head(w, b, h, with_do=with_do)
        for i in range(nt):
            out[i][b, h] = t[i]

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, range(B * H)))
    return tuple(out)


def sampled_rows(w: Workload, b: int, h: int, count: int = 64) -> np.ndarray:
    """Rows checked on the large workloads: fixed tile-boundary rows plus seeded random ones."""
    N = w.N
    fixed = [r for r in (0, 63, 64, 127, 128, 255, 256, N - 1) if 0 <= r < N]
    rng = np.random.default_rng([w.cid, TENSOR_ROWS, b, h])
    extra = rng.choice(N, size=min(N, count), replace=False)
    rows = list(dict.fromkeys(fixed + [int(r) for r in extra]))
    return np.array(sorted(rows[:count]), dtype=np.int64)


def random_tensor(shape, dtype: str, seed, sigma: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, sigma^2) tensor rounded to ``dtype`` (for ad-hoc test shapes)."""
    rng = np.random.default_rng(list(seed) if isinstance(seed, (list, tuple)) else seed)
    return round_to_dtype(rng.standard_normal(shape) * sigma, dtype)
