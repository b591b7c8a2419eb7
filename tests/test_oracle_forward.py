"""Pins for the oracle's forward pass, against things other than itself.

Each test names what fixes the expected value: brute force in pure Python, a closed
form, an independent library routine (scipy / torch CPU), or an invariant the pages
state (the two-block decomposition, the m=-inf/l=0/O=0 initialisation, rows of P
summing to one) or that the mathematics implies (symmetries).
"""

import math

import numpy as np
import pytest

from oracle import (
    attention_forward,
    attention_rows,
    block_state,
    blockwise_forward,
    finalize_state,
    initial_state,
    merge_lse_partials,
    merge_states,
    streaming_rows,
)
from workloads import random_tensor

pytestmark = []


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


# ------------------------------------------------------------ brute force ---

def brute_force(Q, K, V, scale, causal=False):
    """Pure-Python double loops with math.fsum: the definition, nothing vectorised."""
    N, d = len(Q), len(Q[0])
    Nk, dv = len(K), len(V[0])
    O = [[0.0] * dv for _ in range(N)]
    LSE = [0.0] * N
    for i in range(N):
        keys = [j for j in range(Nk) if (not causal or j <= i)]
        s = [scale * math.fsum(Q[i][t] * K[j][t] for t in range(d)) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        for c in range(dv):
            O[i][c] = math.fsum(e[a] * V[j][c] for a, j in enumerate(keys)) / l
        LSE[i] = m + math.log(l)
    return np.array(O), np.array(LSE)


@pytest.mark.parametrize("N,d", [(1, 1), (2, 2), (3, 4), (5, 3), (8, 4), (7, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_brute_force(N, d, causal):
    Q, K, V = (_rand((N, d), [N, d, t], 1.5) for t in range(3))
    scale = 1.0 / math.sqrt(d)
    O, L = attention_forward(Q, K, V, scale, causal=causal)
    Ob, Lb = brute_force(Q.tolist(), K.tolist(), V.tolist(), scale, causal=causal)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


def test_rectangular_value_dim_brute_force():
    # V may have a different width than Q/K; the definition does not care.
    Q, K = _rand((4, 3), 1), _rand((6, 3), 2)
    V = _rand((6, 5), 3)
    O, L = attention_forward(Q, K, V, 0.7)
    Ob, Lb = brute_force(Q.tolist(), K.tolist(), V.tolist(), 0.7)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(L, Lb, atol=1e-13)


# ------------------------------------------------------------ closed forms ---

@pytest.mark.parametrize("N", [1, 2, 17, 4097])
def test_zero_scores_give_column_mean_and_log_n(N):
    # All-zero scores: every key gets weight 1/N, O is the mean of V's rows, LSE = ln N.
    d = 8
    Q = np.zeros((min(N, 5), d))
    K, V = _rand((N, d), 1), _rand((N, d), 2)
    O, L = attention_forward(Q, K, V, 1 / math.sqrt(d))
    np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), O.shape), atol=1e-14)
    np.testing.assert_allclose(L, math.log(N), atol=1e-14)


def test_log_4097_value():
    # The edge-case workload's zero-Q heads must produce LSE = ln 4097 = 8.318010277547...
    O, L = attention_forward(np.zeros((1, 4)), _rand((4097, 4), 0), _rand((4097, 4), 1), 0.5)
    assert abs(L[0] - 8.318010277547) < 1e-11


def test_single_key():
    # N = 1: the only weight is 1, O = V_0, LSE = S_00.
    q, k, v = _rand((1, 6), 1), _rand((1, 6), 2), _rand((1, 6), 3)
    O, L = attention_forward(q, k, v, 0.3)
    np.testing.assert_array_equal(O, v)
    assert abs(L[0] - 0.3 * float(q[0] @ k[0])) < 1e-15


def test_two_keys_logistic():
    # N = 2: P_i0 = sigma(S_i0 - S_i1), the logistic function.
    Q, K, V = _rand((5, 4), 1, 3), _rand((2, 4), 2, 3), _rand((2, 4), 3)
    scale = 0.5
    O, L = attention_forward(Q, K, V, scale)
    for i in range(5):
        s0, s1 = scale * Q[i] @ K[0], scale * Q[i] @ K[1]
        p0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        np.testing.assert_allclose(O[i], p0 * V[0] + (1 - p0) * V[1], atol=1e-14)
        assert abs(L[i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-13


def test_one_hot_boost_selects_row_of_v():
    # One key per query scoring +100 while the others are O(10): O_i = V_{j*(i)} up to
    # e^{-50}-sized weights of the rest ([P1] section 10 asks for tests at value 100).
    rng = np.random.default_rng(7)
    N, d = 300, 128   # at d = 128 the non-boosted scores have sigma ~ 9
    K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    targets = rng.integers(0, N, N)
    scale = 1 / math.sqrt(d)
    Q = rng.standard_normal((N, d))
    kt = K[targets]
    c = (100.0 - scale * np.einsum("nd,nd->n", Q, kt)) / (scale * np.einsum("nd,nd->n", kt, kt))
    Q = Q + c[:, None] * kt
    O, L, P = attention_forward(Q, K, V, scale, return_p=True)
    assert np.all(P.argmax(1) == targets)
    np.testing.assert_allclose(O, V[targets], atol=1e-12)
    np.testing.assert_allclose(L, 100.0, atol=1e-12)


# ---------------------------------------------------------- library routines ---

def test_against_scipy_softmax_and_logsumexp():
    from scipy.special import logsumexp, softmax

    Q, K, V = _rand((2, 3, 40, 8), 1), _rand((2, 3, 50, 8), 2), _rand((2, 3, 50, 8), 3)
    scale = 0.35
    O, L, P = attention_forward(Q, K, V, scale, return_p=True)
    S = scale * np.einsum("bhid,bhjd->bhij", Q, K)
    np.testing.assert_allclose(P, softmax(S, axis=-1), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(L, logsumexp(S, axis=-1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(O, np.einsum("bhij,bhjd->bhid", softmax(S, axis=-1), V), atol=1e-13)


def test_against_torch_cpu_fp64():
    import torch

    Q, K, V = _rand((3, 33, 16), 4), _rand((3, 33, 16), 5), _rand((3, 33, 16), 6)
    scale = 0.25
    O, L = attention_forward(Q, K, V, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (Q, K, V))
    S = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    To = torch.matmul(torch.softmax(S, dim=-1), tv)
    np.testing.assert_allclose(O, To.numpy(), atol=1e-13)
    np.testing.assert_allclose(L, torch.logsumexp(S, dim=-1).numpy(), atol=1e-13)
    Tc = torch.matmul(torch.softmax(S.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1),
                                                  float("-inf")), dim=-1), tv)
    Oc, _ = attention_forward(Q, K, V, scale, causal=True)
    np.testing.assert_allclose(Oc, Tc.numpy(), atol=1e-13)


# ------------------------------------------------------- definitional invariants ---

def test_rows_of_p_sum_to_one():
    Q, K, V = _rand((64, 16), 1, 4), _rand((200, 16), 2, 4), _rand((200, 16), 3)
    _, _, P = attention_forward(Q, K, V, 0.25, return_p=True)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(1) - 1)) <= 200 * 2.0 ** -52


# -------------------------------------------------------- decomposition (pages) ---

def test_two_block_merge_equals_full_softmax_at_every_split():
    # [P2] section 二 / [P4] section 2.2: softmax of x split in two blocks, merged, equals
    # the softmax of the whole row -- at every split point, including empty sides.
    rng = np.random.default_rng(11)
    n, N, d = 6, 23, 5
    S, V = rng.standard_normal((n, N)) * 4, rng.standard_normal((N, d))
    from scipy.special import logsumexp, softmax

    ref_O = softmax(S, axis=1) @ V
    ref_L = logsumexp(S, axis=1)
    for split in range(0, N + 1):
        a = block_state(S[:, :split], V[:split])
        b = block_state(S[:, split:], V[split:])
        O, L = finalize_state(merge_states(a, b))
        np.testing.assert_allclose(O, ref_O, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(L, ref_L, rtol=1e-12, atol=1e-14)
        O2, L2 = finalize_state(merge_states(b, a))   # merge is symmetric
        np.testing.assert_allclose(O2, ref_O, rtol=1e-12, atol=1e-14)


def test_identity_state_merge_is_bit_exact():
    # [P4] section 2.3 / [P1] section 3.1: m=-inf, l=0, O=0 merged with a block
    # reproduces that block's own softmax exactly.
    rng = np.random.default_rng(12)
    S, V = rng.standard_normal((7, 9)) * 30, rng.standard_normal((9, 4))
    blk = block_state(S, V)
    got = merge_states(initial_state(7, 4), blk)
    for g, r in zip(got, blk):
        np.testing.assert_array_equal(g, r)


@pytest.mark.parametrize("order", ["kv_outer", "q_outer"])
@pytest.mark.parametrize("Br,Bc", [(1, 1), (3, 5), (16, 7), (64, 64), (100, 33)])
@pytest.mark.parametrize("causal", [False, True])
def test_block_simulator_equals_three_pass(order, Br, Bc, causal):
    # [P2] section 三 (FA1 loop order) and section 四.2 (FA2 interchange), with block sizes
    # that do not divide N: exact attention either way.
    N, d = 71, 8
    Q, K, V = _rand((N, d), 21, 2), _rand((N, d), 22, 2), _rand((N, d), 23)
    O, L = attention_forward(Q, K, V, 0.4, causal=causal)
    Ob, Lb = blockwise_forward(Q, K, V, 0.4, Br, Bc, order=order, causal=causal)
    np.testing.assert_allclose(Ob, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Lb, L, rtol=1e-12, atol=1e-13)


def test_two_loop_orders_agree():
    N, d = 50, 4
    Q, K, V = _rand((N, d), 31, 3), _rand((N, d), 32, 3), _rand((N, d), 33)
    a = blockwise_forward(Q, K, V, 0.5, 8, 6, order="kv_outer")
    b = blockwise_forward(Q, K, V, 0.5, 8, 6, order="q_outer")
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12, atol=1e-14)


def test_per_column_streaming_recurrence():
    # [P1] section 3.1's recurrence one key at a time, on scores up to |x| ~ 1000
    # ([P1] section 3.2 stresses that the exp(m - m_new) rescale keeps this stable).
    rng = np.random.default_rng(3)
    S, V = rng.standard_normal((5, 40)) * 400, rng.standard_normal((40, 3))
    O, L = streaming_rows(S, V)
    m = S.max(1, keepdims=True)
    E = np.exp(S - m)
    np.testing.assert_allclose(O, (E / E.sum(1, keepdims=True)) @ V, atol=1e-13)
    np.testing.assert_allclose(L, m[:, 0] + np.log(E.sum(1)), rtol=1e-14)
    assert np.all(np.isfinite(O))


@pytest.mark.parametrize("cuts", [[0, 10, 50], [17], [1, 2, 3, 49], [0, 0, 25, 50]])
def test_lse_partial_merge_equals_full(cuts):
    # G partial results over key ranges (the split-KV / context-parallel combine).
    N, d = 50, 6
    Q, K, V = _rand((9, d), 41, 2), _rand((N, d), 42, 2), _rand((N, d), 43)
    O, L = attention_forward(Q, K, V, 0.4)
    edges = [0] + sorted(cuts) + [N]
    parts = []
    for a, b in zip(edges[:-1], edges[1:]):
        if b > a:
            parts.append(attention_forward(Q, K[a:b], V[a:b], 0.4))
        else:
            parts.append((np.zeros((9, d)), np.full(9, -np.inf)))
    Om, Lm = merge_lse_partials(parts)
    np.testing.assert_allclose(Om, O, atol=1e-13)
    np.testing.assert_allclose(Lm, L, atol=1e-13)


# ---------------------------------------------------------------- symmetries ---

def test_joint_permutation_of_keys_and_values():
    Q, K, V = _rand((20, 8), 1), _rand((30, 8), 2), _rand((30, 8), 3)
    perm = np.random.default_rng(0).permutation(30)
    a = attention_forward(Q, K, V, 0.3)
    b = attention_forward(Q, K[perm], V[perm], 0.3)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


def test_query_permutation_permutes_outputs():
    Q, K, V = _rand((20, 8), 1), _rand((30, 8), 2), _rand((30, 8), 3)
    perm = np.random.default_rng(1).permutation(20)
    a = attention_forward(Q, K, V, 0.3)
    b = attention_forward(Q[perm], K, V, 0.3)
    np.testing.assert_allclose(b[0], a[0][perm], atol=1e-15)
    np.testing.assert_allclose(b[1], a[1][perm], atol=1e-15)


def test_key_shift_changes_only_lse():
    # K_j <- K_j + u adds scale <q_i, u> to every score of row i: O unchanged,
    # LSE_i shifts by exactly that amount.
    Q, K, V = _rand((12, 8), 1), _rand((30, 8), 2), _rand((30, 8), 3)
    u = _rand(8, 4)
    a = attention_forward(Q, K, V, 0.3)
    b = attention_forward(Q, K + u, V, 0.3)
    np.testing.assert_allclose(b[0], a[0], atol=1e-13)
    np.testing.assert_allclose(b[1], a[1] + 0.3 * Q @ u, atol=1e-13)


def test_value_affine_map():
    # V <- a V + 1 b^T gives O <- a O + 1 b^T because each row of P sums to one.
    Q, K, V = _rand((12, 8), 1), _rand((30, 8), 2), _rand((30, 5), 3)
    bvec = _rand(5, 9)
    a = attention_forward(Q, K, V, 0.3)
    b = attention_forward(Q, K, 2.5 * V + bvec, 0.3)
    np.testing.assert_allclose(b[0], 2.5 * a[0] + bvec, atol=1e-13)


# ------------------------------------------------------------- sampled rows ---

def test_sampled_rows_equal_full_rows():
    Q, K, V = _rand((300, 8), 1), _rand((300, 8), 2), _rand((300, 8), 3)
    rows = np.array([0, 5, 63, 64, 299])
    O, L = attention_forward(Q, K, V, 0.3)
    for causal in (False, True):
        O, L = attention_forward(Q, K, V, 0.3, causal=causal)
        Or, Lr = attention_rows(Q, K, V, 0.3, rows, causal=causal)
        np.testing.assert_allclose(Or, O[rows], atol=1e-14)
        np.testing.assert_allclose(Lr, L[rows], atol=1e-14)


def test_causal_row_is_prefix_attention():
    # Masked attention of row i equals unmasked attention over keys 0..i.
    Q, K, V = _rand((25, 6), 1), _rand((25, 6), 2), _rand((25, 6), 3)
    Oc, Lc = attention_forward(Q, K, V, 0.5, causal=True)
    for i in (0, 1, 12, 24):
        Oi, Li = attention_forward(Q[i:i + 1], K[:i + 1], V[:i + 1], 0.5)
        np.testing.assert_allclose(Oc[i], Oi[0], atol=1e-14)
        np.testing.assert_allclose(Lc[i], Li[0], atol=1e-14)


def test_bf16_inputs_exactly_representable():
    x = random_tensor((4, 33), "bf16", [1, 2])
    bits = x.astype(np.float32).view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
