"""Pins for the oracle's backward pass: finite differences, torch CPU autograd,
and identities of the softmax Jacobian."""

import numpy as np
import pytest

from oracle import attention_backward, attention_forward, backward_cols_dkdv, backward_rows_dq


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _loss(Q, K, V, dO, scale, causal):
    # L = sum(dO * O): its gradient w.r.t. O is dO.
    return float((attention_forward(Q, K, V, scale, causal=causal)[0] * dO).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 2), (3, 2), (6, 3)])
def test_central_finite_differences(N, d, causal):
    Q, K, V, dO = (_rand((N, d), [7, N, d, t]) for t in range(4))
    scale = 0.6
    dQ, dK, dV = attention_backward(Q, K, V, dO, scale, causal=causal)
    h = 1e-6
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            lp = _loss(Q, K, V, dO, scale, causal)
            X[idx] = old - h
            lm = _loss(Q, K, V, dO, scale, causal)
            X[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(G, num, atol=2e-8, rtol=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_autograd_fp64(causal):
    import torch

    B, H, N, d = 2, 2, 37, 16
    Q, K, V, dO = (_rand((B, H, N, d), [8, t]) for t in range(4))
    scale = 0.25
    dQ, dK, dV = attention_backward(Q, K, V, dO, scale, causal=causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (Q, K, V))
    S = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    if causal:
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    O = torch.matmul(torch.softmax(S, dim=-1), tv)
    O.backward(torch.from_numpy(dO))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-12)


def test_jacobian_identities():
    N, d = 40, 8
    Q, K, V, dO = _rand((N, d), 1, 2), _rand((N, d), 2, 2), _rand((N, d), 3), _rand((N, d), 4)
    dQ, dK, dV, aux = attention_backward(Q, K, V, dO, 0.3, return_all=True)
    # each row of dS sums to zero (softmax Jacobian annihilates constants)
    np.testing.assert_allclose(aux["dS"].sum(1), 0, atol=1e-13)
    # shifting every key by the same vector leaves the loss unchanged: sum_j dK_j = 0
    np.testing.assert_allclose(dK.sum(0), 0, atol=1e-12)
    # sum_j dV_j = sum_i dO_i (rows of P sum to one)
    np.testing.assert_allclose(dV.sum(0), dO.sum(0), atol=1e-12)
    # rowsum(dO * O) = rowsum(P * dP)
    np.testing.assert_allclose(aux["D"], (aux["P"] * aux["dP"]).sum(1), atol=1e-13)


def test_row_and_column_samplers_match_full_backward():
    N, d = 150, 8
    Q, K, V, dO = (_rand((N, d), [9, t]) for t in range(4))
    for causal in (False, True):
        dQ, dK, dV = attention_backward(Q, K, V, dO, 0.35, causal=causal)
        rows = np.array([0, 7, 63, 64, 149])
        np.testing.assert_allclose(backward_rows_dq(Q, K, V, dO, 0.35, rows, causal=causal),
                                   dQ[rows], atol=1e-13)
        cols = np.array([0, 1, 100, 149])
        ck, cv = backward_cols_dkdv(Q, K, V, dO, 0.35, cols, causal=causal, row_block=37)
        np.testing.assert_allclose(ck, dK[cols], atol=1e-13)
        np.testing.assert_allclose(cv, dV[cols], atol=1e-13)
