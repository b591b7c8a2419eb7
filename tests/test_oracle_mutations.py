"""The pins are strong enough: plant plausible mistakes in a copy of the oracle (on the
CPU, in memory) and check that at least one pin rejects each mutant.

Each mutant is the oracle's source with one textual change -- a dropped term, a wrong
sign or index, a transposed operand, an off-by-one mask -- executed as a fresh module.
"""

import inspect
import math
import types

import numpy as np
import pytest

import oracle.attention as oracle_src

from test_oracle_forward import brute_force


def _mutant(old, new):
    src = inspect.getsource(oracle_src)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _rand(shape, seed, sigma=1.5):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _pins_forward(m):
    """Brute force (causal and not) plus the two-block merge at every split."""
    for causal in (False, True):
        for (N, d) in ((5, 3), (6, 6)):
            Q, K, V = (_rand((N, d), [N, d, t]) for t in range(3))
            O, L = m.attention_forward(Q, K, V, 0.45, causal=causal)
            Ob, Lb = brute_force(Q.tolist(), K.tolist(), V.tolist(), 0.45, causal=causal)
            np.testing.assert_allclose(O, Ob, atol=1e-12)
            np.testing.assert_allclose(L, Lb, atol=1e-12)
            Os, Ls = m.blockwise_forward(Q, K, V, 0.45, 2, 4, causal=causal)
            np.testing.assert_allclose(Os, Ob, atol=1e-12)
            np.testing.assert_allclose(Ls, Lb, atol=1e-12)
    from scipy.special import logsumexp, softmax

    S, V = _rand((4, 9), 1, 4), _rand((9, 3), 2)
    for split in range(10):
        O, L = m.finalize_state(m.merge_states(m.block_state(S[:, :split], V[:split]),
                                               m.block_state(S[:, split:], V[split:])))
        np.testing.assert_allclose(O, softmax(S, 1) @ V, atol=1e-12)
        np.testing.assert_allclose(L, logsumexp(S, 1), atol=1e-12)
    parts = [m.attention_forward(_rand((3, 4), 5), _rand((4, 4), 6), _rand((4, 2), 7), 0.5),
             m.attention_forward(_rand((3, 4), 5), _rand((5, 4), 8), _rand((5, 2), 9), 0.5)]
    Om, Lm = m.merge_lse_partials(parts)
    Of, Lf = brute_force(_rand((3, 4), 5).tolist(),
                         np.vstack([_rand((4, 4), 6), _rand((5, 4), 8)]).tolist(),
                         np.vstack([_rand((4, 2), 7), _rand((5, 2), 9)]).tolist(), 0.5)
    np.testing.assert_allclose(Om, Of, atol=1e-12)
    np.testing.assert_allclose(Lm, Lf, atol=1e-12)


def _pins_backward(m):
    import torch

    for causal in (False, True):
        N, d = 7, 4
        Q, K, V, dO = (_rand((N, d), [3, t]) for t in range(4))
        dQ, dK, dV = m.attention_backward(Q, K, V, dO, 0.4, causal=causal)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (Q, K, V))
        S = 0.4 * tq @ tk.T.contiguous()
        if causal:
            S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        (torch.softmax(S, -1) @ tv).backward(torch.from_numpy(dO))
        np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-12)
        rows = np.array([0, 3, 6])
        np.testing.assert_allclose(m.backward_rows_dq(Q, K, V, dO, 0.4, rows, causal=causal),
                                   tq.grad.numpy()[rows], atol=1e-12)
        ck, cv = m.backward_cols_dkdv(Q, K, V, dO, 0.4, rows, causal=causal, row_block=3)
        np.testing.assert_allclose(ck, tk.grad.numpy()[rows], atol=1e-12)
        np.testing.assert_allclose(cv, tv.grad.numpy()[rows], atol=1e-12)


FORWARD_MUTANTS = [
    ("S = scale * (Q @ np.swapaxes(K, -1, -2))", "S = (Q @ np.swapaxes(K, -1, -2))"),  # no scale
    ("O = P @ V\n", "O = P @ np.swapaxes(V, -1, -2)\n"),                              # transposed V
    ("LSE = (m_shift + np.log(l))[..., 0]", "LSE = np.log(l)[..., 0]"),              # dropped m
    ("P = E / l\n", "P = E\n"),                                                     # no normalise
    ("return np.arange(nk)[None, :] <= rows[:, None]",
     "return np.arange(nk)[None, :] < rows[:, None] + 0"),                          # mask off by one
    ("alpha = np.where(np.isfinite(mA), np.exp(np.where(np.isfinite(mA), mA, 0.0) - m_shift), 0.0)",
     "alpha = np.where(np.isfinite(mA), np.exp(m_shift - np.where(np.isfinite(mA), mA, 0.0)), 0.0)"),
    ("return m, alpha * lA + beta * lB,", "return m, alpha * lA + lB,"),            # dropped rescale
    ("beta[:, None] * OB", "alpha[:, None] * OB"),                                  # wrong index
    ("return O / l[:, None], m + np.log(l)", "return O, m + np.log(l)"),            # no final divide
    ("S = scale * (Q[i0:i1] @ K[j0:j1].T)", "S = scale * (Q[i0:i1] @ K[i0:i1].T)"),  # wrong block
    ("O = (w[:, :, None] * Os).sum(axis=0) / tot[:, None]", "O = Os.sum(axis=0)"),  # unweighted
]

BACKWARD_MUTANTS = [
    ("dS = P * (dP - D)\n", "dS = P * dP\n"),                                       # dropped D
    ("dV = np.swapaxes(P, -1, -2) @ dO", "dV = P @ dO"),                            # transposed P
    ("dK = scale * (np.swapaxes(dS, -1, -2) @ Q)", "dK = scale * (dS @ Q)"),
    ("dQ = scale * (dS @ K)\n", "dQ = dS @ K\n"),                                   # no scale
    ("D = (dO * O).sum(axis=-1, keepdims=True)", "D = (dO * V).sum(axis=-1, keepdims=True)"),
]


def test_unmutated_oracle_passes_the_pins():
    _pins_forward(oracle_src)
    _pins_backward(oracle_src)


@pytest.mark.parametrize("old,new", FORWARD_MUTANTS)
def test_forward_mutant_is_rejected(old, new):
    m = _mutant(old, new)
    with pytest.raises((AssertionError, ValueError)):
        _pins_forward(m)


@pytest.mark.parametrize("old,new", BACKWARD_MUTANTS)
def test_backward_mutant_is_rejected(old, new):
    m = _mutant(old, new)
    with pytest.raises((AssertionError, ValueError)):
        _pins_backward(m)
