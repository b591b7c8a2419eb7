"""CPU fp64 oracle for exact attention and its online-softmax decomposition.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP path and the HIP path never calls it.

Everything here is float64 numpy, written for a reader to check by eye against the
pages.  Page titles used in citations:

  [P1] "从零理解Flash Attention中的online softmax" (kwkr.cn)
  [P2] "FlashAttention 硬件感知计算剖析:从 GPU 显存墙到 Online Softmax 与分块计算实践"
       (bbs.huaweicloud.com)
  [P3] FlashAttention FA1/FA2 differences (hotelren.com)
  [P4] "从原理出发理解 Flash Attention Part2" (juzhiart.com)

Conventions: Q, K, V are [..., N, d] arrays (leading batch/head axes allowed);
``scale`` multiplies Q K^T; LSE is the natural-log log-sum-exp of each score row.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _causal_mask(nq: int, nk: int, q_rows=None) -> np.ndarray:
    """True where key j may be attended by query i, i.e. j <= i.  Queries and keys share
    positions; ``q_rows`` gives the query positions when only some rows are evaluated."""
    rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    return np.arange(nk)[None, :] <= rows[:, None]


# ------------------------------------------------------------------ forward ---

def attention_forward(Q, K, V, scale, causal=False, return_p=False):
    """Standard attention, three passes that materialise S and P.

    [P2] section 一.2 states the problem: S = Q K^T / sqrt(d), P = softmax(S), O = P V
    (here the caller passes ``scale``).  The softmax is the safe form of [P2] section 二
    (subtract the row max m before exp) and [P1] section 3.1 names the row statistics
    m = max and l = sum(exp(x - m)).  LSE = m + ln l is the saved statistic.

    Causal (masked) attention drops keys j > i, the lower-triangular mask of [P2]
    section 五.3.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    # pass 1: scores
    S = scale * (Q @ np.swapaxes(K, -1, -2))
    if causal:
        S = np.where(_causal_mask(S.shape[-2], S.shape[-1]), S, NEG_INF)
    # pass 2: safe softmax
    m = S.max(axis=-1, keepdims=True)
    m_shift = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S - m_shift)
    l = E.sum(axis=-1, keepdims=True)
    P = E / l
    # pass 3: weighted sum of V
    O = P @ V
    LSE = (m_shift + np.log(l))[..., 0]
    if return_p:
        return O, LSE, P
    return O, LSE


def attention_rows(Q, K, V, scale, rows, causal=False):
    """The same definition evaluated only for query rows ``rows`` of one head.

    Q, K, V are [N, d]; returns (O[rows], LSE[rows]).  Used to check large problems on
    sampled rows: each output row depends only on its own query row and all of K, V.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    rows = np.asarray(rows)
    S = scale * (Q[rows] @ K.T)
    if causal:
        S = np.where(_causal_mask(len(rows), K.shape[0], rows), S, NEG_INF)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=-1, keepdims=True)
    O = (E / l) @ V
    LSE = (m + np.log(l))[:, 0]
    return O, LSE


# ------------------------------------------------- online softmax building blocks ---

def block_state(S_block, V_block):
    """Statistics of one block of scores, as in [P2] section 二 (online softmax derivation):
    m_B = max(B), l_B = sum(exp(B - m_B)), and the unnormalised output
    O_B = sum_i exp(B_i - m_B) V_i.  Rows are independent (leading axis = query rows).

    An empty block (no columns) is the identity state (m = -inf, l = 0, O = 0).
    """
    S_block, V_block = _f64(S_block), _f64(V_block)
    nq, d = S_block.shape[0], V_block.shape[1]
    if S_block.shape[1] == 0:
        return initial_state(nq, d)
    m = S_block.max(axis=1)
    m_shift = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S_block - m_shift[:, None])
    return m, E.sum(axis=1), E @ V_block


def initial_state(nq, d):
    """The initialisation m = -inf, l = 0, O = 0 ([P1] section 3.1; [P4] section 2.3)."""
    return np.full(nq, NEG_INF), np.zeros(nq), np.zeros((nq, d))


def merge_states(a, b):
    """Merge two blocks' states ([P2] section 二, the two-block formulas):

        m_new = max(m_A, m_B)
        l_new = exp(m_A - m_new) l_A + exp(m_B - m_new) l_B
        O_new = exp(m_A - m_new) O_A + exp(m_B - m_new) O_B

    with O kept unnormalised (O_A = sum exp(A_i - m_A) V_i).  [P2] writes the merge with a
    normalised O_A multiplied back by l_A; that is the same quantity, and dividing by l once
    at the end (:func:`finalize_state`) is the deferred normalisation of [P3] section 2.1.2.
    A side whose m is -inf (an empty block) contributes a factor of exactly 0.
    """
    mA, lA, OA = a
    mB, lB, OB = b
    m = np.maximum(mA, mB)
    fin = np.isfinite(m)
    m_shift = np.where(fin, m, 0.0)
    alpha = np.where(np.isfinite(mA), np.exp(np.where(np.isfinite(mA), mA, 0.0) - m_shift), 0.0)
    beta = np.where(np.isfinite(mB), np.exp(np.where(np.isfinite(mB), mB, 0.0) - m_shift), 0.0)
    return m, alpha * lA + beta * lB, alpha[:, None] * OA + beta[:, None] * OB


def finalize_state(state):
    """O = diag(l)^-1 O_unnormalised and LSE = m + ln l (one division per row)."""
    m, l, O = state
    return O / l[:, None], m + np.log(l)


def merge_lse_partials(parts):
    """Combine G partial results (O_g normalised over its own key range, LSE_g) of the same
    query rows: LSE = ln sum_g exp(LSE_g), O = sum_g exp(LSE_g - LSE) O_g.  This is the
    two-block merge of [P2] section 二 generalised to G blocks and written in log form;
    a part over no keys has LSE_g = -inf and weight 0."""
    lses = np.stack([_f64(p[1]) for p in parts])          # [G, n]
    Os = np.stack([_f64(p[0]) for p in parts])            # [G, n, d]
    mx = lses.max(axis=0)
    mxs = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lses - mxs)
    tot = w.sum(axis=0)
    lse = mxs + np.log(tot)
    O = (w[:, :, None] * Os).sum(axis=0) / tot[:, None]
    return O, lse


# ------------------------------------------------------------- block simulator ---

def blockwise_forward(Q, K, V, scale, Br, Bc, order="q_outer", causal=False):
    """Tiled forward for one head, fp64, following the block algorithm the pages describe.

    order="kv_outer" is the FlashAttention-1 order ([P2] section 三; [P4] section 2.3): the
    outer loop walks K/V column blocks j, the inner loop walks Q row blocks i, and the
    per-row state (m, l, O) of every row block is carried between outer steps.
    order="q_outer" is the FlashAttention-2 interchange ([P2] section 四.2): the outer loop
    walks Q row blocks, each row block streams all K/V blocks and is finished once.
    Both keep O unnormalised and divide by l once at the end; the per-block update is
    :func:`merge_states` of the carried state with the new block's :func:`block_state`.
    Br and Bc need not divide N.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    N, d = Q.shape
    Nk = K.shape[0]
    row_blocks = [(i, min(i + Br, N)) for i in range(0, N, Br)]
    col_blocks = [(j, min(j + Bc, Nk)) for j in range(0, Nk, Bc)]

    def scores(i0, i1, j0, j1):
        S = scale * (Q[i0:i1] @ K[j0:j1].T)
        if causal:
            allowed = np.arange(j0, j1)[None, :] <= np.arange(i0, i1)[:, None]
            S = np.where(allowed, S, NEG_INF)
        return S

    states = {rb: initial_state(rb[1] - rb[0], d) for rb in row_blocks}
    if order == "kv_outer":
        for (j0, j1) in col_blocks:
            for (i0, i1) in row_blocks:
                blk = block_state(scores(i0, i1, j0, j1), V[j0:j1])
                states[(i0, i1)] = merge_states(states[(i0, i1)], blk)
    elif order == "q_outer":
        for (i0, i1) in row_blocks:
            for (j0, j1) in col_blocks:
                blk = block_state(scores(i0, i1, j0, j1), V[j0:j1])
                states[(i0, i1)] = merge_states(states[(i0, i1)], blk)
    else:
        raise ValueError(order)

    O = np.empty((N, d))
    LSE = np.empty(N)
    for (i0, i1) in row_blocks:
        O[i0:i1], LSE[i0:i1] = finalize_state(states[(i0, i1)])
    return O, LSE


def streaming_rows(S, V):
    """The per-row streaming recurrence of [P1] section 3.1, one key column at a time:
    m_new = max(m, x_j); l <- l exp(m - m_new) + exp(x_j - m_new);
    o <- o exp(m - m_new) + exp(x_j - m_new) v_j; m <- m_new.  Returns (O, LSE)."""
    S, V = _f64(S), _f64(V)
    n, nk = S.shape
    state = initial_state(n, V.shape[1])
    for j in range(nk):
        state = merge_states(state, block_state(S[:, j:j + 1], V[j:j + 1]))
    return finalize_state(state)


# ----------------------------------------------------------------- backward ---

def attention_backward(Q, K, V, dO, scale, causal=False, return_all=False):
    """Gradients of O = softmax(scale Q K^T) V, from the plain definition.

    [P4] section 2.4 derives them with the chain rule through O = P V, the row-wise
    softmax and S = Q K^T (the algorithm figures are missing from the extracted text);
    [P1] section 5.1 rebuilds P from the saved statistics.  With D_i = sum_k dO_ik O_ik
    (which equals sum_j P_ij dP_ij):

        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
        dQ = scale dS K,   dK = scale dS^T Q.
    """
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    O, LSE, P = attention_forward(Q, K, V, scale, causal=causal, return_p=True)
    dV = np.swapaxes(P, -1, -2) @ dO
    dP = dO @ np.swapaxes(V, -1, -2)
    D = (dO * O).sum(axis=-1, keepdims=True)
    dS = P * (dP - D)
    dQ = scale * (dS @ K)
    dK = scale * (np.swapaxes(dS, -1, -2) @ Q)
    if return_all:
        return dQ, dK, dV, dict(O=O, LSE=LSE, P=P, dP=dP, D=D[..., 0], dS=dS)
    return dQ, dK, dV


def backward_rows_dq(Q, K, V, dO, scale, rows, causal=False, return_all=False):
    """dQ for selected query rows of one head ([N, d] inputs); each dQ row needs only its own
    query row, dO row and all of K, V (same formulas as :func:`attention_backward`).
    With ``return_all`` also returns the rows' P, dS, O and D."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    rows = np.asarray(rows)
    S = scale * (Q[rows] @ K.T)
    if causal:
        S = np.where(_causal_mask(len(rows), K.shape[0], rows), S, NEG_INF)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    P = E / E.sum(axis=-1, keepdims=True)
    O = P @ V
    dP = dO[rows] @ V.T
    D = (dO[rows] * O).sum(axis=-1, keepdims=True)
    dS = P * (dP - D)
    if return_all:
        return scale * (dS @ K), dict(P=P, dS=dS, O=O, D=D[:, 0])
    return scale * (dS @ K)


def backward_cols_dkdv(Q, K, V, dO, scale, cols, causal=False, row_block=1024):
    """dK and dV for selected key columns of one head ([N, d] inputs).  Column j of dK/dV needs
    P[:, j] and dS[:, j] for every query row, so the full forward is rebuilt in row blocks
    (same formulas as :func:`attention_backward`)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    cols = np.asarray(cols)
    N, d = Q.shape
    dK = np.zeros((len(cols), d))
    dV = np.zeros((len(cols), d))
    for i0 in range(0, N, row_block):
        i1 = min(N, i0 + row_block)
        S = scale * (Q[i0:i1] @ K.T)
        if causal:
            S = np.where(np.arange(K.shape[0])[None, :] <= np.arange(i0, i1)[:, None], S, NEG_INF)
        m = S.max(axis=-1, keepdims=True)
        E = np.exp(S - m)
        P = E / E.sum(axis=-1, keepdims=True)
        O = P @ V
        D = (dO[i0:i1] * O).sum(axis=-1, keepdims=True)
        Pc = P[:, cols]                                  # [rows, c]
        dPc = dO[i0:i1] @ V[cols].T                      # [rows, c]
        dSc = Pc * (dPc - D)
        dV += Pc.T @ dO[i0:i1]
        dK += scale * (dSc.T @ Q[i0:i1])
    return dK, dV
