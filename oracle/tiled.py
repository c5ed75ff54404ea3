"""float64 NumPy models of the tiled online-softmax algorithm.

TEST INFRASTRUCTURE ONLY (see the package docstring).  These follow the steps
of the algorithm as the pages state them, so that the CPU tests can pin the
claim the whole library rests on: the tiled computation reaches the plain
attention result exactly (up to rounding order).  Nothing here is used to
produce an expected value for the GPU path; the GPU is always compared with
the plain-definition oracle in fa_oracle.c.

Sources (page title, then the section or item):
  * "04 Transformers, Attention, and FlashAttention": FlashAttention-2
    Algorithm 1 -- Q blocks outer, K/V blocks inner, running (O~, l, m),
    m_new = max(m_old, rowmax S), P~ = exp(S - m_new),
    l_new = e^(m_old - m_new) l_old + rowsum P~, O~ scaled by e^(m_old - m_new)
    plus P~ V_j, then one division by l and L = m + log l.  fa2_forward keeps
    these in base-2 units and starts the state from the first block instead of
    from the (0, 0, -inf) sentinels; both give the same numbers.
  * "大语言模型研究14", section 1.1 eqs. (4)-(7) and section 2: the scalar and
    row-block recurrences s_k = e^(m_{k-1} - m_k) s_{k-1} + b_k.
  * "FlashAttention: как реально считается attention на GPU", the online
    softmax formulas: correction = exp(m_old - m_new); a correction of 0 is
    used while the running maximum is still -inf.
  * "FlashAttention 深度解析", first article section 3.3: the FA1 form, in
    which exponentials are taken against the block maximum m~ and folded in
    with a second factor beta = exp(m~ - m_new), and O is kept normalised.
  * "FlashAttention 深度解析", second article section 2.3: causal attention
    visits only K/V blocks that start at or before the Q block's last row and
    masks keys after the query inside a block.
"""
from __future__ import annotations

import math

import numpy as np


def _correction(m_old: np.ndarray, m_new: np.ndarray) -> np.ndarray:
    """exp(m_old - m_new), taken as 0 where the old maximum is still -inf."""
    with np.errstate(invalid="ignore"):
        out = np.exp(m_old - m_new)
    return np.where(np.isneginf(m_old), 0.0, out)


def _block_scores(Qi, Kj, scale, causal, rows, cols):
    S = (Qi @ Kj.T) * scale
    if causal:
        S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
    return S


LOG2E = 1.0 / math.log(2.0)


def fa2_forward(Q, K, V, scale: float, Br: int, Bc: int, causal: bool = False):
    """FlashAttention-2 order for one head: Q (L, d), K (L, d), V (L, d) float64.

    The statistics are kept in base-2 units (t = S log2 e, so e^(S - m) is
    2^(t - m2)), and the first K/V block a Q block visits starts the state
    (m2, l, acc) outright; every later block folds in with the factor
    2^(m2_old - m2_new).  The first block always holds key 0, which every row
    sees (causal or not), so each row's state is finite from the start.

    Returns (O, lse, trace) where trace lists, per Q block, the per-row factor
    applied to the carried state at each K/V block (0 at the first block,
    where nothing is carried).
    """
    L, d = Q.shape
    O = np.empty((L, d))
    lse = np.empty(L)
    trace = []
    for r0 in range(0, L, Br):
        r1 = min(r0 + Br, L)
        rows = np.arange(r0, r1)
        Qi = Q[r0:r1]
        # causal: K/V blocks starting after the block's last row are skipped
        last = r1 - 1 if causal else L - 1
        factors = []
        for c0 in range(0, last + 1, Bc):
            c1 = min(c0 + Bc, L)
            T = _block_scores(Qi, K[c0:c1], scale, causal, rows, np.arange(c0, c1)) * LOG2E
            bmax = T.max(axis=1)
            if c0 == 0:
                assert np.all(np.isfinite(bmax)), "every row sees key 0"
                m2 = bmax
                P = np.exp2(T - m2[:, None])
                l = P.sum(axis=1)
                acc = P @ V[c0:c1]
                factors.append(np.zeros(r1 - r0))
                continue
            m2_new = np.maximum(m2, bmax)           # finite: m2 is
            a = np.exp2(m2 - m2_new)
            P = np.exp2(T - m2_new[:, None])        # masked scores give 0
            l = a * l + P.sum(axis=1)
            acc = a[:, None] * acc + P @ V[c0:c1]
            m2 = m2_new
            factors.append(a)
        O[r0:r1] = acc / l[:, None]
        lse[r0:r1] = (m2 + np.log2(l)) / LOG2E
        trace.append(factors)
    return O, lse, trace


def fa1_forward(Q, K, V, scale: float, Br: int, Bc: int, causal: bool = False):
    """FlashAttention-1 order for one head: K/V blocks outer, Q blocks inner.

    O, l, m live in full-length arrays ("HBM") between steps; exponentials are
    taken against the block maximum and folded in with alpha and beta; O is
    kept normalised after every step.
    """
    L, d = Q.shape
    Tr = math.ceil(L / Br)
    Tc = math.ceil(L / Bc)
    O = np.zeros((L, d))
    l = np.zeros(L)
    m = np.full(L, -np.inf)
    for j in range(Tc):
        c0, c1 = j * Bc, min((j + 1) * Bc, L)
        cols = np.arange(c0, c1)
        for i in range(Tr):
            r0, r1 = i * Br, min((i + 1) * Br, L)
            if causal and c0 > r1 - 1:
                continue
            rows = np.arange(r0, r1)
            S = _block_scores(Q[r0:r1], K[c0:c1], scale, causal, rows, cols)
            m_blk = S.max(axis=1)                       # block maximum m~
            live = ~np.isneginf(m_blk)                  # rows with a visible key here
            m_safe = np.where(live, m_blk, 0.0)
            P = np.where(live[:, None], np.exp(S - m_safe[:, None]), 0.0)
            l_blk = P.sum(axis=1)
            m_old, l_old, O_old = m[r0:r1], l[r0:r1], O[r0:r1]
            m_new = np.maximum(m_old, m_blk)
            alpha = _correction(m_old, m_new)
            beta = np.where(live, _correction(m_blk, m_new), 0.0)
            l_new = alpha * l_old + beta * l_blk
            with np.errstate(invalid="ignore", divide="ignore"):
                O_new = (alpha[:, None] * l_old[:, None] * O_old
                         + beta[:, None] * (P @ V[c0:c1])) / l_new[:, None]
            upd = l_new > 0
            O[r0:r1] = np.where(upd[:, None], O_new, O_old)
            l[r0:r1] = np.where(upd, l_new, l_old)
            m[r0:r1] = np.where(upd, m_new, m_old)
    return O, m + np.log(l)


def online_softmax_stats(scores, block: int):
    """Scalar online softmax over one score row, `block` scores at a time.

    Returns (m, l, corrections): the running maximum and running sum after the
    last block, and the correction factor exp(m_old - m_new) used at each block
    (0 at the first block, where the old maximum is -inf).
    """
    x = np.asarray(scores, dtype=np.float64)
    m, l = -np.inf, 0.0
    corrections = []
    for b0 in range(0, x.size, block):
        xb = x[b0:b0 + block]
        m_new = max(m, float(xb.max()))
        c = 0.0 if m == -np.inf else math.exp(m - m_new)
        l = c * l + float(np.exp(xb - m_new).sum())
        m = m_new
        corrections.append(c)
    return m, l, corrections
