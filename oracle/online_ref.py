"""Tile-by-tile online-softmax attention in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

This module exists to pin the *method*: the pages claim that computing
attention tile by tile with a running maximum and a running sum of
exponentials, rescaling earlier partial results whenever the maximum grows,
gives exactly (up to rounding order) the plain three-pass result.  The tests
run both forms below against the three-pass oracle on every small shape.

Two forms are written out, each following its page's description:

``deferred``  -- "FlashAttention dissected" (leren.llmnet.nl), section
    "Algorithmic core in pseudocode": the query-block loop is outside, the
    key/value-block loop inside; per block the running max becomes
    max(m, rowmax(S)), P = exp(S - m_new), l_new = exp(m - m_new) * l +
    rowsum(P), O = diag(exp(m - m_new)) O + P V; after the inner loop O is
    divided by l once.

``normalised`` -- "How Did I Write My First FlashAttention Kernel in CUDA?",
    pseudo-algorithm steps 1-5: key/value blocks outside, query blocks inside,
    the block's own max m~ and P~ = exp(S - m~) with row sums l~, then
    m_new = max(m, m~), l_new = exp(m - m_new) l + exp(m~ - m_new) l~ and
    O <- diag(l_new)^-1 (diag(l) exp(m - m_new) O + exp(m~ - m_new) P~ V), so
    O stays normalised after every step and m, l, O are carried per row
    between outer iterations.

Masked scores (causal: key j > query i) are -inf.  When a row has seen no
visible key yet, its running max is -inf; the shift then uses 0 instead of
-inf so that -inf - (-inf) never forms a NaN (the guard the GitHub README's
design list gives for fully masked rows).
"""
from __future__ import annotations

import numpy as np


def _scores(q_blk, k_blk, scale, rows, cols, causal):
    s = scale * (q_blk @ k_blk.T)
    if causal:
        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
    return s


def _safe(m):
    """Shift to subtract: the running max, or 0 where it is still -inf."""
    return np.where(np.isneginf(m), 0.0, m)


def deferred(q, k, v, scale, causal=False, br=None, bc=None):
    """Query-outer online softmax with one normalisation at the end.

    q, k, v: [N, d] float64 arrays of one head.  Returns (o [N, d], lse [N]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    br = br or n
    bc = bc or n
    o_out = np.zeros((n, v.shape[1]))
    lse_out = np.full(n, -np.inf)
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(i0 + br, n))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        o = np.zeros((rows.size, v.shape[1]))
        for j0 in range(0, n, bc):
            cols = np.arange(j0, min(j0 + bc, n))
            s = _scores(q[rows], k[cols], scale, rows, cols, causal)
            m_new = np.maximum(m, s.max(axis=1))
            shift = _safe(m_new)
            p = np.exp(s - shift[:, None])
            alpha = np.exp(m - shift)
            l = alpha * l + p.sum(axis=1)
            o = alpha[:, None] * o + p @ v[cols]
            m = m_new
        seen = l > 0
        o_out[rows[seen]] = o[seen] / l[seen, None]
        lse_out[rows[seen]] = m[seen] + np.log(l[seen])
    return o_out, lse_out


def normalised(q, k, v, scale, causal=False, br=None, bc=None):
    """Key/value-outer online softmax that keeps O normalised every step.

    q, k, v: [N, d] float64 arrays of one head.  Returns (o [N, d], lse [N]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    br = br or n
    bc = bc or n
    m = np.full(n, -np.inf)          # per-row state carried between outer steps
    l = np.zeros(n)
    o = np.zeros((n, v.shape[1]))
    for j0 in range(0, n, bc):
        cols = np.arange(j0, min(j0 + bc, n))
        for i0 in range(0, n, br):
            rows = np.arange(i0, min(i0 + br, n))
            s = _scores(q[rows], k[cols], scale, rows, cols, causal)
            m_blk = s.max(axis=1)
            p_blk = np.exp(s - _safe(m_blk)[:, None])
            l_blk = p_blk.sum(axis=1)
            m_old, l_old = m[rows], l[rows]
            m_new = np.maximum(m_old, m_blk)
            shift = _safe(m_new)
            a_old = np.exp(m_old - shift)
            a_blk = np.exp(m_blk - shift)
            l_new = a_old * l_old + a_blk * l_blk
            upd = l_new > 0
            o_rows = o[rows]
            o_new = (l_old * a_old)[:, None] * o_rows + a_blk[:, None] * (p_blk @ v[cols])
            o_rows[upd] = o_new[upd] / l_new[upd, None]
            o[rows] = o_rows
            m[rows] = np.where(upd, m_new, m_old)
            l[rows] = np.where(upd, l_new, l_old)
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse
