"""The pages' block recurrences for one head, in float64 (self-checks of the oracle).

TEST INFRASTRUCTURE — part of the oracle; see ``oracle/attention.py`` for who may
import it. These are independent formulations of the same result: the pages state
that tiling with online softmax is exactly equivalent to the one-shot softmax
("FlashAttention" (ruizhehou.github.io), end of §二.2 and §五 "no precision loss";
§六 summary). Agreement of these loops with ``attention.forward`` for every block
size is one of the pins of the oracle.

* ``online_v1``: the running-state update of §二.2 ("FlashAttention",
  ruizhehou.github.io): per key/value block, the running max m and normaliser l are
  updated and the running output is kept *normalised*: the old output is rescaled by
  exp(m_old - m_new) * l_old and the block's exp-weighted values are added, then the
  sum is divided by the new l. (The v1 loop printed in §四.1 drops that division and
  divides once at the end; run for two or more blocks it would compound l, so the
  self-consistent §二.2 form is the one followed here.)
* ``online_v2``: §四.1's FlashAttention-2 form: the output accumulator stays
  unnormalised, is rescaled only by exp(m_old - m_new) per block, and is divided by
  l once after the last block. Q is tiled in an outer loop and K/V in an inner loop,
  as in §三 (the complete computation graph).

The FlashAttention1 article (gitcode.csdn.net, §三) describes the same deferred
recurrence with every query row in one block and K/V blocks clipped to the sequence
length; ``online_v2`` with ``block_q`` = the number of query rows is that case.
"""
from __future__ import annotations

import numpy as np


def _mask(rows, cols, Nq, Nk, causal):
    if not causal:
        return np.ones((len(rows), len(cols)), dtype=bool)
    return np.asarray(cols)[None, :] <= np.asarray(rows)[:, None] + (Nk - Nq)


def _exp_minus(a, b):
    """exp(a - b) with the convention that a running max of -inf means 'empty'."""
    b = np.where(np.isneginf(b), 0.0, b)
    return np.exp(a - b)


def online_v1(q, k, v, scale, block_k, causal=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    Nq, Nk = q.shape[0], k.shape[0]
    rows = np.arange(Nq)
    m = np.full(Nq, -np.inf)
    l = np.zeros(Nq)
    o = np.zeros((Nq, v.shape[1]))
    for j0 in range(0, Nk, block_k):
        cols = np.arange(j0, min(Nk, j0 + block_k))
        s = scale * (q @ k[cols].T)
        s[~_mask(rows, cols, Nq, Nk, causal)] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        alpha = _exp_minus(m, m_new)
        e = _exp_minus(s, m_new[:, None])
        l_new = alpha * l + e.sum(axis=1)
        num = (alpha * l)[:, None] * o + e @ v[cols]
        o = np.where(l_new[:, None] > 0, num / np.where(l_new > 0, l_new, 1.0)[:, None], 0.0)
        m, l = m_new, l_new
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def online_v2(q, k, v, scale, block_q, block_k, causal=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    Nq, Nk = q.shape[0], k.shape[0]
    o = np.zeros((Nq, v.shape[1]))
    lse = np.zeros(Nq)
    for i0 in range(0, Nq, block_q):
        rows = np.arange(i0, min(Nq, i0 + block_q))
        qi = q[rows]
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), v.shape[1]))
        for j0 in range(0, Nk, block_k):
            cols = np.arange(j0, min(Nk, j0 + block_k))
            s = scale * (qi @ k[cols].T)
            s[~_mask(rows, cols, Nq, Nk, causal)] = -np.inf
            m_new = np.maximum(m, s.max(axis=1))
            alpha = _exp_minus(m, m_new)
            pt = _exp_minus(s, m_new[:, None])
            acc = alpha[:, None] * acc + pt @ v[cols]
            l = alpha * l + pt.sum(axis=1)
            m = m_new
        o[rows] = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            lse[rows] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse

