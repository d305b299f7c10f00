"""Exact scaled-dot-product attention in float64, computed straight from its definition.

TEST INFRASTRUCTURE — the oracle. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with the HIP
library or its Python binding and imports neither.

Sources (the pages this follows):

* "FlashAttention" (ruizhehou.github.io), §一 (standard attention's IO problem): the
  per-head score matrix is Q K^T divided by sqrt(d), the weights are its row-wise
  softmax, and the output is the weights times V. §二.2 gives the numerically safe
  softmax that subtracts the row maximum before exponentiating.
* FlashAttention1 article (gitcode.csdn.net), §一: the same formula,
  softmax(Q K^T / sqrt(d_k)) V.
* "FlashAttention" (ruizhehou.github.io), §二.3 (recomputation): the forward keeps two
  statistics per row (its running max m and normaliser l) so that the backward can
  rebuild P; here they are returned folded into one log-sum-exp value per row,
  lse = m + ln(l), from which P = exp(s - lse).
* "FlashAttention" (ruizhehou.github.io), §五: the causal flag of the library call.
* "FlashAttention" (newton.com.tw wiki), 發展歷程 (FlashAttention-2 paragraph): the
  method supports multi-query and grouped-query attention.

Readings where the pages are silent (each is listed in the design notes):

* ``scale`` is an argument; the pages' value is 1/sqrt(d).
* causal masking is aligned to the bottom-right corner: query row i (0-based) sees key
  j iff j <= i + (Nk - Nq). For Nq == Nk this is the usual lower triangle.
* grouped-query mapping: query head h reads key/value head h // (Hq // Hkv).
* a query row that sees no key gets o = 0 and lse = -inf.
* the backward pass is the textbook chain rule of softmax attention (the pages give
  no formulas for it): dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij,
  dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q, with dK and dV summed over
  the query heads of a group.

Row blocking below only bounds memory: every row of S is still formed and
normalised in full, and rows never interact, so no arithmetic is reordered.
"""
from __future__ import annotations

import numpy as np

_ROW_BLOCK = 2048


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _dims(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if k.shape[:3] != v.shape[:3] or Bk != B or dk != d:
        raise ValueError("shape mismatch")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Nq, Nk, d, Hq // Hkv


def visible(rows: np.ndarray, Nq: int, Nk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), Nk]: which keys each query row may attend to."""
    rows = np.asarray(rows)
    if not causal:
        return np.ones((rows.size, Nk), dtype=bool)
    j = np.arange(Nk)[None, :]
    return j <= (rows[:, None] + (Nk - Nq))


def scores(q_rows: np.ndarray, k_head: np.ndarray, scale: float,
           rows: np.ndarray, Nq: int, causal: bool) -> np.ndarray:
    """s_ij = scale * q_i . k_j, with invisible entries set to -inf."""
    s = scale * (_f64(q_rows) @ _f64(k_head).T)
    mask = visible(rows, Nq, k_head.shape[0], causal)
    s[~mask] = -np.inf
    return s


def softmax_rows(s: np.ndarray):
    """Safe softmax of each row of s: returns (P, m, l) with P = exp(s - m) / l.

    Rows that are all -inf give P = 0, m = -inf, l = 0.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return p, m, l


def probabilities(q, k, scale: float, causal: bool) -> np.ndarray:
    """Full attention weights P, shape [B, Hq, Nq, Nk] (small problems only)."""
    q, k = _f64(q), _f64(k)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, Nq, Nk))
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(Hq):
            s = scores(q[b, h], k[b, h // g], scale, rows, Nq, causal)
            out[b, h] = softmax_rows(s)[0]
    return out


def forward_rows(q, k, v, scale: float, causal: bool, b: int, h: int,
                 rows) -> tuple[np.ndarray, np.ndarray]:
    """Output rows o_i and lse_i of head (b, h) for the given query row indices."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, Nq, Nk, d, g = _dims(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    s = scores(q[b, h, rows], k[b, h // g], scale, rows, Nq, causal)
    p, m, l = softmax_rows(s)
    o = p @ v[b, h // g]
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def forward_head(q, k, v, scale: float, causal: bool, b: int, h: int):
    """O [Nq,d] and LSE [Nq] of one head (b, h), every row."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Nq = q.shape[2]
    o = np.zeros((Nq, v.shape[3]))
    lse = np.zeros(Nq)
    for r0 in range(0, Nq, _ROW_BLOCK):
        rows = np.arange(r0, min(Nq, r0 + _ROW_BLOCK))
        o[rows], lse[rows] = forward_rows(q, k, v, scale, causal, b, h, rows)
    return o, lse


def forward(q, k, v, scale: float, causal: bool):
    """O [B,Hq,Nq,d] and LSE [B,Hq,Nq] in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, Nq, Nk, d, g = _dims(q, k, v)
    o = np.zeros((B, Hq, Nq, v.shape[3]))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h] = forward_head(q, k, v, scale, causal, b, h)
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool):
    """Gradients of sum(dO * O) w.r.t. Q, K, V, plus D_i = sum_j P_ij dP_ij.

    Returns (dq [B,Hq,Nq,d], dk [B,Hkv,Nk,d], dv [B,Hkv,Nk,d], D [B,Hq,Nq]).
    P is rebuilt from its definition (the same rows as ``forward``).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Hkv, Nq, Nk, d, g = _dims(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must match Q")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    D = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            for r0 in range(0, Nq, _ROW_BLOCK):
                rows = np.arange(r0, min(Nq, r0 + _ROW_BLOCK))
                s = scores(q[b, h, rows], k[b, kvh], scale, rows, Nq, causal)
                p = softmax_rows(s)[0]
                dO = do[b, h, rows]
                dv[b, kvh] += p.T @ dO
                dp = dO @ v[b, kvh].T
                Di = (p * dp).sum(axis=1)
                ds = p * (dp - Di[:, None])
                dq[b, h, rows] = scale * (ds @ k[b, kvh])
                dk[b, kvh] += scale * (ds.T @ q[b, h, rows])
                D[b, h, rows] = Di
    return dq, dk, dv, D


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine normalised partial results over disjoint key chunks.

    ``o_parts`` [C, ..., d] and ``lse_parts`` [C, ...] hold, for each chunk c, the
    attention output and log-sum-exp over that chunk's keys alone. Rescaling each by
    exp(lse_c - lse) with lse = log sum_c exp(lse_c) is the online-softmax update of
    "FlashAttention" (ruizhehou.github.io), §二.2, applied to whole chunks. Chunks
    with lse_c = -inf (no visible key) contribute nothing.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    m = lse_parts.max(axis=0)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    w = np.exp(lse_parts - m_safe[None])
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
        wn = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse
