"""FP8 (E4M3) decoding and the reference for the FP8 forward pass, in float64.

TEST INFRASTRUCTURE — the oracle. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with the HIP
library or its Python binding and imports neither.

Sources:

* "FlashAttention" (newton.com.tw wiki), 發展歷程 (the third version's paragraph): the
  method has a low-precision FP8 form. The pages give neither its number format nor
  its scaling, so the readings here are: inputs are E4M3 codes with one float32 scale
  per tensor, the true tensors are ``descale * decoded codes``, and the result to
  match is the exact attention of those true tensors, as defined in ``attention.py``
  ("FlashAttention" (ruizhehou.github.io), §一).
* The E4M3 encoding is the public OCP 8-bit floating-point format (OFP8): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
  m * 2^-9; the codes with all exponent and mantissa bits set (0x7f, 0xff) are NaN;
  there are no infinities, and the largest finite value is 448.
* The FP8 forward rounds each softmax weight to E4M3 before the product with V (the
  one rounding its design adds; a reading, since the pages do not say where FP8 is
  used inside the loop). ``p_rounding_bound`` turns that into a per-element error
  bound: a value w rounded to nearest E4M3 moves by at most max(w / 16, 2^-10)
  (half the spacing: 2^-4 relative in the normal range, 2^-10 absolute among the
  subnormals). Weights are formed as 2^(s - m) against a base m no larger than the
  row's maximum score, so in units of the row's largest weight the absolute floor is
  at most 2^-10; after normalisation by the row sum L that is 2^-10 * P_max.
* Scores may carry an accumulation error of the matrix instruction that forms them
  (a hardware property the pages do not cover). ``score_error`` bounds it per row as
  E_i = acc_eps * scale * descale_q * descale_k * max_j sum_d |Q8_id K8_jd| over the
  visible keys j, with acc_eps supplied by the caller. Scores off by at most E_i move
  lse by at most E_i and each normalised weight by a factor within exp(+-2 E_i), which
  ``p_rounding_bound`` adds when given the same acc_eps:
      bound_ic = e^(2E_i) sum_j max(P_ij/16, 2^-10 P_max_i) |v_jc|
                 + (e^(2E_i) - 1) sum_j P_ij |v_jc|.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

_ROW_BLOCK = 1024


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode E4M3 bytes to float64 (NaN for 0x7f / 0xff), from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    sub = sign * np.ldexp(m.astype(np.float64), -9)
    val = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def dequantize(codes, descale: float) -> np.ndarray:
    """The true tensor: descale times the decoded codes (float64, exact)."""
    return float(descale) * e4m3_to_f64(codes)


def forward_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
                scale: float, causal: bool):
    """O [B,Hq,Nq,d] and LSE [B,Hq,Nq] (float64) of the dequantised inputs."""
    return A.forward(dequantize(q8, descale_q), dequantize(k8, descale_k),
                     dequantize(v8, descale_v), scale, causal)


def _one_head(q8, k8, v8, descale_q, descale_k, descale_v, b, h):
    """Dequantised [1,1,N,d] slices of query head (b, h) and its key/value head; the
    slices keep their row counts, so the causal alignment is unchanged."""
    g = q8.shape[1] // k8.shape[1]
    kvh = h // g
    return (dequantize(q8[b:b + 1, h:h + 1], descale_q),
            dequantize(k8[b:b + 1, kvh:kvh + 1], descale_k),
            dequantize(v8[b:b + 1, kvh:kvh + 1], descale_v))


def forward_fp8_rows(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
                     scale: float, causal: bool, b: int, h: int, rows):
    """Rows of O and LSE of head (b, h) of the dequantised inputs."""
    q, k, v = _one_head(q8, k8, v8, descale_q, descale_k, descale_v, b, h)
    return A.forward_rows(q, k, v, scale, causal, 0, 0, np.asarray(rows, dtype=np.int64))


def _score_error_rows(q, k, scale, causal, b, h, rows, acc_eps):
    """E_i for the given rows of head (b, h) (q, k dequantised)."""
    g = q.shape[1] // k.shape[1]
    mag = np.abs(q[b, h, rows]) @ np.abs(k[b, h // g]).T          # sum_d |q_d k_d|
    mag = np.where(A.visible(rows, q.shape[2], k.shape[2], causal), mag, 0.0)
    return acc_eps * abs(scale) * mag.max(axis=1, initial=0.0)


def _bound_rows(q, k, v, scale, causal, b, h, rows, acc_eps):
    g = q.shape[1] // k.shape[1]
    s = A.scores(q[b, h, rows], k[b, h // g], scale, rows, q.shape[2], causal)
    p = A.softmax_rows(s)[0]
    pmax = p.max(axis=1, keepdims=True)
    err = np.where(p > 0, np.maximum(p / 16.0, 2.0 ** -10 * pmax), 0.0)
    grow = np.exp(2.0 * _score_error_rows(q, k, scale, causal, b, h, rows, acc_eps))[:, None]
    av = np.abs(v[b, h // g])
    return grow * (err @ av) + (grow - 1.0) * (p @ av)


def score_error(q8, k8, descale_q: float, descale_k: float, scale: float, causal: bool,
                acc_eps: float) -> np.ndarray:
    """E [B,Hq,Nq]: bound on the score error of each row given the relative accumulation
    error acc_eps of the score product (see the module notes); also bounds |lse error|."""
    q = dequantize(q8, descale_q)
    k = dequantize(k8, descale_k)
    B, Hq, Nq, _ = q.shape
    out = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Nq, _ROW_BLOCK):
                rows = np.arange(r0, min(Nq, r0 + _ROW_BLOCK))
                out[b, h, rows] = _score_error_rows(q, k, scale, causal, b, h, rows, acc_eps)
    return out


def score_error_rows(q8, k8, descale_q: float, descale_k: float, scale: float,
                     causal: bool, b: int, h: int, rows, acc_eps: float) -> np.ndarray:
    """``score_error`` for some query rows of head (b, h) only."""
    q, k, _ = _one_head(q8, k8, k8, descale_q, descale_k, 1.0, b, h)
    return _score_error_rows(q, k, scale, causal, 0, 0, np.asarray(rows, dtype=np.int64),
                             acc_eps)


def p_rounding_bound(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
                     scale: float, causal: bool, acc_eps: float = 0.0) -> np.ndarray:
    """Per-element bound [B,Hq,Nq,d] on |O_fp8 - O_exact| from rounding the weights,
    sum_j max(P_ij / 16, 2^-10 P_max_i) |v_jc| with P the exact softmax weights, widened
    for score errors of relative size acc_eps (module notes)."""
    q = dequantize(q8, descale_q)
    k = dequantize(k8, descale_k)
    v = dequantize(v8, descale_v)
    B, Hq, Nq, d = q.shape
    out = np.zeros((B, Hq, Nq, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Nq, _ROW_BLOCK):
                rows = np.arange(r0, min(Nq, r0 + _ROW_BLOCK))
                out[b, h, rows] = _bound_rows(q, k, v, scale, causal, b, h, rows, acc_eps)
    return out


def p_rounding_bound_rows(q8, k8, v8, descale_q: float, descale_k: float,
                          descale_v: float, scale: float, causal: bool, b: int, h: int,
                          rows, acc_eps: float = 0.0) -> np.ndarray:
    """``p_rounding_bound`` for some query rows of head (b, h) only."""
    q, k, v = _one_head(q8, k8, v8, descale_q, descale_k, descale_v, b, h)
    return _bound_rows(q, k, v, scale, causal, 0, 0, np.asarray(rows, dtype=np.int64),
                       acc_eps)
