"""Brute-force attention with plain Python scalars (tiny problems only).

TEST INFRASTRUCTURE — part of the oracle; see ``oracle/attention.py`` for who may
import it. No numpy: every dot product and row sum goes through ``math.fsum`` and
every exponential through ``math.exp``. This is the definition of
"FlashAttention" (ruizhehou.github.io), §一 (scores, softmax, weighted sum of V) with
the safe softmax of §二.2, written a second time in a different way, so that it can
pin the vectorised oracle on inputs with N <= 16.
"""
from __future__ import annotations

import math


def _visible(i, j, nq, nk, causal):
    return (not causal) or (j <= i + (nk - nq))


def forward_head(q, k, v, scale, causal=False):
    """q: Nq lists of d floats; k, v: Nk lists. Returns (o rows, lse list)."""
    nq, nk = len(q), len(k)
    d = len(v[0]) if nk else 0
    o, lse = [], []
    for i in range(nq):
        s = {}
        for j in range(nk):
            if _visible(i, j, nq, nk, causal):
                s[j] = scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i])))
        if not s:
            o.append([0.0] * d)
            lse.append(-math.inf)
            continue
        m = max(s.values())
        e = {j: math.exp(x - m) for j, x in s.items()}
        z = math.fsum(e.values())
        o.append([math.fsum(e[j] * v[j][c] for j in e) / z for c in range(d)])
        lse.append(m + math.log(z))
    return o, lse


def forward(q, k, v, scale, causal=False):
    """Nested lists [B][Hq][Nq][d] and [B][Hkv][Nk][d]; kv head = h // (Hq // Hkv)."""
    B, Hq, Hkv = len(q), len(q[0]), len(k[0])
    g = Hq // Hkv
    o = [[None] * Hq for _ in range(B)]
    lse = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            o[b][h], lse[b][h] = forward_head(q[b][h], k[b][h // g], v[b][h // g],
                                              scale, causal)
    return o, lse
