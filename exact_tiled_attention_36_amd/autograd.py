"""PyTorch autograd entry point over the C-ABI forward and backward.

The user-level call on the pages is ``torch.nn.functional.scaled_dot_product_attention``
with ``attn_mask=None``, ``dropout_p=0.0`` and ``is_causal`` ("FlashAttention"
(ruizhehou.github.io), §五). ``scaled_dot_product_attention`` below takes the same
arguments for the case the library computes and refuses the rest; every step runs in
libfa.so (``fa_fwd`` / ``fa_fwd_f32`` forward, ``fa_bwd`` backward), this module only
marshals tensors and saves what the backward needs: q, k, v, O and the per-row LSE, the
statistics the pages keep instead of the score matrix (§二.3).

Differences from torch's function, stated here because they change results:
  * causal masking is aligned bottom-right when Nq != Nk (query row i sees keys
    j <= i + Nk - Nq); torch aligns top-left. For Nq == Nk the two agree.
  * a query row that sees no key (only possible for causal with Nq > Nk) returns 0.
  * layouts are contiguous [B, H, N, d]; bf16 supports forward and backward, float32
    forward only; head dims 64, 128, 256 for bf16.
"""
from __future__ import annotations

import math
from typing import Optional

from . import fa


def _torch():
    import torch
    return torch


class _FlashAttention(_torch().autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale: float):
        o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if q.dtype != _torch().bfloat16:
            raise NotImplementedError("the backward pass supports bfloat16 inputs only")
        dq, dk, dv = fa.bwd(q, k, v, o, do.contiguous(), lse, causal=ctx.causal,
                            scale=ctx.scale)
        return dq, dk, dv, None, None


def scaled_dot_product_attention(query, key, value, attn_mask=None, dropout_p: float = 0.0,
                                 is_causal: bool = False, scale: Optional[float] = None,
                                 enable_gqa: bool = False):
    """softmax(scale * query key^T [causal mask]) value, exact, with gradients.

    query [B, Hq, Nq, d], key/value [B, Hkv, Nk, d] (Hkv < Hq needs enable_gqa=True and
    Hq % Hkv == 0; query head h uses key/value head h // (Hq / Hkv)). scale defaults to
    1/sqrt(d). Raises NotImplementedError for masks and dropout, ValueError for shapes,
    dtypes or devices the library does not take (there is no fallback path)."""
    if attn_mask is not None:
        raise NotImplementedError("attn_mask is not supported (only is_causal)")
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported")
    for name, t in (("query", query), ("key", key), ("value", value)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
    if query.shape[1] != key.shape[1] and not enable_gqa:
        raise ValueError("query and key/value head counts differ: pass enable_gqa=True")
    d = query.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return _FlashAttention.apply(query.contiguous(), key.contiguous(), value.contiguous(),
                                 bool(is_causal), sc)
