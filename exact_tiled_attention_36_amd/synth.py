"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module holds no attention arithmetic. It only draws numbers and stores them:

* values are i.i.d. standard normal float32 from ``numpy.random.default_rng(seed)``
  (PCG64), drawn in the fixed order Q, K, V, dO;
* bf16 inputs are those float32 draws rounded to bfloat16 with round-to-nearest-even;
  the generator hands out the raw 16-bit patterns so that the GPU buffers and the
  oracle's float64 copies are built from exactly the same bits;
* an optional power-of-two multiplier on Q (exact in binary floating point) drives
  large logits through the online-softmax rescale.

The pages' own accuracy harness (FlashAttention1 pseudo-implementation article on
gitcode.csdn.net, §三, its test block) draws ``torch.randn`` Q, K, V; these inputs
follow the same distribution with a reproducible generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Inputs here are finite normal draws, so NaN handling is not needed; infinities
    and overflow to infinity still follow the usual IEEE rounding result.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    return bf16_bits_to_f32(b).astype(np.float64)


@dataclass
class AttnInputs:
    """One seeded problem. Shapes: q/do ``[B,Hq,Nq,d]``, k/v ``[B,Hkv,Nk,d]``.

    ``dtype`` is ``"bf16"`` (arrays hold uint16 bit patterns) or ``"f32"`` (arrays
    hold float32 values).
    """

    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    scale: float
    dtype: str
    seed: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f64(a)
        return np.asarray(a, dtype=np.float64)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a)
        return np.asarray(a, dtype=np.float32)


def make_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, *,
                causal: bool, seed: int, dtype: str = "bf16",
                q_mult: float = 1.0, with_do: bool = False,
                scale: Optional[float] = None) -> AttnInputs:
    """Draw Q, K, V (and dO) in that order from ``default_rng(seed)``.

    ``q_mult`` must be a power of two so that scaling before or after rounding gives
    the same bits. ``scale`` defaults to 1/sqrt(d).
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    m, e = np.frexp(q_mult)
    if m != 0.5:
        raise ValueError("q_mult must be a power of two")
    rng = np.random.default_rng(seed)
    shp_q = (B, Hq, Nq, d)
    shp_kv = (B, Hkv, Nk, d)
    q = rng.standard_normal(shp_q, dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    k = rng.standard_normal(shp_kv, dtype=np.float32)
    v = rng.standard_normal(shp_kv, dtype=np.float32)
    do = rng.standard_normal(shp_q, dtype=np.float32) if with_do else None
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        if do is not None:
            do = f32_to_bf16_bits(do)
    sc = float(1.0 / np.sqrt(d)) if scale is None else float(scale)
    return AttnInputs(B, Hq, Hkv, Nq, Nk, d, bool(causal), sc, dtype, seed,
                      q, k, v, do)


# The workloads of the method's benchmark table: name -> (shape args, options).
# Seeds are fixed per workload; the Q-times-4 variant of the small bf16 case uses
# its own seed.
WORKLOADS = {
    "c1_f32_B1H1N256d64":
        dict(B=1, Hq=1, Hkv=1, Nq=256, Nk=256, d=64, causal=False, seed=101,
             dtype="f32"),
    "c2_bf16_B2H16N1024d64":
        dict(B=2, Hq=16, Hkv=16, Nq=1024, Nk=1024, d=64, causal=False, seed=201),
    "c2_bf16_B2H16N1024d64_qx4":
        dict(B=2, Hq=16, Hkv=16, Nq=1024, Nk=1024, d=64, causal=False, seed=202,
             q_mult=4.0),
    "c3a_bf16_causal_B4H32N4096d128":
        dict(B=4, Hq=32, Hkv=32, Nq=4096, Nk=4096, d=128, causal=True, seed=301),
    "c3b_bf16_causal_B2H16N4096d256":
        dict(B=2, Hq=16, Hkv=16, Nq=4096, Nk=4096, d=256, causal=True, seed=302),
    "c4a_bf16_causal_B1H8N32768d128":
        dict(B=1, Hq=8, Hkv=8, Nq=32768, Nk=32768, d=128, causal=True, seed=401),
    "c4b_bf16_decode_B8H8Nq1Nk32768d128":
        dict(B=8, Hq=8, Hkv=8, Nq=1, Nk=32768, d=128, causal=True, seed=402),
    "c5_bf16_causal_gqa_B2Hq32Hkv8N8192d128":
        dict(B=2, Hq=32, Hkv=8, Nq=8192, Nk=8192, d=128, causal=True, seed=501,
             with_do=True),
}


def workload(name: str, **over) -> AttnInputs:
    kw = dict(WORKLOADS[name])
    kw.update(over)
    return make_inputs(**kw)
