"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module holds no attention arithmetic. It only draws numbers and stores them:

* values are i.i.d. standard normal float32 from ``numpy.random.default_rng(seed)``
  (PCG64), drawn in the fixed order Q, K, V, dO;
* bf16 inputs are those float32 draws rounded to bfloat16 with round-to-nearest-even;
  the generator hands out the raw 16-bit patterns so that the GPU buffers and the
  oracle's float64 copies are built from exactly the same bits;
* an optional power-of-two multiplier on Q (exact in binary floating point) drives
  large logits through the online-softmax rescale;
* FP8 inputs (``make_fp8_inputs``) are E4M3 codes with one float32 scale per tensor:
  either the same normal draws scaled so that each tensor's largest magnitude maps to
  E4M3's largest finite value 448 and rounded to nearest even ("gauss"), or sparse
  sign patterns whose scores are small integers ("signs", see that function).

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


# ----------------------------------------------------------------------------------
# FP8 (OCP E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, exponent
# field 0 for subnormals m * 2^-9, codes 0x7f / 0xff NaN, no infinities, max 448)
# ----------------------------------------------------------------------------------

E4M3_MAX = 448.0


def f64_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round finite values with |x| <= 448 to E4M3 (nearest, ties to even); uint8 codes.

    Normal range: the spacing of representable values in [2^e, 2^(e+1)) is 2^(e-3);
    below 2^-6 (subnormals) it is 2^-9. Rounding is np.rint on the value divided by
    its spacing (exact power-of-two scaling), which rounds ties to even.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("E4M3 input must be finite with |x| <= 448")
    sign = np.signbit(x)
    a = np.abs(x)
    _, e2 = np.frexp(a)                       # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, -6)                # exponent of the binade; subnormals use -6
    spacing = np.ldexp(1.0, e - 3)
    n = np.rint(a / spacing)                  # integer multiple of the spacing
    # n in [8, 16] for normals (16 = carry into the next binade), [0, 8] below 2^-6
    carry = n >= 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, n / 2, n)
    normal = n >= 8
    code = np.where(normal, ((e + 7) << 3) + (n - 8), n).astype(np.int64)
    code = np.where(a == 0, 0, code)
    if np.any(code > 0x7E):
        raise ValueError("value rounds past 448")
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


@dataclass
class Fp8Inputs:
    """One seeded FP8 problem: q/k/v uint8 E4M3 codes and float32 descales; the true
    tensors are descale * decoded codes."""

    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    scale: float
    seed: int
    kind: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    descale_q: float
    descale_k: float
    descale_v: float


def _quantize_per_tensor(x: np.ndarray):
    amax = float(np.max(np.abs(x)))
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(x.astype(np.float64) / float(s), -E4M3_MAX, E4M3_MAX)
    return f64_to_e4m3_bits(y), float(s)


def make_fp8_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, *,
                    causal: bool, seed: int, kind: str = "gauss",
                    scale: Optional[float] = None) -> Fp8Inputs:
    """Draw an FP8 problem from ``default_rng(seed)`` (order Q, K, V).

    kind "gauss": standard normal Q, K, V, each quantised with its own scale
    amax / 448 (the float32 descale returned). ``scale`` defaults to 1/sqrt(d).

    kind "signs": every Q row has exactly 4 entries of +-1 (random positions and
    signs) and zeros elsewhere; K entries are -1, 0, +1 with probability 1/3 each; V is
    quantised normal as above; descale_q = descale_k = 1 and scale = float32(ln 2).
    Every score q.k is then an integer in [-4, 4] and scale * log2(e) is 1 up to
    float32 rounding, so each softmax weight 2^(s - m), taken against any base m within
    8 of the scores, is a power of two that E4M3 holds exactly.
    """
    rng = np.random.default_rng(seed)
    shp_q, shp_kv = (B, Hq, Nq, d), (B, Hkv, Nk, d)
    if kind == "gauss":
        q, dq = _quantize_per_tensor(rng.standard_normal(shp_q, dtype=np.float32))
        k, dk = _quantize_per_tensor(rng.standard_normal(shp_kv, dtype=np.float32))
        v, dv = _quantize_per_tensor(rng.standard_normal(shp_kv, dtype=np.float32))
        sc = float(1.0 / np.sqrt(d)) if scale is None else float(scale)
    elif kind == "signs":
        if d < 4:
            raise ValueError("signs needs d >= 4")
        qv = np.zeros(shp_q)
        pos = np.argsort(rng.random(shp_q), axis=-1)[..., :4]
        sgn = rng.choice([-1.0, 1.0], size=shp_q[:-1] + (4,))
        np.put_along_axis(qv, pos, sgn, axis=-1)
        kv = rng.integers(-1, 2, size=shp_kv).astype(np.float64)
        q, dq = f64_to_e4m3_bits(qv), 1.0
        k, dk = f64_to_e4m3_bits(kv), 1.0
        v, dv = _quantize_per_tensor(rng.standard_normal(shp_kv, dtype=np.float32))
        sc = float(np.float32(np.log(2.0)))
    else:
        raise ValueError(kind)
    return Fp8Inputs(B, Hq, Hkv, Nq, Nk, d, bool(causal), sc, seed, kind, q, k, v,
                     float(dq), float(dk), float(dv))
