"""GPU parity of the FP8 forward (fa_fwd_fp8) against the float64 oracle.

The oracle is the exact attention of the dequantised inputs (oracle/fp8.py). The
kernel adds one rounding, the softmax weights to E4M3 before the product with V, so
the parity bar is derived from that arithmetic:

* "signs" inputs (scores are integers in [-4, 4], scale * log2(e) = 1 to float32
  rounding): every weight is a power of two that E4M3 holds exactly, so O must match
  the exact result to bf16 output rounding: |err| <= 2^-8 |O| + 1e-4 max|v|. A wrong
  key/column permutation, mask or scale shows here at full size.
* normal ("gauss") inputs with per-tensor amax scaling: elementwise
  |err| <= 1.02 * bound + 2^-8 |O| + 1e-4 max|v|, with the oracle's
  p_rounding_bound = sum_j max(P_ij / 16, 2^-10 P_max) |v_jc|; and, since rounding
  errors of many weights partly cancel, the mean error must stay below a quarter of
  the mean bound.
* lse comes from unrounded float32 weights: |err| <= 1e-4 where the scores are exact
  (signs inputs). In general the FP8 matrix instruction does not sum its 64 products
  exactly in float32: with one key per row (lse = the score) its error measured up to
  2^-15.2 of sum_d |q_d k_d| over 49k normal scores at d = 64, 128, 256. The bar takes
  acc_eps = 2^-13 of that sum (the oracle's score_error E_i) and allows
  |lse err| <= E_i + 1e-5 (1 + |lse|), with O's bound widened to match.
"""
import math

import numpy as np
import pytest

from exact_tiled_attention_36_amd import synth
from oracle import fp8 as F
from gpu_util import announce, to_host64

pytestmark = pytest.mark.gpu

TOL_LSE_FP8 = 1e-4
BF16_HALF_ULP = 2.0 ** -8
ACC_EPS = 2.0 ** -13


def run_fp8(fa, a, scale=None):
    import torch
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    o, lse = fa.fwd_fp8(dev(a.q), dev(a.k), dev(a.v), a.descale_q, a.descale_k,
                        a.descale_v, causal=a.causal, scale=a.scale if scale is None else scale)
    torch.cuda.synchronize()
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


def vmax(a):
    return float(np.abs(F.dequantize(a.v, a.descale_v)).max())


def check_lse(lse, lse_ref, what, score_err=None):
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: -inf rows differ"
    assert np.all(lse[~fin] == lse_ref[~fin])
    if score_err is None:
        tol = np.full(lse_ref.shape, TOL_LSE_FP8)
    else:
        tol = score_err + 1e-5 * (1.0 + np.abs(np.where(fin, lse_ref, 0.0)))
    ratio = (np.abs(lse[fin] - lse_ref[fin]) / tol[fin]).max(initial=0.0)
    assert ratio <= 1.0, f"{what}: lse err/tol {ratio:.3f}"


def check_exact_weights(o, lse, o_ref, lse_ref, vm, what):
    err = np.abs(o - o_ref)
    tol = BF16_HALF_ULP * np.abs(o_ref) + 1e-4 * vm
    worst = float((err / tol).max(initial=0.0))
    assert worst <= 1.0, f"{what}: err/tol {worst:.3f} (max err {err.max():.3e})"
    check_lse(lse, lse_ref, what)


def check_bounded(o, lse, o_ref, lse_ref, bound, score_err, vm, what, mean_check=True):
    err = np.abs(o - o_ref)
    tol = 1.02 * bound + BF16_HALF_ULP * np.abs(o_ref) + 1e-4 * vm
    worst = float((err / tol).max(initial=0.0))
    assert worst <= 1.0, f"{what}: err/tol {worst:.3f}"
    if mean_check:
        assert err.mean() <= 0.25 * bound.mean() + 1e-5 * vm, (
            f"{what}: mean err {err.mean():.3e} vs mean bound {bound.mean():.3e}")
    check_lse(lse, lse_ref, what, score_err)


SHAPES = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 1, 1, 128, False),
    (1, 2, 1, 3, 3, 64, True),
    (2, 4, 2, 300, 300, 128, True),        # several tiles and a ragged tail, GQA
    (1, 4, 4, 256, 256, 64, False),
    (1, 2, 1, 200, 77, 128, False),        # Nk not a multiple of the key tile
    (1, 2, 2, 77, 333, 128, True),         # Nq < Nk: bottom-right diagonal
    (1, 2, 1, 300, 100, 128, True),        # Nq > Nk: first rows see no key
    (1, 3, 1, 130, 130, 256, True),
    (2, 4, 2, 300, 300, 256, True),        # d = 256: GQA, ragged tail
    (1, 2, 1, 200, 77, 256, False),        # d = 256: key tail
    (1, 2, 2, 77, 333, 256, True),         # d = 256: bottom-right diagonal
    (1, 2, 1, 300, 100, 256, True),        # d = 256: first rows see no key
    (1, 8, 1, 129, 511, 256, True),        # d = 256: MQA
    (1, 8, 1, 129, 511, 64, True),         # MQA
    (2, 2, 2, 1, 700, 128, True),          # one query row
]


@pytest.mark.parametrize("shape", SHAPES)
def test_exact_weights(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    a = synth.make_fp8_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, seed=3000 + Nq + Nk + d,
                              kind="signs")
    announce(f"fwd_fp8 signs {shape}")
    o, lse = run_fp8(gpu_lib, a)
    o_ref, lse_ref = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                                   a.scale, causal)
    check_exact_weights(o, lse, o_ref, lse_ref, vmax(a), f"signs{shape}")


@pytest.mark.parametrize("shape", SHAPES)
def test_gauss_within_rounding_bound(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    a = synth.make_fp8_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, seed=4000 + Nq + Nk + d)
    announce(f"fwd_fp8 gauss {shape}")
    o, lse = run_fp8(gpu_lib, a)
    o_ref, lse_ref = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                                   a.scale, causal)
    bound = F.p_rounding_bound(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                               a.scale, causal, ACC_EPS)
    E = F.score_error(a.q, a.k, a.descale_q, a.descale_k, a.scale, causal, ACC_EPS)
    check_bounded(o, lse, o_ref, lse_ref, bound, E, vmax(a), f"gauss{shape}")


def test_sharp_scores_move_the_base(gpu_lib):
    """Scores spread over many units of log2: the running base moves often (the lazy
    rescale) and most weights underflow; still inside the rounding bound."""
    a = synth.make_fp8_inputs(1, 2, 1, 400, 400, 128, causal=True, seed=41)
    announce("fwd_fp8 sharp scores")
    scale = 8.0 / math.sqrt(128)
    o, lse = run_fp8(gpu_lib, a, scale=scale)
    o_ref, lse_ref = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                                   scale, True)
    bound = F.p_rounding_bound(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                               scale, True, ACC_EPS)
    E = F.score_error(a.q, a.k, a.descale_q, a.descale_k, scale, True, ACC_EPS)
    # few keys carry each row here, so their rounding errors do not average out
    check_bounded(o, lse, o_ref, lse_ref, bound, E, vmax(a), "sharp", mean_check=False)


def test_deterministic(gpu_lib):
    import torch
    a = synth.make_fp8_inputs(1, 4, 2, 600, 600, 128, causal=True, seed=42)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    q, k, v = dev(a.q), dev(a.k), dev(a.v)
    o1, l1 = gpu_lib.fwd_fp8(q, k, v, a.descale_q, a.descale_k, a.descale_v, causal=True)
    o2, l2 = gpu_lib.fwd_fp8(q.view(torch.float8_e4m3fn), k.view(torch.float8_e4m3fn),
                             v.view(torch.float8_e4m3fn), a.descale_q, a.descale_k,
                             a.descale_v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


# the shapes of the bf16 causal forward workloads at d = 128, in FP8
FULL = [("B4H32N4096d128", dict(B=4, Hq=32, Hkv=32, Nq=4096, Nk=4096, d=128)),
        ("B1H8N32768d128", dict(B=1, Hq=8, Hkv=8, Nq=32768, Nk=32768, d=128))]


@pytest.mark.parametrize("name,shape", FULL)
@pytest.mark.parametrize("kind", ["signs", "gauss"])
def test_full_size_sampled_rows(gpu_lib, name, shape, kind):
    import torch
    a = synth.make_fp8_inputs(**shape, causal=True, seed=5000 + shape["Nq"], kind=kind)
    announce(f"full-size fwd_fp8 {name} {kind}")
    o, lse = run_fp8(gpu_lib, a)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    vm = vmax(a)
    rng = np.random.default_rng(6)
    for _ in range(3):
        b, h = int(rng.integers(a.B)), int(rng.integers(a.Hq))
        rows = np.unique(np.concatenate([[0, a.Nq - 1], rng.integers(0, a.Nq, 20)]))
        args = (a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v, a.scale, True, b, h, rows)
        o_ref, lse_ref = F.forward_fp8_rows(*args)
        what = f"{name} {kind} b{b} h{h}"
        if kind == "signs":
            check_exact_weights(o[b, h, rows], lse[b, h, rows], o_ref, lse_ref, vm, what)
        else:
            bound = F.p_rounding_bound_rows(*args, acc_eps=ACC_EPS)
            E = F.score_error_rows(a.q, a.k, a.descale_q, a.descale_k, a.scale, True, b, h,
                                   rows, ACC_EPS)
            check_bounded(o[b, h, rows], lse[b, h, rows], o_ref, lse_ref, bound, E, vm, what)
    del a
    torch.cuda.empty_cache()
