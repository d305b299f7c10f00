"""Pins of the oracle's FP8 pieces against facts that do not come from the oracle.

* E4M3 decoding: torch's float8_e4m3fn conversion (a library routine) on all 256
  codes, and the format's defining values (largest finite 448, smallest subnormal
  2^-9, NaN codes).
* The FP8 reference: torch's CPU float64 attention on the decoded tensors, and the
  scale identities of the definition (descale_q and descale_k only multiply the
  scores, descale_v only the output).
* The weight-rounding bound: its two constants (2^-4 relative, 2^-10 absolute) are
  the largest errors of round-to-nearest E4M3 as torch's cast rounds; it covers a
  simulated FP8 forward (weights against any base up to 8 below the row max, rounded
  by torch's cast); and a two-key case reaches 93% of it, so it is not slack.
* The score-error bound: raising every score by its largest accumulation error moves
  lse by between half of E and E.
* Planted mistakes in copies of the decoder (exponent bias, mantissa scale, subnormal
  scale), the bound (relative constant, absolute floor, signed V) and the score error
  (4x too small or too large) each fail one of these pins.
"""
import math

import numpy as np
import pytest

from exact_tiled_attention_36_amd import synth
from oracle import fp8 as F

torch = pytest.importorskip("torch")


def torch_round_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn).double().numpy()


def test_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = F.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_decode_defining_values():
    v = F.e4m3_to_f64(np.array([0x38, 0x7E, 0x01, 0x07, 0x08, 0xB8, 0x80, 0x00, 0x7F, 0xFF],
                               dtype=np.uint8))
    assert v[0] == 1.0 and v[1] == 448.0
    assert v[2] == 2.0 ** -9 and v[3] == 7 * 2.0 ** -9 and v[4] == 2.0 ** -6
    assert v[5] == -1.0 and v[6] == 0.0 and math.copysign(1, v[6]) < 0 and v[7] == 0.0
    assert np.isnan(v[8]) and np.isnan(v[9])
    finite = F.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.nanmax(finite) == 448.0 and np.sum(np.isnan(finite)) == 2


@pytest.mark.parametrize("causal", [False, True])
def test_forward_fp8_matches_torch_sdpa(causal):
    a = synth.make_fp8_inputs(2, 4, 2, 33, 33, 64, causal=causal, seed=11)
    o, lse = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                           a.scale, causal)
    deq = lambda c, s: torch.from_numpy(c).view(torch.float8_e4m3fn).double() * s
    q, k, v = deq(a.q, a.descale_q), deq(a.k, a.descale_k), deq(a.v, a.descale_v)
    k = k.repeat_interleave(2, dim=1)
    v = v.repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal,
                                                           scale=a.scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = (q @ k.transpose(-1, -2)) * a.scale
    if causal:
        s = s.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_descale_identities():
    a = synth.make_fp8_inputs(1, 2, 1, 20, 27, 64, causal=True, seed=12)
    o1, l1 = F.forward_fp8(a.q, a.k, a.v, 0.5, 3.0, 1.0, 0.2, True)
    o2, l2 = F.forward_fp8(a.q, a.k, a.v, 1.0, 1.0, 1.0, 0.2 * 0.5 * 3.0, True)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)
    o3, l3 = F.forward_fp8(a.q, a.k, a.v, 0.5, 3.0, 0.25, 0.2, True)
    np.testing.assert_allclose(o3, 0.25 * o1, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(l3, l1)


def test_rounding_constants_are_the_largest_e4m3_errors():
    r = np.random.default_rng(5)
    w = np.exp2(r.uniform(-16, 8, 400000))
    err = np.abs(torch_round_e4m3(w) - w)
    ratio = err / np.maximum(w / 16.0, 2.0 ** -10)
    assert ratio.max() <= 1.0
    # each constant is (nearly) reached on its own range: among normals the largest
    # relative error is 1/17 (a midpoint 1 + 1/16 above a power of two), 94% of 1/16;
    # among subnormals the largest absolute error is 2^-10
    normal = w >= 2.0 ** -6
    assert (err[normal] / (w[normal] / 16.0)).max() >= 0.93
    assert (err[~normal] / 2.0 ** -10).max() >= 0.99


def simulate_fp8_forward(a, base_drop):
    """Softmax weights 2^(s log2 e - m) against a base m = rowmax - base_drop (log2
    units, base_drop in [0, 8]), rounded to E4M3 by torch's cast, summed unrounded."""
    q = F.dequantize(a.q, a.descale_q)
    k = F.dequantize(a.k, a.descale_k)
    v = F.dequantize(a.v, a.descale_v)
    g = a.Hq // a.Hkv
    out = np.zeros(q.shape)
    for b in range(a.B):
        for h in range(a.Hq):
            s = a.scale * (q[b, h] @ k[b, h // g].T) * math.log2(math.e)
            if a.causal:
                i = np.arange(a.Nq)[:, None]
                j = np.arange(a.Nk)[None, :]
                s = np.where(j <= i + a.Nk - a.Nq, s, -np.inf)
            m = s.max(axis=1, keepdims=True) - base_drop[b, h][:, None]
            w = np.exp2(s - m)
            out[b, h] = (torch_round_e4m3(w) @ v[b, h // g]) / w.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("seed,causal", [(21, False), (22, True)])
def test_bound_covers_simulated_rounding(seed, causal):
    a = synth.make_fp8_inputs(1, 2, 1, 70, 70, 64, causal=causal, seed=seed)
    o, _ = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v, a.scale,
                         causal)
    bound = F.p_rounding_bound(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                               a.scale, causal)
    r = np.random.default_rng(seed)
    for drop in (np.zeros((1, 2, 70)), r.uniform(0, 8, (1, 2, 70)), np.full((1, 2, 70), 8.0)):
        sim = simulate_fp8_forward(a, drop)
        assert np.all(np.abs(sim - o) <= bound * (1 + 1e-9) + 1e-15)
    # the sampled rows of one head agree with the whole-tensor bound
    rows = np.array([0, 5, 69])
    np.testing.assert_allclose(
        F.p_rounding_bound_rows(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                                a.scale, causal, 0, 1, rows), bound[0, 1, rows], rtol=1e-14)


def test_bound_is_nearly_reached():
    # one query, two keys: weights 1 and w1 = 0.53125 - 2^-12 (just below the midpoint
    # of 0.5 and 0.5625, so it rounds down by almost w1 / 17); v = (0, 1)
    w1 = 0.53125 - 2.0 ** -12
    one = synth.f64_to_e4m3_bits(np.array([1.0]))[0]
    mone = synth.f64_to_e4m3_bits(np.array([-1.0]))[0]
    q8 = np.zeros((1, 1, 1, 4), np.uint8)
    q8[..., 0] = one
    k8 = np.zeros((1, 1, 2, 4), np.uint8)
    k8[0, 0, 1, 0] = mone
    v8 = np.zeros((1, 1, 2, 4), np.uint8)
    v8[0, 0, 1, :] = one
    scale = -math.log(w1)  # scores 0 and -scale: weights 1 and w1
    o, _ = F.forward_fp8(q8, k8, v8, 1.0, 1.0, 1.0, scale, False)
    bound = F.p_rounding_bound(q8, k8, v8, 1.0, 1.0, 1.0, scale, False)
    w = np.array([1.0, w1])
    sim = (torch_round_e4m3(w) @ np.array([0.0, 1.0])) / w.sum()
    err = abs(sim - o[0, 0, 0, 0])
    assert err <= bound[0, 0, 0, 0]
    assert err >= 0.93 * bound[0, 0, 0, 0]


def test_signs_inputs_make_exact_power_of_two_weights():
    a = synth.make_fp8_inputs(1, 2, 1, 40, 50, 64, causal=False, seed=31, kind="signs")
    q = F.dequantize(a.q, a.descale_q)
    k = F.dequantize(a.k, a.descale_k)
    s = q[0, 0] @ k[0, 0].T
    assert np.all(s == np.rint(s)) and s.min() >= -4 and s.max() <= 4
    assert abs(a.scale * math.log2(math.e) - 1.0) < 1e-7
    # every weight 2^(s - m) with the base m anywhere from max-8 to max is exact in E4M3
    for m in (s.max(), s.max() - 8):
        w = np.exp2(s - m)
        np.testing.assert_array_equal(torch_round_e4m3(w), w)


def test_synth_e4m3_encoder_matches_torch_cast():
    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(100000) * 60, r.standard_normal(100000) * 0.01,
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -11, 1.0625,
                         1.1875, 2.0 ** -6 * (1 - 1 / 32)]])
    x = np.clip(x, -448, 448)
    np.testing.assert_array_equal(
        synth.f64_to_e4m3_bits(x),
        torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    with pytest.raises(ValueError):
        synth.f64_to_e4m3_bits(np.array([449.0]))


@pytest.mark.parametrize("causal", [False, True])
def test_bound_covers_score_errors_and_rounding(causal):
    """Scores perturbed by up to acc_eps * scale * sum_d |q_d k_d| (random and worst-case
    signs), weights then rounded to E4M3: O stays within p_rounding_bound(acc_eps) and
    lse within score_error."""
    eps = 2.0 ** -8
    a = synth.make_fp8_inputs(1, 2, 1, 60, 60, 64, causal=causal, seed=23)
    q = F.dequantize(a.q, a.descale_q)
    k = F.dequantize(a.k, a.descale_k)
    v = F.dequantize(a.v, a.descale_v)
    o, lse = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v, a.scale,
                           causal)
    bound = F.p_rounding_bound(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                               a.scale, causal, acc_eps=eps)
    E = F.score_error(a.q, a.k, a.descale_q, a.descale_k, a.scale, causal, eps)
    assert np.all(bound >= F.p_rounding_bound(a.q, a.k, a.v, a.descale_q, a.descale_k,
                                              a.descale_v, a.scale, causal))
    r = np.random.default_rng(4)
    i = np.arange(60)[:, None]
    j = np.arange(60)[None, :]
    vis = (j <= i) if causal else np.ones((60, 60), bool)
    for trial in range(4):
        for h in range(2):
            s = a.scale * (q[0, h] @ k[0, 0].T)
            emax = eps * a.scale * (np.abs(q[0, h]) @ np.abs(k[0, 0]).T)
            if trial == 0:
                delta = r.uniform(-1, 1, s.shape) * emax
            else:  # push the largest scores up and the rest down (or the reverse)
                sign = np.where(s >= np.median(s, axis=1, keepdims=True), 1.0, -1.0)
                delta = (sign if trial % 2 else -sign) * emax
            sp = np.where(vis, s + delta, -np.inf)
            m = sp.max(axis=1, keepdims=True)
            w = np.exp(sp - m)
            lse_sim = m[:, 0] + np.log(w.sum(axis=1))
            o_sim = (torch_round_e4m3(w) @ v[0, 0]) / w.sum(axis=1, keepdims=True)
            assert np.all(np.abs(lse_sim - lse[0, h]) <= E[0, h] * (1 + 1e-9) + 1e-12)
            assert np.all(np.abs(o_sim - o[0, h]) <= bound[0, h] * (1 + 1e-9) + 1e-12)
    rows = np.array([3, 59])
    np.testing.assert_allclose(
        F.score_error_rows(a.q, a.k, a.descale_q, a.descale_k, a.scale, causal, 0, 1, rows,
                           eps), E[0, 1, rows], rtol=1e-14)


# ----------------------------------------------------------------------------------
# planted mistakes in copies of the FP8 oracle: each must fail one of the pins above
# (restated here as functions of the code under test)
# ----------------------------------------------------------------------------------

def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _mut_decode(kind):
    def dec(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = c & 0x7
        bias = 8 if kind == "bias8" else 7
        mden = 16.0 if kind == "mant16" else 8.0
        sub_exp = -10 if kind == "sub_scale" else -9
        normal = sign * np.ldexp(1.0 + m / mden, e - bias)
        sub = sign * np.ldexp(m.astype(np.float64), sub_exp)
        val = np.where(e == 0, sub, normal)
        return np.where((c & 0x7F) == 0x7F, np.nan, val)
    return dec


def pin_decoder(dec):
    codes = np.arange(256, dtype=np.uint8)
    mine = dec(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[ok], ref[ok])


def _mut_bound(kind):
    """p_rounding_bound with one planted mistake (float64, whole tensors)."""
    def bound(q8, k8, v8, dq, dk, dv, scale, causal, acc_eps=0.0):
        from oracle import attention as A
        q, k, v = F.dequantize(q8, dq), F.dequantize(k8, dk), F.dequantize(v8, dv)
        B, Hq, Nq, _ = q.shape
        g = Hq // k.shape[1]
        out = np.zeros(q.shape[:3] + (v.shape[3],))
        u = 1 / 32 if kind == "u32" else 1 / 16
        floor = 2.0 ** -14 if kind == "floor_small" else 2.0 ** -10
        for b in range(B):
            for h in range(Hq):
                rows = np.arange(Nq)
                s = A.scores(q[b, h], k[b, h // g], scale, rows, Nq, causal)
                p = A.softmax_rows(s)[0]
                pmax = p.max(axis=1, keepdims=True)
                err = np.where(p > 0, np.maximum(p * u, floor * pmax), 0.0)
                vv = v[b, h // g] if kind == "signed_v" else np.abs(v[b, h // g])
                mag = np.abs(q[b, h]) @ np.abs(k[b, h // g]).T
                mag = np.where(A.visible(rows, Nq, k.shape[2], causal), mag, 0.0)
                E = acc_eps * scale * mag.max(axis=1)
                grow = np.exp(2 * E)[:, None]
                out[b, h] = grow * (err @ vv) + (grow - 1) * (p @ np.abs(v[b, h // g]))
        return out
    return bound


def pin_bound_covers(bound):
    """Simulated FP8 forwards (bases 0 and 8 below the row max, E4M3 rounding by
    torch's cast; sharp scores where most weights are subnormal; perturbed scores)
    stay within the bound."""
    for seed, causal, mult in ((21, False, 1.0), (22, True, 1.0), (24, False, 6.0)):
        a = synth.make_fp8_inputs(1, 2, 1, 70, 70, 64, causal=causal, seed=seed)
        sc = a.scale * mult
        o, _ = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v, sc, causal)
        bd = bound(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v, sc, causal)
        aa = synth.Fp8Inputs(a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d, causal, sc, a.seed, a.kind,
                             a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v)
        for drop in (np.zeros((1, 2, 70)), np.full((1, 2, 70), 8.0)):
            sim = simulate_fp8_forward(aa, drop)
            assert np.all(np.abs(sim - o) <= bd * (1 + 1e-9) + 1e-15)
    eps = 2.0 ** -8
    a = synth.make_fp8_inputs(1, 1, 1, 60, 60, 64, causal=False, seed=23)
    q, k, v = (F.dequantize(x, s) for x, s in ((a.q, a.descale_q), (a.k, a.descale_k),
                                               (a.v, a.descale_v)))
    o, _ = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v, a.scale, False)
    bd = bound(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v, a.scale, False, eps)
    s = a.scale * (q[0, 0] @ k[0, 0].T)
    emax = eps * a.scale * (np.abs(q[0, 0]) @ np.abs(k[0, 0]).T)
    sign = np.where(s >= np.median(s, axis=1, keepdims=True), 1.0, -1.0)
    for sg in (sign, -sign):
        sp = s + sg * emax
        w = np.exp(sp - sp.max(axis=1, keepdims=True))
        sim = (torch_round_e4m3(w) @ v[0, 0]) / w.sum(axis=1, keepdims=True)
        assert np.all(np.abs(sim - o[0, 0]) <= bd[0, 0] * (1 + 1e-9) + 1e-12)


def pin_score_error(score_error):
    """All scores raised by their largest accumulation error move lse by a weighted mean
    of those errors: at most E_i, and (the errors of one row's keys differ little) at
    least half of it."""
    eps = 2.0 ** -8
    for causal in (False, True):
        a = synth.make_fp8_inputs(1, 2, 1, 50, 50, 64, causal=causal, seed=25)
        q, k = F.dequantize(a.q, a.descale_q), F.dequantize(a.k, a.descale_k)
        _, lse = F.forward_fp8(a.q, a.k, a.v, a.descale_q, a.descale_k, a.descale_v,
                               a.scale, causal)
        E = score_error(a.q, a.k, a.descale_q, a.descale_k, a.scale, causal, eps)
        for h in range(2):
            s = a.scale * (q[0, h] @ k[0, 0].T)
            emax = eps * a.scale * (np.abs(q[0, h]) @ np.abs(k[0, 0]).T)
            if causal:
                s = np.where(np.tri(50, dtype=bool), s, -np.inf)
            sp = s + emax
            m = sp.max(axis=1, keepdims=True)
            lse_up = m[:, 0] + np.log(np.exp(sp - m).sum(axis=1))
            shift = lse_up - lse[0, h]
            assert np.all(shift <= E[0, h] * (1 + 1e-9) + 1e-15)
            assert np.all(shift >= 0.5 * E[0, h])


def test_pins_accept_the_oracle():
    pin_decoder(F.e4m3_to_f64)
    pin_bound_covers(F.p_rounding_bound)
    pin_score_error(F.score_error)


@pytest.mark.parametrize("kind", ["bias8", "mant16", "sub_scale"])
def test_planted_decoder_mistakes_are_caught(kind):
    assert _fails(pin_decoder, _mut_decode(kind))


@pytest.mark.parametrize("kind", ["u32", "floor_small", "signed_v"])
def test_planted_bound_mistakes_are_caught(kind):
    assert _fails(pin_bound_covers, _mut_bound(kind))


@pytest.mark.parametrize("factor", [0.25, 4.0])
def test_planted_score_error_mistakes_are_caught(factor):
    def wrong(*args):
        return factor * F.score_error(*args)
    assert _fails(pin_score_error, wrong)
