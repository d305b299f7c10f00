"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each check names what fixes the expected value: a closed form, an invariant of the
definition, brute force with Python scalars, central finite differences, the pages'
own block recurrences, or torch's CPU float64 attention (a library routine the
pages call, "FlashAttention" (ruizhehou.github.io), §五). The mutation tests at the
bottom plant plausible mistakes into a copy of the oracle and show that some pin
here fails for each.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import online, scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def problem(B, Hq, Hkv, Nq, Nk, d, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, Nq, d))
    k = r.standard_normal((B, Hkv, Nk, d))
    v = r.standard_normal((B, Hkv, Nk, d))
    do = r.standard_normal((B, Hq, Nq, d))
    return q, k, v, do


# ----------------------------------------------------------------------------------
# pin functions (take the forward/backward under test so mutations can reuse them)
# ----------------------------------------------------------------------------------

def pin_rows_sum_to_one(probs):
    q, k, _, _ = problem(2, 4, 2, 9, 13, 8, 1)
    for causal in (False, True):
        p = probs(q, k, 0.37, causal)
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)


def pin_identical_keys(fwd):
    """All keys equal: uniform weights over the visible keys.

    Non-causal: o_i = mean_j v_j, lse_i = s_i + ln Nk.
    Causal (bottom-right): o_i = mean of v_0..v_{i+Nk-Nq}, lse_i = s_i + ln(i+Nk-Nq+1).
    """
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 5, 11, 6
    q, k, v, _ = problem(B, Hq, Hkv, Nq, Nk, d, 2)
    k[:] = k[:, :, :1, :]
    sc = 0.5
    o, lse = fwd(q, k, v, sc, False)
    s = sc * np.einsum("bhid,bd->bhi", q, k[:, 0, 0, :])
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               atol=1e-13)
    np.testing.assert_allclose(lse, s + math.log(Nk), atol=1e-13)
    o, lse = fwd(q, k, v, sc, True)
    for i in range(Nq):
        last = i + Nk - Nq
        want = np.broadcast_to(v[:, 0, : last + 1].mean(axis=1)[:, None], o[:, :, i].shape)
        np.testing.assert_allclose(o[:, :, i], want, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], s[:, :, i] + math.log(last + 1), atol=1e-13)


def pin_dominant_logit(fwd):
    """One logit exceeds every other in its row by delta: o_i is within
    (Nk-1) e^-delta max|v| of that key's value row (closed-form bound)."""
    Nk, d, delta = 20, 4, 30.0
    r = np.random.default_rng(3)
    k = np.zeros((1, 1, Nk, d))
    k[0, 0, :, 0] = r.uniform(-1, 1, Nk)
    jstar = 7
    k[0, 0, jstar, 0] = 1.0 + delta + 1.0
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    v = r.standard_normal((1, 1, Nk, d))
    o, lse = fwd(q, k, v, 1.0, False)
    bound = (Nk - 1) * math.exp(-delta) * np.abs(v).max()
    assert np.abs(o[0, 0, 0] - v[0, 0, jstar]).max() <= bound
    assert abs(lse[0, 0, 0] - k[0, 0, jstar, 0]) <= (Nk - 1) * math.exp(-delta)


def pin_brute_force(fwd):
    for (B, Hq, Hkv, Nq, Nk, d, causal, seed) in [
        (1, 1, 1, 7, 7, 5, False, 10), (2, 4, 2, 6, 9, 3, True, 11),
        (1, 3, 1, 16, 16, 8, True, 12), (1, 2, 2, 9, 4, 4, True, 13),
        (1, 2, 1, 1, 12, 6, True, 14), (1, 1, 1, 16, 3, 2, False, 15),
    ]:
        q, k, v, _ = problem(B, Hq, Hkv, Nq, Nk, d, seed)
        sc = 1.0 / math.sqrt(d)
        o, lse = fwd(q, k, v, sc, causal)
        ob, lb = scalar.forward(q.tolist(), k.tolist(), v.tolist(), sc, causal)
        np.testing.assert_allclose(o, np.array(ob), atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse, np.array(lb), atol=1e-13, rtol=0)


def _loss(fwd, q, k, v, do, sc, causal):
    return float((fwd(q, k, v, sc, causal)[0] * do).sum())


def pin_finite_differences(fwd, bwd):
    """Central differences of L = sum(dO * O) in float64 (h = 1e-5)."""
    for (B, Hq, Hkv, Nq, Nk, d, causal, seed) in [
        (1, 2, 1, 5, 7, 3, True, 20), (1, 2, 2, 6, 6, 4, False, 21),
    ]:
        q, k, v, do = problem(B, Hq, Hkv, Nq, Nk, d, seed)
        sc = 0.6
        dq, dk, dv, _ = bwd(q, k, v, do, sc, causal)
        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                old = x[idx]
                x[idx] = old + h
                lp = _loss(fwd, q, k, v, do, sc, causal)
                x[idx] = old - h
                lm = _loss(fwd, q, k, v, do, sc, causal)
                x[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(g, num, atol=1e-8, rtol=1e-6, err_msg=name)


def pin_recurrences(fwd):
    """The pages' online recurrences equal the one-shot softmax for every block size."""
    r = np.random.default_rng(4)
    N, d = 33, 5
    q = r.standard_normal((N, d)) * 3
    k = r.standard_normal((N, d))
    v = r.standard_normal((N, d))
    sc = 0.8
    for causal in (False, True):
        o_ref, l_ref = fwd(q[None, None], k[None, None], v[None, None], sc, causal)
        o_ref, l_ref = o_ref[0, 0], l_ref[0, 0]
        for bk in range(1, N + 1):
            o1, l1 = online.online_v1(q, k, v, sc, bk, causal)
            np.testing.assert_allclose(o1, o_ref, atol=1e-12, rtol=0)
            np.testing.assert_allclose(l1, l_ref, atol=1e-12, rtol=0)
            for bq in (1, 4, 7, N):
                o2, l2 = online.online_v2(q, k, v, sc, bq, bk, causal)
                np.testing.assert_allclose(o2, o_ref, atol=1e-12, rtol=0)
                np.testing.assert_allclose(l2, l_ref, atol=1e-12, rtol=0)
    # the FlashAttention1 article's case: all query rows in one block, scale 1/sqrt(d_k)
    o_ref = fwd(q[None, None], k[None, None], v[None, None], 1 / math.sqrt(d), False)[0][0, 0]
    for bs in range(1, N + 1):
        o_pg, _ = online.online_v2(q, k, v, 1 / math.sqrt(d), N, bs)
        np.testing.assert_allclose(o_pg, o_ref, atol=1e-12, rtol=0)


def pin_torch_sdpa(fwd, bwd):
    """torch.nn.functional.scaled_dot_product_attention on CPU in float64."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    for (B, Hq, Hkv, N, d, causal, seed) in [
        (2, 4, 4, 19, 8, False, 30), (1, 6, 2, 23, 16, True, 31), (1, 2, 1, 40, 4, True, 32),
    ]:
        q, k, v, do = problem(B, Hq, Hkv, N, N, d, seed)
        sc = 1.0 / math.sqrt(d)
        g = Hq // Hkv
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        o_t = F.scaled_dot_product_attention(
            tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1),
            attn_mask=None, dropout_p=0.0, is_causal=causal, scale=sc)
        o_t.backward(torch.tensor(do))
        o, _ = fwd(q, k, v, sc, causal)
        np.testing.assert_allclose(o, o_t.detach().numpy(), atol=1e-12, rtol=0)
        dq, dk, dv, _ = bwd(q, k, v, do, sc, causal)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11, rtol=0)


# ----------------------------------------------------------------------------------
# the pins applied to the oracle
# ----------------------------------------------------------------------------------

def test_rows_sum_to_one():
    pin_rows_sum_to_one(A.probabilities)


def test_identical_keys_closed_form():
    pin_identical_keys(A.forward)


def test_dominant_logit_bound():
    pin_dominant_logit(A.forward)


def test_brute_force_scalar_loops():
    pin_brute_force(A.forward)


def test_backward_finite_differences():
    pin_finite_differences(A.forward, A.backward)


def test_online_recurrences_every_block_size():
    pin_recurrences(A.forward)


def test_torch_float64_sdpa_and_autograd():
    pin_torch_sdpa(A.forward, A.backward)


def test_tiny_closed_form_logits_ln123():
    """Logits 0, ln 2, ln 3 give weights 1/6, 2/6, 3/6 (safe softmax, "FlashAttention"
    (ruizhehou.github.io), §二.2); a second query doubles them to 1, 4, 9 over 14.
    Causal bottom-right with Nq=2, Nk=3: row 0 sees keys 0..1 only."""
    q = np.array([[[[1.0], [2.0]]]])
    k = np.array([[[[0.0], [math.log(2)], [math.log(3)]]]])
    v = np.array([[[[6.0, 1.0], [0.0, 1.0], [12.0, 1.0]]]])
    o, lse = A.forward(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0, 0], [7.0, 1.0], atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], [114.0 / 14.0, 1.0], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [math.log(6), math.log(14)], atol=1e-14)
    o, lse = A.forward(q, k, v, 1.0, True)
    np.testing.assert_allclose(o[0, 0, 0], [2.0, 1.0], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(3), atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], [114.0 / 14.0, 1.0], atol=1e-14)


def test_invariants():
    q, k, v, do = problem(2, 4, 2, 12, 12, 6, 40)
    sc = 0.4
    o, lse = A.forward(q, k, v, sc, False)
    # per-row logit shift: K + 1 c^T changes s_i by a constant per row
    c = np.random.default_rng(41).standard_normal(6)
    o2, _ = A.forward(q, k + c, v, sc, False)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    # V + 1 b^T shifts every output row by b
    bvec = np.random.default_rng(42).standard_normal(6)
    o3, _ = A.forward(q, k, v + bvec, sc, False)
    np.testing.assert_allclose(o3, o + bvec, atol=1e-12)
    # permuting keys and values together (non-causal) leaves O unchanged
    perm = np.random.default_rng(43).permutation(12)
    o4, lse4 = A.forward(q, k[:, :, perm], v[:, :, perm], sc, False)
    np.testing.assert_allclose(o4, o, atol=1e-12)
    np.testing.assert_allclose(lse4, lse, atol=1e-12)
    # causal, Nq == Nk: the first row sees only key 0
    oc, lsec = A.forward(q, k, v, sc, True)
    np.testing.assert_allclose(oc[:, :, 0], np.repeat(v[:, :, 0], 2, axis=1), atol=1e-14)
    # causal with one query row (decode) sees every key: equals non-causal
    od, ld = A.forward(q[:, :, -1:], k, v, sc, True)
    on, ln_ = A.forward(q[:, :, -1:], k, v, sc, False)
    np.testing.assert_allclose(od, on, atol=0)
    np.testing.assert_allclose(ld, ln_, atol=0)
    # backward identities: D_i = sum_c dO_ic O_ic, and rows of dS sum to zero
    dq, dk, dv, D = A.backward(q, k, v, do, sc, True)
    oc, _ = A.forward(q, k, v, sc, True)
    np.testing.assert_allclose(D, (do * oc).sum(-1), atol=1e-12)
    p = A.probabilities(q, k, sc, True)
    dp = np.einsum("bhid,bhjd->bhij", do, np.repeat(v, 2, axis=1))
    ds = p * (dp - D[..., None])
    np.testing.assert_allclose(ds.sum(-1), 0.0, atol=1e-12)


def test_gqa_equals_repeated_mha():
    q, k, v, do = problem(1, 6, 2, 10, 14, 4, 50)
    g = 3
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    for causal in (False, True):
        o, lse = A.forward(q, k, v, 0.5, causal)
        o_m, lse_m = A.forward(q, kr, vr, 0.5, causal)
        np.testing.assert_allclose(o, o_m, atol=0)
        np.testing.assert_allclose(lse, lse_m, atol=0)
        dq, dk, dv, _ = A.backward(q, k, v, do, 0.5, causal)
        dq_m, dk_m, dv_m, _ = A.backward(q, kr, vr, do, 0.5, causal)
        np.testing.assert_allclose(dq, dq_m, atol=1e-13)
        np.testing.assert_allclose(dk, dk_m.reshape(1, 2, g, 14, 4).sum(2), atol=1e-13)
        np.testing.assert_allclose(dv, dv_m.reshape(1, 2, g, 14, 4).sum(2), atol=1e-13)
        # mapping h -> h // g, spelled out head by head
        for h in range(6):
            oh, _ = A.forward(q[:, h:h + 1], k[:, h // g:h // g + 1], v[:, h // g:h // g + 1],
                              0.5, causal)
            np.testing.assert_allclose(o[:, h:h + 1], oh, atol=0)


def test_merge_partials_equals_direct():
    """Split keys into chunks, attend to each, merge with LSE weights: same as direct."""
    q, k, v, _ = problem(2, 2, 2, 3, 50, 8, 60)
    sc = 0.3
    for causal in (False, True):
        o_ref, lse_ref = A.forward(q, k, v, sc, causal)
        for bounds in ([0, 50], [0, 7, 50], [0, 1, 2, 30, 49, 50], list(range(0, 51, 10))):
            os_, ls_ = [], []
            Nq, Nk = q.shape[2], k.shape[2]
            for a, b in zip(bounds[:-1], bounds[1:]):
                # a chunk of keys with the causal limit of the full sequence
                rows = np.arange(Nq)
                ob = np.zeros(q.shape)
                lb = np.zeros(q.shape[:3])
                for bb in range(2):
                    for h in range(2):
                        s = A.scores(q[bb, h], k[bb, h], sc, rows, Nq, causal)[:, a:b]
                        p, m, l = A.softmax_rows(s)
                        ob[bb, h] = p @ v[bb, h, a:b]
                        with np.errstate(divide="ignore"):
                            lb[bb, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1)),
                                                 -np.inf)
                os_.append(ob)
                ls_.append(lb)
            o, lse = A.merge_partials(np.stack(os_), np.stack(ls_))
            np.testing.assert_allclose(o, o_ref, atol=1e-13)
            np.testing.assert_allclose(lse, lse_ref, atol=1e-13)


def test_fully_masked_rows():
    """Causal with Nq > Nk: the first Nq - Nk rows see no key -> o = 0, lse = -inf."""
    q, k, v, _ = problem(1, 1, 1, 6, 3, 4, 70)
    o, lse = A.forward(q, k, v, 1.0, True)
    assert np.all(o[0, 0, :3] == 0) and np.all(np.isneginf(lse[0, 0, :3]))
    assert np.all(np.isfinite(lse[0, 0, 3:]))
    ob, lb = scalar.forward(q.tolist(), k.tolist(), v.tolist(), 1.0, True)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-14)


def test_pages_printed_figures():
    with open(os.path.join(GOLDEN, "pages_figures.json")) as f:
        g = json.load(f)
    s = g["score_matrix_bytes_n4096_fp16"]
    assert round(s["N"] * s["N"] * s["bytes_per_element"] / 2**20) == s["approx_megabytes"]
    h = g["accuracy_harness_shape"]
    from exact_tiled_attention_36_amd.synth import WORKLOADS
    c2 = WORKLOADS["c2_bf16_B2H16N1024d64"]
    assert (c2["B"], c2["Nq"], c2["d"]) == (h["batch"], h["seq_len"], h["d"])
    # the harness's block size of 256 gives the same result as the direct form
    q, k, v, _ = problem(1, 1, 1, 300, 300, 8, 80)
    o_ref = A.forward(q, k, v, 1 / math.sqrt(8), False)[0][0, 0]
    o_pg, _ = online.online_v2(q[0, 0], k[0, 0], v[0, 0], 1 / math.sqrt(8), 300,
                               h["block_size"])
    np.testing.assert_allclose(o_pg, o_ref, atol=1e-12)


def test_sampled_rows_match_full():
    q, k, v, _ = problem(1, 4, 2, 40, 40, 8, 90)
    o, lse = A.forward(q, k, v, 0.3, True)
    rows = np.array([0, 5, 39, 17])
    orow, lrow = A.forward_rows(q, k, v, 0.3, True, 0, 3, rows)
    np.testing.assert_array_equal(orow, o[0, 3, rows])
    np.testing.assert_array_equal(lrow, lse[0, 3, rows])


# ----------------------------------------------------------------------------------
# planted mistakes: each mutated oracle must fail at least one pin
# ----------------------------------------------------------------------------------

def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _mut_forward(kind):
    def fwd(q, k, v, scale, causal):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, Hq, Nq, d = q.shape
        Hkv, Nk = k.shape[1], k.shape[2]
        g = Hq // Hkv
        o = np.zeros(q.shape[:3] + (v.shape[3],))
        lse = np.zeros(q.shape[:3])
        for b in range(B):
            for h in range(Hq):
                kh = (h % Hkv) if kind == "gqa_modulo" else h // g
                sc = scale if kind != "no_scale" else 1.0
                s = sc * q[b, h] @ k[b, kh].T
                if causal:
                    i = np.arange(Nq)[:, None]
                    j = np.arange(Nk)[None, :]
                    lim = i if kind == "top_left" else i + (Nk - Nq)
                    s = np.where(j <= lim, s, -np.inf)
                m = s.max(1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(1, keepdims=True)
                vv = v[b, kh]
                o[b, h] = (e / l) @ (vv[::-1] if kind == "reversed_v" else vv)
                lse[b, h] = (m + np.log(l))[:, 0] + (1e-6 if kind == "lse_bias" else 0)
        return o, lse
    return fwd


def _mut_backward(kind):
    def bwd(q, k, v, do, scale, causal):
        dq, dk, dv, D = A.backward(q, k, v, do, scale, causal)
        if kind == "ds_sign":
            # recompute dq with (D - dP) instead of (dP - D)
            return -dq, -dk, dv, D
        if kind == "dk_no_scale":
            return dq, dk / scale, dv, D
        return dq, dk, dv, D
    return bwd


@pytest.mark.parametrize("kind", ["no_scale", "top_left", "reversed_v", "lse_bias"])
def test_planted_forward_mistakes_are_caught(kind):
    fwd = _mut_forward(kind)
    caught = (_fails(pin_identical_keys, fwd) or _fails(pin_brute_force, fwd)
              or _fails(pin_torch_sdpa, fwd, A.backward))
    assert caught, kind


def test_planted_gqa_mapping_mistake_is_caught():
    fwd = _mut_forward("gqa_modulo")
    assert _fails(pin_brute_force, fwd)


@pytest.mark.parametrize("kind", ["ds_sign", "dk_no_scale"])
def test_planted_backward_mistakes_are_caught(kind):
    assert _fails(pin_finite_differences, A.forward, _mut_backward(kind))
