"""The seeded input generator: determinism and bf16 rounding (against torch's cast)."""
import numpy as np
import pytest

from exact_tiled_attention_36_amd import synth


def test_bf16_rne_matches_torch_cast():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32) * 7,
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, 65504.0,
                  1.00390625, 1.01171875, 1.0078125], dtype=np.float32),
        # exact ties: mantissa low half 0x8000 (even and odd upper halves)
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    mine = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    back = synth.bf16_bits_to_f32(mine)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeded_and_ordered():
    a = synth.make_inputs(1, 2, 1, 5, 7, 8, causal=True, seed=9, with_do=True)
    b = synth.make_inputs(1, 2, 1, 5, 7, 8, causal=True, seed=9, with_do=True)
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(getattr(a, n), getattr(b, n))
    # draw order Q, K, V, dO from one generator
    r = np.random.default_rng(9)
    q = r.standard_normal((1, 2, 5, 8), dtype=np.float32)
    k = r.standard_normal((1, 1, 7, 8), dtype=np.float32)
    np.testing.assert_array_equal(a.k, synth.f32_to_bf16_bits(k))
    np.testing.assert_array_equal(a.q, synth.f32_to_bf16_bits(q))
    assert a.scale == pytest.approx(1 / np.sqrt(8))


def test_power_of_two_q_multiplier_commutes_with_rounding():
    a = synth.make_inputs(1, 1, 1, 64, 8, 16, causal=False, seed=3, q_mult=4.0)
    b = synth.make_inputs(1, 1, 1, 64, 8, 16, causal=False, seed=3)
    np.testing.assert_array_equal(a.as_f64("q"), 4.0 * b.as_f64("q"))
    with pytest.raises(ValueError):
        synth.make_inputs(1, 1, 1, 4, 4, 16, causal=False, seed=3, q_mult=3.0)


def test_workload_table_shapes():
    w = synth.WORKLOADS
    assert w["c5_bf16_causal_gqa_B2Hq32Hkv8N8192d128"]["Hkv"] == 8
    assert w["c4b_bf16_decode_B8H8Nq1Nk32768d128"]["Nq"] == 1
    assert w["c1_f32_B1H1N256d64"]["dtype"] == "f32"
