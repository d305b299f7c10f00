"""The matrix-core rate probe (fa_mfma_probe) runs through the C ABI and its products
are real: zero operands give exactly zero, normal-like operands give finite sums."""
import pytest

pytestmark = pytest.mark.gpu


def test_mfma_probe_outputs(gpu_lib):
    import torch
    flop, out = gpu_lib.mfma_probe(64, 3, "zeros")
    torch.cuda.synchronize()
    assert flop == 64 * 4 * 3 * 16 * 32768
    assert out.shape == (64 * 256,) and bool((out == 0).all())
    _, out = gpu_lib.mfma_probe(64, 3, "normal_bf16")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and float(out.abs().max()) > 0.0
