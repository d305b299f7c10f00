"""The autograd entry point (scaled_dot_product_attention over fa_fwd / fa_bwd): same
numbers as the direct calls, gradients within the oracle's tolerances, and refusals
for what the library does not compute."""
import numpy as np
import pytest

from exact_tiled_attention_36_amd import synth
from oracle import attention as A
from gpu_util import (announce, assert_grad_close, assert_o_close, to_dev, to_host64)

pytestmark = pytest.mark.gpu


def run_autograd(inp, **kw):
    import torch
    from exact_tiled_attention_36_amd.autograd import scaled_dot_product_attention
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    o = scaled_dot_product_attention(q, k, v, is_causal=inp.causal, scale=inp.scale,
                                     enable_gqa=inp.Hq != inp.Hkv, **kw)
    o.backward(do)
    torch.cuda.synchronize()
    return q, k, v, do, o


@pytest.mark.parametrize("shape", [
    (1, 4, 4, 300, 300, 128, True),
    (2, 8, 2, 256, 256, 64, False),     # GQA
    (1, 4, 1, 129, 129, 128, True),     # MQA, ragged
])
def test_autograd_matches_direct_calls_and_oracle(gpu_lib, shape):
    import torch
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True, seed=4100 + Nq + Hq)
    announce(f"autograd {shape}")
    q, k, v, do, o = run_autograd(inp)
    # bitwise the same as the direct calls (same kernels, same arguments)
    o2, lse2 = gpu_lib.fwd(q.detach(), k.detach(), v.detach(), causal=causal, scale=inp.scale)
    dq2, dk2, dv2 = gpu_lib.bwd(q.detach(), k.detach(), v.detach(), o2, do, lse2,
                                causal=causal, scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    assert torch.equal(q.grad, dq2) and torch.equal(k.grad, dk2) and torch.equal(v.grad, dv2)
    # and within tolerance of the float64 oracle
    ro, _ = A.forward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.scale, causal)
    assert_o_close(to_host64(o), ro, "autograd O")
    rq, rk, rv, _ = A.backward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                               inp.as_f64("do"), inp.scale, causal)
    assert_grad_close(to_host64(q.grad), rq, "autograd dQ")
    assert_grad_close(to_host64(k.grad), rk, "autograd dK")
    assert_grad_close(to_host64(v.grad), rv, "autograd dV")


def test_autograd_default_scale_and_loss(gpu_lib):
    import torch
    from exact_tiled_attention_36_amd.autograd import scaled_dot_product_attention
    inp = synth.make_inputs(1, 2, 2, 64, 64, 64, causal=False, with_do=True, seed=4200)
    announce("autograd default scale")
    q, k, v = (to_dev(inp, n).requires_grad_(True) for n in ("q", "k", "v"))
    o = scaled_dot_product_attention(q, k, v)       # scale 1/sqrt(d), not causal
    loss = (o.float() * to_dev(inp, "do").float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    ro, _ = A.forward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), 1 / np.sqrt(64), False)
    assert_o_close(to_host64(o), ro, "default scale O")
    rq, _, _, _ = A.backward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                             inp.as_f64("do"), 1 / np.sqrt(64), False)
    assert_grad_close(to_host64(q.grad), rq, "default scale dQ")


def test_autograd_refusals(gpu_lib):
    import torch
    from exact_tiled_attention_36_amd.autograd import scaled_dot_product_attention
    q = torch.zeros(1, 4, 8, 64, device="cuda", dtype=torch.bfloat16)
    kv = torch.zeros(1, 2, 8, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        scaled_dot_product_attention(q, q, q, attn_mask=torch.zeros(8, 8, device="cuda"))
    with pytest.raises(NotImplementedError):
        scaled_dot_product_attention(q, q, q, dropout_p=0.1)
    with pytest.raises(ValueError):
        scaled_dot_product_attention(q, kv, kv)          # GQA needs enable_gqa=True
    with pytest.raises(ValueError):
        scaled_dot_product_attention(q.half(), q.half(), q.half())   # fp16 not taken
    qf = torch.zeros(1, 2, 8, 64, device="cuda", dtype=torch.float32, requires_grad=True)
    o = scaled_dot_product_attention(qf, qf, qf)      # fp32 forward works
    with pytest.raises(NotImplementedError):
        o.sum().backward()                             # fp32 backward does not exist
