"""fa_bwd_noalloc (the backward with the library's fixed scratch instead of a caller
workspace) against fa_bwd, whose kernels it shares: bit-identical gradients, on two
calls in a row, the second with a smaller problem, so the scratch holds the first
call's values when the second starts. Also one comparison with the float64 oracle."""
import numpy as np
import pytest

from exact_tiled_attention_36_amd import synth
from oracle import attention as A
from gpu_util import announce, assert_grad_close, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _run_pair(fa, inp):
    import torch
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=inp.causal, scale=inp.scale)
    ref = fa.bwd(q, k, v, o, do, lse, causal=inp.causal, scale=inp.scale)
    outs = [torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)]
    fa.bwd_noalloc(q, k, v, o, do, lse, *outs, causal=inp.causal, scale=inp.scale)
    torch.cuda.synchronize()
    return ref, outs


@pytest.mark.parametrize("first,second", [
    ((2, 8, 2, 1000, 1000, 128, True), (1, 4, 1, 300, 300, 128, True)),
    ((1, 16, 4, 2048, 2048, 64, False), (1, 2, 2, 77, 130, 256, True)),
])
def test_noalloc_matches_workspace_entry(gpu_lib, first, second):
    import torch
    for i, shape in enumerate((first, second)):
        B, Hq, Hkv, Nq, Nk, d, causal = shape
        announce(f"bwd_noalloc call {i} {shape}")
        inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True,
                                seed=5100 + 17 * i + Nq)
        ref, outs = _run_pair(gpu_lib, inp)
        for name, a, b in zip(("dq", "dk", "dv"), ref, outs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (shape, name)
        if i == 1:
            rq, rk, rv, _ = A.backward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                       inp.as_f64("do"), inp.scale, inp.causal)
            for name, got, want in zip(("dQ", "dK", "dV"), outs, (rq, rk, rv)):
                assert_grad_close(to_host64(got), want, f"noalloc {shape} {name}")


def test_noalloc_rejects_too_many_rows(gpu_lib):
    import torch
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, gpu_lib.BWD_NOALLOC_MAX_ROWS // 2 + 64, 64, 64
    t = torch.empty(16, device="cuda", dtype=torch.bfloat16)
    lib = gpu_lib.load()
    p = t.data_ptr()
    st = lib.fa_bwd_noalloc(p, p, p, p, p, p, p, p, p, B, Hq, Hkv, Nq, Nk, d, 0.125, 1,
                            torch.cuda.current_stream().cuda_stream)
    assert st == -13, gpu_lib.status_string(st)
