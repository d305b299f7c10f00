"""Race check: the debug build (libfa_sync.so, FA_DEBUG_BARRIERS=1) adds, in every key
or query step of every tiled kernel, a wait for the step's copies and a workgroup
barrier. Barriers only change timing, so its outputs must equal the normal build's
bit for bit; a difference would mean an LDS access that the kernels' own waits and
barriers do not order."""
import os

import numpy as np
import pytest

from exact_tiled_attention_36_amd import build as B
from exact_tiled_attention_36_amd import fa, synth
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (2, 32, 8, 1000, 1000, 128, True),    # 4-wave forward and dQ, dK/dV
    (1, 24, 24, 4200, 4300, 128, True),   # 8-wave forward
    (1, 8, 2, 700, 900, 128, True),       # small-grid forward (key split) and dQ, split dK/dV
    (1, 4, 4, 300, 130, 64, False),       # key-split forward, odd key-tile count
    (2, 16, 16, 1024, 1024, 64, False),
    (1, 8, 2, 520, 520, 256, True),       # 4-wave d = 256 forward
    (1, 32, 8, 2100, 2000, 256, False),   # two-group d = 256 forward
    (1, 32, 16, 8200, 8200, 128, True),   # two-group d = 128 forward, head pairs
    (2, 32, 8, 2100, 2200, 128, True),    # 4-wave d = 128 forward, head pairs
    (1, 32, 32, 8200, 8200, 128, True),   # two-group d = 128 forward, 64 rows per wave
]


def _run(inp, fp8):
    import torch
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=inp.causal, scale=inp.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=inp.causal, scale=inp.scale)
    outs = [o, lse, dq, dk, dv]
    if fp8:
        q8, k8, v8 = ((t.float() * 8).to(torch.float8_e4m3fn) for t in (q, k, v))
        outs += list(fa.fwd_fp8(q8, k8, v8, 0.125, 0.125, 0.125, causal=inp.causal,
                                scale=inp.scale))
    torch.cuda.synchronize()
    return [t.detach().view(torch.int16) if t.dtype == torch.bfloat16 else t.detach()
            for t in outs]


@pytest.mark.parametrize("shape", SHAPES)
def test_debug_barriers_bitwise_equal(gpu_lib, shape):
    import torch
    if not os.path.exists(B.SYNC_LIB):
        pytest.fail(f"{B.SYNC_LIB} is not built (run __graft_entry__.build())")
    Bz, Hq, Hkv, Nq, Nk, d, causal = shape
    inp = synth.make_inputs(Bz, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True,
                            seed=4100 + Nq + d)
    announce(f"debug barriers {shape}")
    try:
        fa.load(B.LIB)
        ref = _run(inp, fp8=d != 64)
        fa.load(B.SYNC_LIB)
        got = _run(inp, fp8=d != 64)
    finally:
        fa.load(B.LIB)
    names = ["o", "lse", "dq", "dk", "dv", "o_fp8", "lse_fp8"]
    for n, a, b in zip(names, ref, got):
        assert torch.equal(a, b), f"{shape}: {n} differs between the normal and debug builds"
    assert np.isfinite(got[1].cpu().numpy()).all()
