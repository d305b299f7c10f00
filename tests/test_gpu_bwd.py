"""GPU parity of the recompute backward (fa_bwd) against the float64 oracle."""
import numpy as np
import pytest

from exact_tiled_attention_36_amd import synth
from oracle import attention as A
from gpu_util import announce, assert_grad_close, to_dev, to_host64

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(fa, inp):
    import torch
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=inp.causal, scale=inp.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=inp.causal, scale=inp.scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(fa, inp, what):
    announce(f"bwd {what} B{inp.B} Hq{inp.Hq} Hkv{inp.Hkv} Nq{inp.Nq} Nk{inp.Nk} d{inp.d} "
             f"causal={inp.causal} seed={inp.seed}")
    dq, dk, dv = (to_host64(t) for t in gpu_fwd_bwd(fa, inp))
    rq, rk, rv, _ = A.backward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                               inp.as_f64("do"), inp.scale, inp.causal)
    assert_grad_close(dq, rq, f"{what} dQ")
    assert_grad_close(dk, rk, f"{what} dK")
    assert_grad_close(dv, rv, f"{what} dV")


SHAPES = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (2, 16, 16, 1024, 1024, 64, False),   # the small bf16 config's shape
    (1, 4, 4, 1024, 1024, 128, True),
    (1, 2, 2, 512, 512, 256, True),
    (1, 8, 2, 600, 600, 128, True),       # GQA, ragged
    (1, 4, 1, 300, 300, 64, True),        # MQA
    (1, 1, 1, 1, 1, 64, False), (1, 2, 1, 3, 3, 128, True), (1, 2, 2, 17, 17, 128, False),
    (1, 2, 2, 1000, 1000, 64, True),
    (1, 2, 1, 200, 77, 128, False), (1, 2, 2, 77, 300, 128, True),
    (1, 2, 1, 300, 100, 64, True),        # rows that see no key
    (1, 2, 2, 130, 260, 256, False),
]

# Head size 256 (the d = 256 dQ and dK/dV kernels): GQA and MQA groups, N >= 1000,
# causal with ragged tails on both sides, both causal alignments, large logits.
SHAPES_D256 = [
    (1, 8, 2, 1000, 1000, 256, True),
    (2, 4, 1, 1030, 1030, 256, True),
    (1, 4, 2, 1100, 700, 256, False),
    (1, 2, 1, 700, 1300, 256, True),
    (1, 6, 3, 1027, 1027, 256, False),
]


# At most 256 workgroups of 128 keys: the dK/dV kernel's split form (64 keys per
# workgroup, two wave pairs per query tile); most SHAPES above take it too.
SHAPES_SPLIT = [
    (1, 8, 8, 2048, 2048, 128, True),
    (1, 8, 2, 2000, 2000, 64, True),
    (2, 4, 4, 1000, 1500, 128, False),
    (1, 6, 3, 1500, 700, 128, True),
    (1, 32, 8, 4000, 4090, 128, True),     # exactly 256 workgroups of 128 keys; GQA
]


@pytest.mark.parametrize("shape", SHAPES_SPLIT)
def test_bwd_split_dkdv(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    assert -(-Nk // 128) * Hkv * B <= 256
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True,
                            seed=3600 + Nq + 5 * Nk + Hq)
    check(gpu_lib, inp, f"bwd-split{shape}")


@pytest.mark.parametrize("shape", SHAPES_D256)
def test_bwd_d256(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True,
                            seed=3400 + Nq + 3 * Nk + Hq)
    check(gpu_lib, inp, f"bwd-d256{shape}")


def test_bwd_d256_large_logits(gpu_lib):
    inp = synth.make_inputs(1, 4, 2, 1000, 1000, 256, causal=True, with_do=True, seed=3450,
                            q_mult=4.0)
    check(gpu_lib, inp, "bwd d256 q*4")


@pytest.mark.parametrize("shape", SHAPES)
def test_bwd_shapes(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True,
                            seed=3000 + Nq + 7 * Nk + d + Hq)
    check(gpu_lib, inp, f"bwd{shape}")


@pytest.mark.parametrize("shape", [
    # at least 256 workgroups of 256 query rows (large grids: many dQ workgroups per
    # compute unit, dK/dV in 128-key workgroups), ragged tails
    (2, 32, 8, 1000, 1000, 128, True),
    (2, 32, 16, 1024, 1100, 64, False),
    # causal orders: dQ over 72 (batch, head) pairs (9 per XCD), dK/dV over 24 kv
    # pairs (3 per XCD); then 68 and 17 pairs, which do not split evenly over 8 XCDs
    (3, 24, 8, 1000, 1000, 128, True),
    (1, 68, 17, 1000, 1000, 64, True),
])
def test_bwd_large_grid_shapes(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    assert -(-Nq // 256) * Hq * B >= 256
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True,
                            seed=3200 + Nq + Nk + d)
    check(gpu_lib, inp, f"bwd-large{shape}")


def test_bwd_large_logits(gpu_lib):
    inp = synth.make_inputs(1, 4, 4, 512, 512, 64, causal=True, with_do=True, seed=3100,
                            q_mult=4.0)
    check(gpu_lib, inp, "bwd q*4")


@pytest.mark.parametrize("d", [128, 256])
def test_bwd_bitwise_deterministic(gpu_lib, d):
    import torch
    inp = synth.make_inputs(1, 8, 2, 700, 700, d, causal=True, with_do=True, seed=3200)
    a = gpu_fwd_bwd(gpu_lib, inp)
    b = gpu_fwd_bwd(gpu_lib, inp)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("shape", [(1, 8, 2, 700, 700, 128, True), (2, 32, 8, 1000, 1000, 128, True),
                                   (1, 4, 4, 300, 500, 64, False)])
def test_bwd_stages_equal_whole(gpu_lib, shape):
    """fa_bwd_stage 0 (dQ, with D and LSE*log2e into the workspace) then 1 (dK/dV) on one
    stream gives exactly what fa_bwd gives, with workspaces that start out different."""
    import torch
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True, seed=3300 + Nq)
    announce(f"bwd stages {shape}")
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o, lse = gpu_lib.fwd(q, k, v, causal=causal, scale=inp.scale)
    nbytes = gpu_lib.bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
    ws_a = torch.zeros(nbytes, device=q.device, dtype=torch.uint8)
    ws_b = torch.full((nbytes,), 0x7f, device=q.device, dtype=torch.uint8)
    whole = gpu_lib.bwd(q, k, v, o, do, lse, causal=causal, scale=inp.scale, workspace=ws_a)
    outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    for stage in (0, 1):
        gpu_lib.bwd(q, k, v, o, do, lse, causal=causal, scale=inp.scale, dq=outs[0], dk=outs[1],
                    dv=outs[2], workspace=ws_b, stage=stage)
    torch.cuda.synchronize()
    for x, y in zip(whole, outs):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


# d = 128 with at least 256 workgroups of 128 keys: the large-grid dK/dV kernel (one
# 32-key slot per wave, 4 waves). Ragged query and key tails, both causal alignments
# (Nq > Nk: the first rows see no key), GQA, MQA, non-causal and large logits; the GPU
# computes every gradient, the oracle the first and the last (batch, kv-head) group.
SHAPES_DKDV_LARGE = [
    (1, 64, 16, 2100, 2100, 128, True, 1.0),
    (2, 32, 32, 1000, 1300, 128, True, 1.0),    # Nk > Nq, key tail
    (2, 32, 16, 1500, 1100, 128, True, 1.0),    # Nq > Nk: rows < 400 see no key
    (1, 32, 32, 1100, 4200, 128, False, 1.0),
    (4, 4, 1, 700, 9000, 128, True, 1.0),       # MQA, long keys
    (1, 32, 32, 4100, 4100, 128, True, 4.0),    # large logits
]


@pytest.mark.parametrize("shape", SHAPES_DKDV_LARGE)
def test_bwd_dkdv_large_grid_shapes(gpu_lib, shape):
    import torch
    B, Hq, Hkv, Nq, Nk, d, causal, qm = shape
    assert -(-Nk // 128) * Hkv * B >= 256
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, with_do=True, q_mult=qm,
                            seed=3600 + Nq + 5 * Nk + Hkv)
    what = f"dkdv-large{shape}"
    announce(f"bwd {what}")
    dq, dk, dv = gpu_fwd_bwd(gpu_lib, inp)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    g = Hq // Hkv
    for (b, kvh) in ((0, 0), (B - 1, Hkv - 1)):
        hs = slice(kvh * g, (kvh + 1) * g)
        rq, rk, rv, _ = A.backward(inp.as_f64("q")[b:b + 1, hs], inp.as_f64("k")[b:b + 1, kvh:kvh + 1],
                                   inp.as_f64("v")[b:b + 1, kvh:kvh + 1],
                                   inp.as_f64("do")[b:b + 1, hs], inp.scale, causal)
        assert_grad_close(to_host64(dq[b:b + 1, hs]), rq, f"{what} b{b} g{kvh} dQ")
        assert_grad_close(to_host64(dk[b:b + 1, kvh:kvh + 1]), rk, f"{what} b{b} g{kvh} dK")
        assert_grad_close(to_host64(dv[b:b + 1, kvh:kvh + 1]), rv, f"{what} b{b} g{kvh} dV")


def test_c5_full_size_one_kv_group(gpu_lib):
    """The GQA training config at full size: the GPU computes every gradient; the
    oracle recomputes one (batch, kv-head) group in full (4 query heads, 8192 rows)."""
    import torch
    inp = synth.workload("c5_bf16_causal_gqa_B2Hq32Hkv8N8192d128")
    announce("bwd full-size c5")
    dq, dk, dv = gpu_fwd_bwd(gpu_lib, inp)
    g = inp.Hq // inp.Hkv
    for (b, kvh) in ((1, 5),):
        hs = slice(kvh * g, (kvh + 1) * g)
        q = inp.as_f64("q")[b:b + 1, hs]
        k = inp.as_f64("k")[b:b + 1, kvh:kvh + 1]
        v = inp.as_f64("v")[b:b + 1, kvh:kvh + 1]
        do = inp.as_f64("do")[b:b + 1, hs]
        rq, rk, rv, _ = A.backward(q, k, v, do, inp.scale, True)
        assert_grad_close(to_host64(dq[b:b + 1, hs]), rq, "c5 dQ")
        assert_grad_close(to_host64(dk[b:b + 1, kvh:kvh + 1]), rk, "c5 dK")
        assert_grad_close(to_host64(dv[b:b + 1, kvh:kvh + 1]), rv, "c5 dV")
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
