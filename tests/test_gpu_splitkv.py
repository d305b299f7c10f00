"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the float64 oracle."""
import numpy as np
import pytest

from exact_tiled_attention_36_amd import synth
from oracle import attention as A
from gpu_util import TOL_LSE_BF16, announce, assert_lse_close, assert_o_close, to_dev, to_host64

pytestmark = pytest.mark.gpu


def run_split(fa, inp, splits):
    import torch
    q, k, v = to_dev(inp, "q"), to_dev(inp, "k"), to_dev(inp, "v")
    o, lse = fa.fwd_splitkv(q, k, v, causal=inp.causal, scale=inp.scale, num_splits=splits)
    torch.cuda.synchronize()
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


def check(fa, inp, splits, what):
    announce(f"splitkv {what} B{inp.B} Hq{inp.Hq} Hkv{inp.Hkv} Nq{inp.Nq} Nk{inp.Nk} d{inp.d} "
             f"causal={inp.causal} splits={splits}")
    o, lse = run_split(fa, inp, splits)
    o_ref, lse_ref = A.forward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                               inp.scale, inp.causal)
    assert_o_close(o, o_ref, what)
    assert_lse_close(lse, lse_ref, TOL_LSE_BF16, what)


def test_c4b_decode_full_size(gpu_lib):
    inp = synth.workload("c4b_bf16_decode_B8H8Nq1Nk32768d128")
    check(gpu_lib, inp, 0, "c4b")


def test_gqa_decode_full_size(gpu_lib):
    """Eight query heads per kv-head at one query each: the chunks run on the matrix
    cores (rows of a kv-head = the GQA group)."""
    inp = synth.make_inputs(16, 32, 4, 1, 8192, 128, causal=True, seed=4200)
    check(gpu_lib, inp, 0, "gqa-decode")


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Nq, Nk, d, causal, splits
    (1, 32, 8, 1, 5000, 128, True, 0),      # GQA decode, 4 rows per kv head
    (2, 8, 2, 4, 3001, 128, True, 7),       # 16 rows per kv head, causal limit per row
    (1, 4, 4, 3, 100, 64, False, 1),
    (1, 2, 1, 2, 999, 256, True, 64),
    (1, 2, 2, 1, 10, 128, True, 6),         # a chunk past the last key stays empty
    (1, 2, 2, 1, 77, 64, True, 77),         # one key per chunk
    (1, 4, 1, 4, 2, 128, True, 2),          # Nq > Nk: rows that see no key
    (2, 16, 1, 1, 1000, 64, False, 5),      # MQA, 16 rows per kv head
    (1, 6, 3, 5, 333, 128, True, 3),        # 10 rows, ragged chunks and tiles
    (1, 8, 8, 1, 32768, 128, True, 0),      # default: 32 chunks of 1024 keys (vector)
    (1, 32, 8, 1, 20000, 128, True, 0),     # default: 39 chunks of 513 keys (matrix)
])
def test_splitkv_shapes(gpu_lib, case):
    B, Hq, Hkv, Nq, Nk, d, causal, splits = case
    inp = synth.make_inputs(B, Hq, Hkv, Nq, Nk, d, causal=causal, seed=4000 + Nk + Nq)
    check(gpu_lib, inp, splits, f"split{case}")


def test_splitkv_matches_tiled_forward(gpu_lib):
    import torch
    inp = synth.make_inputs(4, 8, 8, 1, 8192, 128, causal=True, seed=4100)
    q, k, v = to_dev(inp, "q"), to_dev(inp, "k"), to_dev(inp, "v")
    o1, l1 = gpu_lib.fwd(q, k, v, causal=True)
    o2, l2 = gpu_lib.fwd_splitkv(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4
