"""The C-ABI library loads, exports every symbol include/fa.h declares, and rejects
bad arguments on the host before any HIP call (these calls enqueue nothing, so they
run without a GPU)."""
import ctypes
import os
import re

import pytest

from exact_tiled_attention_36_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", src)))


def declared_codes():
    src = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(FA_[A-Z_]+)\s*=\s*(-?\d+)", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.load(require_torch=False)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fa.EXPORTED)


def test_version_and_status_strings(lib):
    assert lib.fa_version() == 10000
    for name, code in declared_codes().items():
        s = lib.fa_status_string(code).decode()
        assert s.startswith(name), (name, s)
    assert "unknown" in lib.fa_status_string(12345).decode()


NULL = None
P = ctypes.c_void_p(4096)  # aligned, never dereferenced: validation fails first
PU = ctypes.c_void_p(4096 + 2)  # misaligned


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128,
        scale=0.1, causal=0, fn="fa_fwd"):
    return getattr(lib, fn)(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, None)


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32"])
def test_forward_validation(lib, fn):
    assert fwd(lib, q=NULL, fn=fn) == -1
    assert fwd(lib, lse=NULL, fn=fn) == -1
    for kw in (dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Nq=0), dict(Nk=0), dict(d=0),
               dict(Nq=-3)):
        assert fwd(lib, fn=fn, **kw) == -2, kw
    assert fwd(lib, Hq=3, Hkv=2, fn=fn) == -3
    assert fwd(lib, scale=0.0, fn=fn) == -10
    assert fwd(lib, scale=-1.0, fn=fn) == -10
    assert fwd(lib, scale=float("nan"), fn=fn) == -10
    assert fwd(lib, scale=float("inf"), fn=fn) == -10
    assert fwd(lib, q=PU, fn=fn) == -5
    assert fwd(lib, o=PU, fn=fn) == -5
    assert fwd(lib, B=1 << 20, Hq=1 << 12, Hkv=1, Nq=1 << 10, fn=fn) == -8


def test_head_dim_rules(lib):
    for d in (32, 96, 100, 512, 257):
        assert fwd(lib, d=d) == -4, d
    for d in (2, 6, 260, 512):
        assert fwd(lib, d=d, fn="fa_fwd_f32") == -4, d


def test_splitkv_validation_and_sizes(lib):
    ws = lib.fa_fwd_splitkv_workspace_bytes(8, 8, 8, 1, 32768, 128, 16)
    assert ws == 8 * 8 * 16 * 128 * 4 + 8 * 8 * 16 * 4
    s = lib.fa_splitkv_default_splits(8, 8, 8, 1, 32768, 128)
    assert 1 <= s <= 1024
    assert lib.fa_splitkv_default_splits(1, 1, 1, 1, 100, 128) == 1
    args = [P, P, P, P, P, 1, 2, 1, 1, 64, 128, 0.1, 1]
    ws = lib.fa_fwd_splitkv_workspace_bytes(1, 2, 1, 1, 64, 128, 4)
    assert lib.fa_fwd_splitkv(*args, 4, NULL, ws, None) == -6
    assert lib.fa_fwd_splitkv(*args, 4, P, ws - 1, None) == -6
    assert lib.fa_fwd_splitkv(*args, 2000, P, 1 << 30, None) == -9
    assert lib.fa_fwd_splitkv(*args, -1, P, 1 << 30, None) == -9
    assert lib.fa_fwd_splitkv(*args, 65, P, 1 << 30, None) == -9   # more splits than keys
    bad = [P, P, P, P, P, 1, 32, 1, 1, 64, 128, 0.1, 1]              # 32 rows per kv head
    assert lib.fa_fwd_splitkv(*bad, 4, P, 1 << 30, None) == -2
    assert lib.fa_fwd_splitkv(P, P, P, P, P, 1, 2, 1, 1, 64, 96, 0.1, 1, 4, P, 1 << 30,
                              None) == -4


def test_bwd_validation_and_workspace(lib):
    assert lib.fa_bwd_workspace_bytes(2, 32, 8, 8192, 8192, 128) == 2 * (2 * 32 * 8192 * 4)
    assert lib.fa_bwd_workspace_bytes(1, 1, 1, 3, 3, 64) == 256
    ws = lib.fa_bwd_workspace_bytes(1, 2, 1, 8, 8, 128)
    base = [P] * 9
    tail = [1, 2, 1, 8, 8, 128, 0.1, 1, None]
    assert lib.fa_bwd(*base, NULL, ws, *tail) == -6
    assert lib.fa_bwd(*base, P, ws - 1, *tail) == -6
    assert lib.fa_bwd(NULL, *base[1:], P, ws, *tail) == -1
    assert lib.fa_bwd(*base[:8], NULL, P, ws, *tail) == -1
    assert lib.fa_bwd(*base[:4], PU, *base[5:], P, ws, *tail) == -5
    assert lib.fa_bwd(*base, P, ws, 1, 3, 2, 8, 8, 128, 0.1, 1, None) == -3
    assert lib.fa_bwd(*base, P, ws, 1, 2, 1, 8, 8, 80, 0.1, 1, None) == -4


def test_bwd_noalloc_validation(lib):
    """fa_bwd_noalloc: the same argument checks as fa_bwd, and B*Hq*Nq beyond its fixed
    scratch is refused (FA_ERR_SCRATCH) before the library touches the HIP runtime."""
    base = [P] * 9
    assert lib.fa_bwd_noalloc(NULL, *base[1:], 1, 2, 1, 8, 8, 128, 0.1, 1, None) == -1
    assert lib.fa_bwd_noalloc(*base[:8], NULL, 1, 2, 1, 8, 8, 128, 0.1, 1, None) == -1
    assert lib.fa_bwd_noalloc(*base[:4], PU, *base[5:], 1, 2, 1, 8, 8, 128, 0.1, 1, None) == -5
    assert lib.fa_bwd_noalloc(*base, 1, 3, 2, 8, 8, 128, 0.1, 1, None) == -3
    assert lib.fa_bwd_noalloc(*base, 1, 2, 1, 8, 8, 80, 0.1, 1, None) == -4
    assert lib.fa_bwd_noalloc(*base, 1, 2, 1, 0, 8, 128, 0.1, 1, None) == -2
    assert lib.fa_bwd_noalloc(*base, 1, 2, 1, 8, 8, 128, 0.0, 1, None) == -10
    rows = fa.BWD_NOALLOC_MAX_ROWS
    assert lib.fa_bwd_noalloc(*base, 1, 1, 1, rows + 1, 8, 64, 0.1, 1, None) == -13
    assert lib.fa_bwd_noalloc(*base, 4, 8, 8, rows // 32 + 1, 8, 64, 0.1, 0, None) == -13
    assert "FA_BWD_NOALLOC_MAX_ROWS" in lib.fa_status_string(-13).decode()
    hdr = open(HEADER).read()
    assert f"#define FA_BWD_NOALLOC_MAX_ROWS {rows}" in hdr


def test_bwd_stage_validation(lib):
    ws = lib.fa_bwd_workspace_bytes(1, 2, 1, 8, 8, 128)
    args = [P] * 9 + [P, ws, 1, 2, 1, 8, 8, 128, 0.1, 1, None]
    for stage in (-2, 2, 3, 7):
        assert lib.fa_bwd_stage(stage, *args) == -11, stage
    assert lib.fa_bwd_stage(0, *([NULL] + [P] * 8 + [P, ws, 1, 2, 1, 8, 8, 128, 0.1, 1, None])) == -1


def test_autograd_refuses_host_tensors():
    """No host fallback: CPU tensors are rejected before any HIP call."""
    import torch
    from exact_tiled_attention_36_amd.autograd import scaled_dot_product_attention
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        scaled_dot_product_attention(q, q, q)


def test_fwd_variant_validation(lib):
    args = [P, P, P, P, P, P, 1 << 30, 1, 2, 1, 8, 8, 128, 0.1, 1]
    assert lib.fa_fwd_variant(*args, 4, None) == -12
    assert lib.fa_fwd_variant(*args, -1, None) == -12
    d256 = [P, P, P, P, P, P, 1 << 30, 1, 2, 1, 8, 8, 256, 0.1, 1]
    assert lib.fa_fwd_variant(*d256, 1, None) == -4
    assert lib.fa_fwd_variant(*d256, 2, None) == -4
    ws = lib.fa_fwd_variant_workspace_bytes(1, 2, 1, 8, 8, 128, 2)
    assert ws >= 2 * 128 * 128 * 4                     # one 128-row block of O per head
    assert lib.fa_fwd_variant_workspace_bytes(1, 2, 1, 8, 8, 128, 1) == 0
    small = [P, P, P, P, P, P, ws - 1, 1, 2, 1, 8, 8, 128, 0.1, 1]
    assert lib.fa_fwd_variant(*small, 2, None) == -6
    nows = [P, P, P, P, P, NULL, ws, 1, 2, 1, 8, 8, 128, 0.1, 1]
    assert lib.fa_fwd_variant(*nows, 2, None) == -6
    assert lib.fa_fwd_variant(NULL, *args[1:], 1, None) == -1


def test_fwd_fp8_validation(lib):
    def call(q=P, o=P, d=128, scale=0.1, dq=1.0, dk=1.0, dv=1.0, Hq=2, Hkv=1):
        return lib.fa_fwd_fp8(q, P, P, o, P, 1, Hq, Hkv, 8, 8, d, scale, dq, dk, dv, 1, None)
    assert call(q=NULL) == -1
    assert call(Hq=3, Hkv=2) == -3
    assert call(d=96) == -4
    assert call(q=PU) == -5
    assert call(o=PU) == -5
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert call(dq=bad) == -10
        assert call(dk=bad) == -10
        assert call(dv=bad) == -10
        assert call(scale=bad) == -10
    # the folded score scale must stay a finite positive float
    assert call(scale=1e30, dq=1e30, dk=1e30) == -10
    assert call(scale=1e-30, dq=1e-30, dk=1e-30) == -10


def test_binding_rejects_wrong_output_buffers():
    torch = pytest.importorskip("torch")
    dev = torch.device("cpu")
    with pytest.raises(ValueError):
        fa._buf(torch.empty(2, 3), (2, 4), torch.float32, dev, "out")
    with pytest.raises(ValueError):
        fa._buf(torch.empty(4, 2).t(), (2, 4), torch.float32, dev, "out")
    with pytest.raises(ValueError):
        fa._buf(torch.empty(2, 4, dtype=torch.float64), (2, 4), torch.float32, dev, "out")
    t = torch.empty(2, 4)
    assert fa._buf(t, (2, 4), torch.float32, dev, "out") is t
    with pytest.raises(ValueError):
        fa._workspace(torch.empty(16, dtype=torch.float32), 16, dev)


def test_binding_requires_backward_inputs():
    """O, dO and LSE are read by the backward: the binding never allocates them."""
    torch = pytest.importorskip("torch")
    dev = torch.device("cpu")
    with pytest.raises(ValueError):
        fa._inp(None, (2, 4), torch.float32, dev, "o")
    with pytest.raises(ValueError):
        fa._inp(torch.empty(2, 4, dtype=torch.bfloat16), (2, 4), torch.float32, dev, "lse")
    with pytest.raises(ValueError):
        fa._inp(torch.empty(4, 2).t(), (2, 4), torch.float32, dev, "do")
    t = torch.empty(2, 4)
    assert fa._inp(t, (2, 4), torch.float32, dev, "o") is t


def test_mfma_probe_validation(lib):
    assert lib.fa_mfma_probe(NULL, 1, 1, 0, None) == -1
    assert lib.fa_mfma_probe(PU, 1, 1, 0, None) == -5
    for blocks, iters, kind in ((0, 1, 0), (1, 0, 0), (1 << 21, 1, 0), (1, 1 << 21, 0),
                                (1, 1, 2), (1, 1, -1)):
        assert lib.fa_mfma_probe(P, blocks, iters, kind, None) == -2, (blocks, iters, kind)
