"""Python binding of libfa.so (ctypes). Argument marshalling only.

PyTorch supplies device memory and streams; every step of the attention computation
runs in the library's HIP kernels. There is no fallback: if the library is missing
or a call fails, an exception is raised.

The library must share PyTorch's HIP runtime. Both carry the soname
``libamdhip64.so.7``; importing torch first makes the loader resolve libfa.so's
dependency to the runtime torch already loaded, so device pointers and stream handles
are valid on both sides.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

_lib = None

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes)
_SIGNATURES = {
    "fa_version": (_c_int, []),
    "fa_status_string": (ctypes.c_char_p, [_c_int]),
    "fa_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "fa_fwd_f32": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "fa_fwd_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 6 + [_c_float] * 4
                   + [_c_int, _vp]),
    "fa_splitkv_default_splits": (_c_int, [_c_int] * 6),
    "fa_fwd_splitkv_workspace_bytes": (_c_size, [_c_int] * 7),
    "fa_fwd_splitkv": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 6
                       + [_c_float, _c_int, _c_int, _vp, _c_size, _vp]),
    "fa_bwd_workspace_bytes": (_c_size, [_c_int] * 6),
    "fa_bwd": (_c_int, [_vp] * 10 + [_c_size] + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "fa_bwd_stage": (_c_int, [_c_int] + [_vp] * 10 + [_c_size] + [_c_int] * 6
                     + [_c_float, _c_int, _vp]),
    "fa_bwd_noalloc": (_c_int, [_vp] * 9 + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "fa_fwd_variant_workspace_bytes": (_c_size, [_c_int] * 7),
    "fa_fwd_variant": (_c_int, [_vp] * 6 + [_c_size] + [_c_int] * 6
                       + [_c_float, _c_int, _c_int, _vp]),
    "fa_mfma_probe": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp]),
}

EXPORTED = tuple(_SIGNATURES)


class FAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load(path: Optional[str] = None, require_torch: bool = True):
    """Load libfa.so once and attach the C signatures. Raises if it is not built.

    The library next to this file is used unless ``path`` or the environment variable
    FA_LIBRARY names another build of the same sources. The library loaded last is
    the one every call of this module uses."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    if require_torch:
        import torch  # noqa: F401  (loads the HIP runtime the library must share)
    p = path or os.environ.get("FA_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run __graft_entry__.build() or "
                           "python -m exact_tiled_attention_36_amd.build")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise FAError(fn, status, status_string(status))


def _stream(dev) -> int:
    import torch
    return torch.cuda.current_stream(dev).cuda_stream


def _dims(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("k and v must be [B, Hkv, Nk, d] with q's B and d")
    return B, Hq, Hkv, Nq, Nk, d


def _buf(t, shape, dtype, device, name: str):
    """Allocate an output buffer, or check that the caller's one fits exactly: the
    library writes every element of it, so a smaller or strided buffer would be
    overrun."""
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)} on {device}")
    return t


def _inp(t, shape, dtype, device, name: str):
    """Check a required input tensor (never allocated: the library reads it)."""
    import torch
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)} on {device}")
    return t


def _launch(name: str, fn, device, *args):
    """Call a library entry point with the tensors' device current (the library
    launches on the current HIP device and the stream passed in) and raise on error."""
    import torch
    with torch.cuda.device(device):
        _check(name, fn(*args, _stream(device)))


def _workspace(t, nbytes: int, device):
    """A byte workspace of at least nbytes (allocated if None)."""
    import torch
    if t is None:
        return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.device != device
            or not t.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    return t


def fwd(q, k, v, causal: bool = False, scale: Optional[float] = None,
        out=None, lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O and LSE for bf16 (fa_fwd) or float32 (fa_fwd_f32) inputs."""
    import torch
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _buf(out, q.shape, q.dtype, q.device, "out")
    lse = _buf(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    if q.dtype == torch.bfloat16:
        fn, name = lib.fa_fwd, "fa_fwd"
    elif q.dtype == torch.float32:
        fn, name = lib.fa_fwd_f32, "fa_fwd_f32"
    else:
        raise ValueError("dtype must be bfloat16 or float32")
    _launch(name, fn, q.device, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, sc, int(bool(causal)))
    return out, lse


def fwd_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
            causal: bool = False, scale: Optional[float] = None, out=None,
            lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O (bf16) and LSE (float32) from FP8 E4M3 inputs with per-tensor descales
    (fa_fwd_fp8): the attention of descale_q*q8, descale_k*k8, descale_v*v8.

    q8/k8/v8 are uint8 tensors of E4M3 codes or torch.float8_e4m3fn tensors."""
    import torch
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q8, k8, v8)
    if q8.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError("fwd_fp8 takes uint8 E4M3 codes or float8_e4m3fn tensors")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _buf(out, (B, Hq, Nq, d), torch.bfloat16, q8.device, "out")
    lse = _buf(lse, (B, Hq, Nq), torch.float32, q8.device, "lse")
    _launch("fa_fwd_fp8", lib.fa_fwd_fp8, q8.device, q8.data_ptr(), k8.data_ptr(),
            v8.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, sc,
            float(descale_q), float(descale_k), float(descale_v), int(bool(causal)))
    return out, lse


FWD_VARIANTS = {"deferred": 0, "renorm_every_block": 1, "v1_loop_order": 2,
                "poly_exp_1_in_8": 3}


def fwd_variant(q, k, v, variant, causal: bool = False, scale: Optional[float] = None,
                out=None, lse=None, workspace=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O and LSE (bf16) through one of the comparison variants of fa_fwd_variant:
    0 / "deferred" (fa_fwd), 1 / "renorm_every_block", 2 / "v1_loop_order",
    3 / "poly_exp_1_in_8"."""
    import torch
    lib = load()
    var = FWD_VARIANTS[variant] if isinstance(variant, str) else int(variant)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("fwd_variant takes bfloat16 inputs")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _buf(out, q.shape, q.dtype, q.device, "out")
    lse = _buf(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    nbytes = lib.fa_fwd_variant_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, var)
    if workspace is not None or nbytes:
        workspace = _workspace(workspace, nbytes, q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wlen = workspace.numel() if workspace is not None else 0
    _launch("fa_fwd_variant", lib.fa_fwd_variant, q.device, q.data_ptr(), k.data_ptr(),
            v.data_ptr(), out.data_ptr(), lse.data_ptr(), wptr, wlen, B, Hq, Hkv, Nq, Nk,
            d, sc, int(bool(causal)), var)
    return out, lse


def splitkv_default_splits(B, Hq, Hkv, Nq, Nk, d) -> int:
    return load().fa_splitkv_default_splits(B, Hq, Hkv, Nq, Nk, d)


def splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits=0) -> int:
    return load().fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits)


def fwd_splitkv(q, k, v, causal: bool = True, scale: Optional[float] = None,
                num_splits: int = 0, out=None, lse=None, workspace=None):
    """Split-KV forward (decode shapes), bf16."""
    import torch
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if q.dtype != torch.bfloat16:
        raise ValueError("fa_fwd_splitkv takes bfloat16")
    out = _buf(out, q.shape, q.dtype, q.device, "out")
    lse = _buf(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    nbytes = lib.fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits)
    workspace = _workspace(workspace, nbytes, q.device)
    _launch("fa_fwd_splitkv", lib.fa_fwd_splitkv, q.device, q.data_ptr(), k.data_ptr(),
            v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, sc,
            int(bool(causal)), int(num_splits), workspace.data_ptr(), workspace.numel())
    return out, lse


def bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d) -> int:
    return load().fa_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)


def bwd(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
        dq=None, dk=None, dv=None, workspace=None, stage: int = -1):
    """dQ, dK, dV (bf16) by recomputation from the forward's O and LSE.

    ``stage`` -1 runs the whole backward (fa_bwd); 0, 1 run one kernel stage
    (fa_bwd_stage: dQ with the row statistics D, then dK/dV) with the same buffers."""
    import torch
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = _inp(o, q.shape, q.dtype, q.device, "o")
    do = _inp(do, q.shape, q.dtype, q.device, "do")
    lse = _inp(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    dq = _buf(dq, q.shape, q.dtype, q.device, "dq")
    dk = _buf(dk, k.shape, k.dtype, k.device, "dk")
    dv = _buf(dv, v.shape, v.dtype, v.device, "dv")
    nbytes = lib.fa_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            workspace.data_ptr(), workspace.numel(), B, Hq, Hkv, Nq, Nk, d, sc,
            int(bool(causal)))
    if stage == -1:
        _launch("fa_bwd", lib.fa_bwd, q.device, *args)
    else:
        _launch("fa_bwd_stage", lib.fa_bwd_stage, q.device, int(stage), *args)
    return dq, dk, dv


# Largest B * Hq * Nq that fa_bwd_noalloc takes (include/fa.h).
BWD_NOALLOC_MAX_ROWS = 1048576


def bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal: bool = False,
                scale: Optional[float] = None):
    """dQ, dK, dV (bf16) through fa_bwd_noalloc: the library's own fixed scratch instead
    of a workspace. The output buffers are required (nothing is allocated here either)."""
    import torch
    lib = load()
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = _inp(o, q.shape, q.dtype, q.device, "o")
    do = _inp(do, q.shape, q.dtype, q.device, "do")
    lse = _inp(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    dq = _inp(dq, q.shape, q.dtype, q.device, "dq")
    dk = _inp(dk, k.shape, k.dtype, k.device, "dk")
    dv = _inp(dv, v.shape, v.dtype, v.device, "dv")
    _launch("fa_bwd_noalloc", lib.fa_bwd_noalloc, q.device, q.data_ptr(), k.data_ptr(),
            v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nk, d, sc, int(bool(causal)))
    return dq, dk, dv


MFMA_PROBE_KINDS = {"zeros": 0, "normal_bf16": 1}


def mfma_probe(blocks: int, iters: int, kind="normal_bf16", device=None, out=None):
    """Enqueue fa_mfma_probe on the current stream of `device` (a measurement helper:
    blocks * 4 waves, each iters * 16 bf16 32x32x16 matrix products on register
    operands, zeros or normal-like bf16). Returns (flop, out); time the call with
    events on the same stream."""
    import torch
    lib = load()
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    k = MFMA_PROBE_KINDS[kind] if isinstance(kind, str) else int(kind)
    out = _buf(out, (int(blocks) * 256,), torch.float32, dev, "out")
    _launch("fa_mfma_probe", lib.fa_mfma_probe, dev, out.data_ptr(), int(blocks), int(iters), k)
    return float(blocks) * 4 * iters * 16 * 32768, out
