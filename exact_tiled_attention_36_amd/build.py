"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m exact_tiled_attention_36_amd.build`` or ``build()`` from Python.
Objects go to ``<repo>/_build/``; the library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
# Debug build: every kernel step also waits for its copies and passes a workgroup
# barrier (csrc/common.h debug_sync); its results must match libfa.so bit for bit.
SYNC_LIB = os.path.join(PKG, "libfa_sync.so")
SYNC_FLAGS = ("-DFA_DEBUG_BARRIERS=1",)
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off for all device code (see DESIGN notes);
# the host pass warns that it does not know the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
          "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]
# Options for single files: the d = 128 dK/dV kernel and the 4-wave forward and d = 64/128
# dQ kernels have their matrix products write ordinary vector registers (see the files'
# headers). The d = 128 dK/dV kernel is scheduled by the compiler's max-ILP strategy (0.6-2 %
# faster than the default, no scratch), the rest of the backward (bwd.hip: d = 64 and 256
# dK/dV, d = 256 dQ) by its iterative-ILP strategy (no kernel in that file spills more).
FILE_FLAGS = {"bwd_dkdv_d128.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form",
                                    "-mllvm", "--amdgpu-sched-strategy=max-ilp"],
              "fwd_bf16_small.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
              "bwd_dq_small.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
              "bwd.hip": ["-mllvm", "--amdgpu-sched-strategy=iterative-ilp"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def _compile(src: str, extra=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra,
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), lib_path: str = LIB) -> str:
    """Compile all sources and link ``lib_path``. ``extra_flags`` (e.g. -D options)
    go to every compile; objects of such variant builds get their own names."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    tag = "" if not extra_flags else "." + hashlib.sha1(" ".join(extra_flags).encode()).hexdigest()[:8]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, tuple(extra_flags), tag), srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
