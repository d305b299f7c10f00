"""The C ABI's argument checks under the host address and undefined-behaviour
sanitizers: csrc/fa_api.hip built with hipcc's host pass only (no device code), linked
with the stubs of tests/abi_sanitize_check.cpp in place of the kernel launchers and
the HIP runtime, and driven through every FA_ERR_* path of every entry point plus
valid calls that reach a launcher. Needs no GPU."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# host-only sanitizer flags (each -fsanitize= applies to the host pass)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
INC = ["-I", os.path.join(ROOT, "include"),
       "-I", os.path.join(ROOT, "exact_tiled_attention_36_amd", "csrc")]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not available")
def test_abi_checks_under_asan_ubsan(tmp_path):
    api_o, chk_o, exe = (str(tmp_path / n) for n in ("api.o", "check.o", "check"))
    base = [HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", *SAN, *INC, "-c"]
    r = subprocess.run(base + [os.path.join(ROOT, "exact_tiled_attention_36_amd", "csrc",
                                            "fa_api.hip"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    syms = subprocess.run(["nm", api_o], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "library object not instrumented"
    fatbin = re.search(r"__hip_fatbin_[0-9a-f]+", syms)
    assert fatbin, "no fat-binary reference in the host object"
    r = subprocess.run(base + [f"-DFA_FATBIN_SYMBOL={fatbin.group(0)}",
                               os.path.join(ROOT, "tests", "abi_sanitize_check.cpp"),
                               "-o", chk_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([CLANGXX, "-fsanitize=address,undefined", chk_o, api_o, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
