"""Host-side check of the kernels' workgroup-to-tile maps (xcd_remap, causal_order):
every tile exactly once for every grid size, each XCD's share when heads split evenly
over the 8 XCDs, and the longest-first order. Compiles tests/grid_order_check.cpp with
hipcc's host pass (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_grid_order(tmp_path):
    exe = str(tmp_path / "grid_order_check")
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1",
           "-I", os.path.join(ROOT, "exact_tiled_attention_36_amd", "csrc"),
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "grid_order_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
