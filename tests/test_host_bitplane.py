"""Host build of the plane -> code rebuild network (csrc/bitplane.hpp) checked
bit by bit against the store's definition (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_bitplane_network_on_host(tmp_path):
    exe = tmp_path / "bitplane_check"
    cmd = [HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "decode_stage_gemv_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "bitplane_check.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "bitplane rebuild ok" in run.stdout
