"""Host logic of the library on the CPU: the LM-head row layout and the
workspace bounds (tests/host/layout_check.cpp, built with hipcc as a host-only
program; no HIP runtime call is made)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_row_layout_and_workspace_bounds(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc unavailable")
    exe = str(tmp_path / "layout_check")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "host", "layout_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    res = subprocess.run([exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
