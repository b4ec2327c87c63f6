"""AddressSanitizer and UndefinedBehaviorSanitizer on the CPU code: the fp64
oracle (tests/host/oracle_sanitize.c, every rule with every output buffer at
its exact size) and the library's host side (the row layout and workspace
bounds check, tests/host/layout_check.cpp, with the sanitizers on its host
code only).  Any report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1")


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc unavailable")
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(HOST, "oracle_sanitize.c"), "-o", exe, "-lm"], check=True, capture_output=True)
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "5 runs, 0 failures" in res.stdout
    assert "Sanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr


def test_host_layout_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc unavailable")
    exe = str(tmp_path / "layout_check_sanitized")
    host_only = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "include"), *host_only,
                    os.path.join(HOST, "layout_check.cpp"), "-o", exe], check=True, capture_output=True)
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=900)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
    assert "Sanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr
