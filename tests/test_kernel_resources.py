"""Register and scratch budgets of the built kernels (CPU: reads the gfx950
code object's metadata notes, no GPU).

A kernel that spills registers, or that copies its by-value launch
parameters into per-lane scratch to index them at run time, runs its hot
path through memory: at the batched 70B head either made the matrix-core
GEMM about a quarter slower, with unchanged results.  These checks keep
both out of every kernel of the library."""
import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_verification_philox_amd import binding as Bd

ROCM_LLVM = "/opt/rocm/llvm/bin"
# kernels allowed a small fixed scratch area (a short local array indexed at
# run time, outside any inner loop), with its limit in bytes
SCRATCH_ALLOWED = {"k_filter": 128}


def _tool(name):
    path = os.path.join(ROCM_LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(Bd.LIB_PATH):
        pytest.skip("libdmverify.so is not built")
    objcopy, bundler, readelf = shutil.which("objcopy"), _tool("clang-offload-bundler"), _tool("llvm-readelf")
    if not (objcopy and bundler and readelf):
        pytest.skip("objcopy / clang-offload-bundler / llvm-readelf not available")
    d = tmp_path_factory.mktemp("co")
    fat, co = str(d / "fatbin"), str(d / "gfx950.co")
    subprocess.run([objcopy, "-O", "binary", "--only-section=.hip_fatbin", Bd.LIB_PATH, fat], check=True)
    subprocess.run([bundler, "--unbundle", "--type=o", f"--input={fat}", f"--output={co}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950"], check=True)
    notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True, text=True).stdout
    out, cur = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s*\.name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.match(r"\s*\.(vgpr_spill_count|sgpr_spill_count|private_segment_fixed_size|vgpr_count):\s+(\d+)",
                     line)
        if m and cur is not None:
            out[cur][m.group(1)] = int(m.group(2))
    assert out, "no kernel metadata in the code object"
    return out


def _short(mangled):
    m = re.search(r"(k_[a-z_0-9]+)", mangled)
    return m.group(1) if m else mangled


def test_every_hot_kernel_is_in_the_code_object(kernels):
    names = {_short(k) for k in kernels}
    for k in ("k_prep", "k_prep_packed", "k_gemm_panel", "k_gemm_tile", "k_gemm_skinny", "k_combine", "k_vocab",
              "k_finish", "k_filter", "k_pack_w"):
        assert k in names, k
    # every sub-tile count of the matrix-core kernel, both element types
    assert sum(_short(k) == "k_gemm_tile" for k in kernels) == 14


def test_no_kernel_spills_registers(kernels):
    bad = {k: v for k, v in kernels.items() if v.get("vgpr_spill_count", 0) or v.get("sgpr_spill_count", 0)}
    assert not bad, bad


def test_no_kernel_takes_scratch_beyond_its_allowance(kernels):
    bad = {k: v["private_segment_fixed_size"] for k, v in kernels.items()
           if v.get("private_segment_fixed_size", 0) > SCRATCH_ALLOWED.get(_short(k), 0)}
    assert not bad, bad
