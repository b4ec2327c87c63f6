"""Host logic of bench.py (no GPU): the rule that names the LM-head kernel the
library launches for a workload (checked against the kernels the committed
kernel traces recorded), the check that voids an HBM traffic record once the
profiled kernel's source has changed, and the single-GPU guard."""
import dataclasses
import glob
import json
import os
import re
import subprocess
import sys

import pytest

import bench
from speculative_decoding_verification_philox_amd import rocprof_summary as RS
from speculative_decoding_verification_philox_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMMS = ("k_gemm_panel", "k_gemm_tile", "k_gemm_skinny")


def _kernel(cfg, panels=True, ragged_seed=0):
    modes = wl.modes_for(cfg)
    n_lossless = int((modes == wl.LOSSLESS).sum())
    if not ragged_seed:
        return bench.gemm_kernel(cfg, panels, n_lossless)
    per_seq = bench.ragged_gammas(cfg, ragged_seed) + 1
    lossless = modes == wl.LOSSLESS
    return bench.gemm_kernel(cfg, panels, n_lossless, int(per_seq[~lossless].sum()), int(per_seq[lossless].sum()))


def test_kernel_rule_per_workload():
    # one 64-row tile at B = 1 (40 rows, 8 positions of 5 heads; 20 rows at
    # the tiny workload); several tiles for the batched, mixed and tree ones
    expect = {0: "k_gemm_panel", 1: "k_gemm_panel", 2: "k_gemm_panel", 3: "k_gemm_tile", 4: "k_gemm_tile",
              5: "k_gemm_tile"}
    for cfg in wl.CONFIGS:
        assert _kernel(cfg) == expect[cfg.index], cfg.name
        assert _kernel(cfg, panels=False) == "k_gemm_skinny"


def test_kernel_rule_at_the_one_tile_boundary():
    # JS at K = 5: four lane groups of 3 positions fit one 64-row tile
    one = wl.CONFIGS[1]
    assert bench.gemm_kernel(dataclasses.replace(one, B=1, gamma=11), True, 0) == "k_gemm_panel"  # 12 positions
    assert bench.gemm_kernel(dataclasses.replace(one, B=1, gamma=12), True, 0) == "k_gemm_tile"   # 13
    # lossless rows (one per position) share no tile with lossy ones
    two = dataclasses.replace(one, B=2, gamma=7)
    assert bench.gemm_kernel(two, True, 0) == "k_gemm_tile"    # 16 JS positions: two tiles
    assert bench.gemm_kernel(two, True, 2) == "k_gemm_panel"   # 16 lossless rows: one tile
    assert bench.gemm_kernel(two, True, 1) == "k_gemm_tile"    # one tile each


def test_kernel_rule_matches_the_recorded_traces():
    traces = glob.glob(os.path.join(ROOT, "profiles", "k_gemm_*_kernel_trace.md"))
    assert traces
    by_name = {cfg.name: cfg for cfg in wl.CONFIGS}
    seen = 0
    for path in traces:
        m = re.match(r"(k_gemm_[a-z]+)_(.+?)(_ragged(\d+))?_kernel_trace\.md$", os.path.basename(path))
        assert m, path
        cfg = by_name[m.group(2)]
        launched = {k for k in GEMMS if f"dmv::{k}" in open(path).read()}
        assert launched == {_kernel(cfg, ragged_seed=int(m.group(4) or 0))} == {m.group(1)}, path
        seen += 1
    assert seen >= 2


def _record(tmp_path, workload, kernel, digest, nbytes=123456789):
    rec = {"kernel": kernel, "workload": workload, "kernel_source_sha256_16": digest, "hbm_bytes_per_launch": nbytes}
    (tmp_path / f"k_gemm_{workload}_traffic.json").write_text(json.dumps(rec))


def test_traffic_record_kept_only_for_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    _record(tmp_path, "w_now", "k_gemm_tile", RS.kernel_source_hash("k_gemm_tile"))
    _record(tmp_path, "w_old", "k_gemm_tile", "0" * 16)
    _record(tmp_path, "w_panel", "k_gemm_panel", RS.kernel_source_hash("k_gemm_panel"), nbytes=7)
    assert bench.measured_traffic("w_now", "k_gemm_tile") == 123456789
    assert bench.measured_traffic("w_old", "k_gemm_tile") is None      # the kernel changed since
    assert bench.measured_traffic("w_now", "k_gemm_panel") is None     # another kernel was profiled
    assert bench.measured_traffic("w_panel", "k_gemm_panel") == 7
    assert bench.measured_traffic("absent", "k_gemm_tile") is None


def test_committed_traffic_records_are_well_formed():
    for path in glob.glob(os.path.join(ROOT, "profiles", "k_gemm_*_traffic.json")):
        rec = json.load(open(path))
        assert rec["kernel"] in GEMMS
        assert os.path.basename(path) == f"k_gemm_{rec['workload']}_traffic.json"
        assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
        assert len(rec["kernel_source_sha256_16"]) == 16


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})],
                         ids=["gpus2", "gpus8", "world2"])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                         env=dict(os.environ, **env), timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""
