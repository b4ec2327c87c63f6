"""Host logic of the rocprofv3 summariser (profiles/ records), on synthetic
CSV files shaped like rocprofv3's: the kernel-trace table, HBM traffic scaled
by a plain copy's counters, counter means with the matrix-core rate, and the
per-kernel source hash that keys a traffic record to the kernel it measured."""
import csv
import json

import pytest

from speculative_decoding_verification_philox_amd import rocprof_summary as RS

COUNTER_FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]


def _write(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _counters(path, counter, per_kernel):
    rows, d = [], 0
    for name, values in per_kernel:
        for v in values:
            d += 1
            rows.append({"Correlation_Id": d, "Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": v, "Start_Timestamp": 1000 * d, "End_Timestamp": 1000 * d + 500_000})
    _write(path, COUNTER_FIELDS, rows)


def test_stats_table(tmp_path, capsys):
    p = tmp_path / "run_kernel_stats.csv"
    _write(p, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [{"Name": "void dmv::k_gemm_panel<true, 3, false>(dmv::Plan, ...)", "Calls": 12, "AverageNs": 166000,
             "MinNs": 160000, "MaxNs": 207000, "Percentage": 71.8}])
    RS.main(["stats", str(p), "--command", "cmd", "--title", "T"])
    out = capsys.readouterr().out
    assert out.startswith("# T")
    assert "| `void dmv::k_gemm_panel<true, 3, false>` | 12 | 166.0 | 160.0 | 207.0 | 71.80% |" in out


def test_traffic_scales_each_counter_by_the_copy(tmp_path, capsys):
    # the copy of 1 GiB reads as half its bytes on FETCH_SIZE and exactly on WRITE_SIZE
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counters(fetch, "FETCH_SIZE", [(copy, [524288.0]), ("dmv::k_gemm_panel<true, 3, false>", [1000.0, 1200.0])])
    _counters(write, "WRITE_SIZE", [(copy, [1048576.0]), ("dmv::k_gemm_panel<true, 3, false>", [300.0, 300.0])])
    js = tmp_path / "rec.json"
    RS.main(["traffic", "--fetch", str(fetch), "--write", str(write), "--kernel", "k_gemm_panel", "--workload", "w",
             "--alg-bytes", "2000000", "--command", "cmd", "--json", str(js)])
    rec = json.load(open(js))
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == round(1100.0 * 1024 * 2)
    assert rec["hbm_write_bytes_per_launch"] == round(300.0 * 1024)
    assert rec["traffic_over_algorithmic"] == pytest.approx((1100 * 2048 + 300 * 1024) / 2e6, abs=1e-4)
    assert rec["kernel_source_sha256_16"] == RS.kernel_source_hash("k_gemm_panel")
    assert "| traffic / algorithmic |" in capsys.readouterr().out


def test_traffic_refuses_an_ambiguous_kernel_name(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    both = [("__amd_rocclr_copyBuffer", [1.0]), ("dmv::k_gemm_tile<true, 10>", [1.0]),
            ("dmv::k_gemm_tile<true, 9>", [1.0])]
    _counters(fetch, "FETCH_SIZE", both)
    _counters(write, "WRITE_SIZE", both)
    with pytest.raises(SystemExit):
        RS.main(["traffic", "--fetch", str(fetch), "--write", str(write), "--kernel", "k_gemm_tile", "--workload",
                 "w", "--alg-bytes", "1", "--command", "cmd"])


def test_counters_mean_and_matrix_core_rate(tmp_path, capsys):
    p = tmp_path / "c.csv"
    rows = []
    for d, (flops, util) in enumerate([(2.0e12, 50.0), (2.0e12, 54.0)], start=1):
        for name, v in (("MfmaFlopsBF16", flops), ("MfmaUtil", util)):
            rows.append({"Correlation_Id": d, "Dispatch_Id": d, "Kernel_Name": "dmv::k_gemm_tile<true, 10>",
                         "Counter_Name": name, "Counter_Value": v, "Start_Timestamp": 0,
                         "End_Timestamp": 2_000_000})  # 2 ms
    rows.append({"Correlation_Id": 9, "Dispatch_Id": 9, "Kernel_Name": "dmv::k_vocab<5>", "Counter_Name": "MfmaUtil",
                 "Counter_Value": 0.0, "Start_Timestamp": 0, "End_Timestamp": 1})
    _write(p, COUNTER_FIELDS, rows)
    RS.main(["counters", str(p), "--kernel", "k_gemm_tile", "--command", "cmd", "--title", "T"])
    out = capsys.readouterr().out
    assert "Dispatches of `k_gemm_tile`: 2; mean duration under counter collection 2000.0 us." in out
    assert "| MfmaUtil | 52.00 |" in out
    assert "| bf16 matrix-core rate (MfmaFlopsBF16 / duration) | 1,000.0 TFLOP/s |" in out


@pytest.mark.parametrize("kernel", ["k_gemm_panel", "k_gemm_tile", "k_vocab", "k_finish"])
def test_kernel_sections_are_separate(kernel):
    sec = RS.kernel_section(kernel)
    assert sec.startswith(RS._HEADER + kernel + ":")
    others = [k for k in ("k_gemm_panel", "k_gemm_tile", "k_vocab", "k_finish") if k != kernel]
    assert not any(RS._HEADER + o + ":" in sec for o in others)
    assert len(RS.kernel_source_hash(kernel)) == 16


def test_trace_table_leaves_out_the_warmup_dispatches(tmp_path, capsys):
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows, t = [], 0
    # two warm-up steps (slow), then three timed ones; the weight reorder runs once
    for us in (3000, 2900, 2200, 2210, 2190):
        for name, dur in (("void dmv::k_gemm_tile<true, 10, 1>(dmv::Plan, ...)", us), ("dmv::k_combine", 9)):
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur * 1000})
            t += dur * 1000 + 100
    rows.append({"Kernel_Name": "dmv::k_pack_w", "Start_Timestamp": t, "End_Timestamp": t + 900_000})
    p = tmp_path / "run_kernel_trace.csv"
    _write(p, fields, rows)
    RS.main(["trace", str(p), "--warmup", "2", "--command", "cmd", "--title", "T"])
    out = capsys.readouterr().out
    assert "| `void dmv::k_gemm_tile<true, 10, 1>` | 5 | 3 | 2200.0 | 2200.0 | 2190.0 | 2210.0 |" in out
    assert "| `dmv::k_pack_w` | 1 | 1 | 900.0 |" in out
    assert RS.kernel_source_hash() in out
