"""Summaries of rocprofv3 output for the profiles/ directory.

  python -m speculative_decoding_verification_philox_amd.rocprof_summary stats \
      RUN_kernel_stats.csv --command "..." --title "..." > profiles/X.md

  python -m speculative_decoding_verification_philox_amd.rocprof_summary trace \
      RUN_kernel_trace.csv --warmup W --command "..." --title "..." > profiles/X.md

  python -m speculative_decoding_verification_philox_amd.rocprof_summary traffic \
      --fetch FETCH_counter_collection.csv --write WRITE_counter_collection.csv \
      --kernel k_gemm_panel --workload llama3_8b_head --alg-bytes N \
      --calib-kernel __amd_rocclr_copyBuffer --calib-bytes 1073741824 \
      --command "..." --json profiles/k_gemm_llama3_8b_head_traffic.json > profiles/Y.md

  python -m speculative_decoding_verification_philox_amd.rocprof_summary counters \
      RUN_counter_collection.csv --kernel k_gemm_tile --command "..." --title "..." > profiles/Z.md

`counters` prints the mean per dispatch of every counter collected for one
kernel, with the dispatch duration from the same records; MfmaFlopsBF16 is
also turned into TFLOP/s over that duration.

`traffic` turns the per-dispatch FETCH_SIZE / WRITE_SIZE counters (KiB) of a
kernel into HBM bytes per launch.  Each counter is scaled by the factor that
makes it read the known size of a plain copy kernel captured in the same run
(bytes read = bytes written = --calib-bytes).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(PKG, "csrc", "dm_kernels.hip")
COMMON_SRC = os.path.join(PKG, "csrc", "dm_common.hpp")
_HEADER = "// =====================================================================\n// "


def kernel_section(kernel: str) -> str:
    """The part of the kernel source that defines `kernel`: from its header
    comment to the next kernel's header."""
    text = open(KERNEL_SRC).read()
    start = text.find(_HEADER + kernel + ":")
    if start < 0:
        raise KeyError(f"no header comment for {kernel} in {KERNEL_SRC}")
    end = text.find(_HEADER, start + len(_HEADER))
    return text[start:end if end >= 0 else len(text)]


def kernel_source_hash(kernel: str | None = None) -> str:
    """sha256 (first 16 hex digits) of the whole kernel file, or, for one
    kernel, of its section; either way followed by the shared header every
    kernel includes (the Philox rounds, the row layout, the statistics)."""
    body = open(KERNEL_SRC).read() if kernel is None else kernel_section(kernel)
    return hashlib.sha256((body + open(COMMON_SRC).read()).encode()).hexdigest()[:16]


def _short(name: str) -> str:
    return re.sub(r"\(.*", "", name).strip()


def stats(args) -> None:
    rows = list(csv.DictReader(open(args.csv)))
    print(f"# {args.title}\n")
    print(f"Command (from the repository root):\n\n```\n{args.command}\n```\n")
    print("| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    print(f"\nKernel source sha256 (first 16 hex digits) of csrc/dm_kernels.hip plus csrc/dm_common.hpp: "
          f"`{kernel_source_hash()}`")


def trace(args) -> None:
    """Per-kernel durations from the kernel-trace records, leaving out the
    first `--warmup` dispatches of every kernel launched more often than that
    (the untimed warm-up steps), so the table shows the timed steps only."""
    per: dict[str, list[float]] = {}
    for r in csv.DictReader(open(args.csv)):
        us = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3
        per.setdefault(_short(r["Kernel_Name"]), []).append(us)
    timed = {k: (v[args.warmup:] if len(v) > args.warmup else v) for k, v in per.items()}
    total = sum(sum(v) for v in timed.values())
    print(f"# {args.title}\n")
    print(f"Command (from the repository root):\n\n```\n{args.command}\n```\n")
    print(f"The first {args.warmup} dispatches of each kernel launched more than {args.warmup} times are the "
          f"warm-up steps and are left out; the other columns cover the remaining dispatches.\n")
    print("| kernel | dispatches | timed | mean (us) | median (us) | min (us) | max (us) | share of timed GPU time |")
    print("|---|---|---|---|---|---|---|---|")
    for k in sorted(timed, key=lambda k: -sum(timed[k])):
        v = timed[k]
        print(f"| `{k}` | {len(per[k])} | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | "
              f"{min(v):.1f} | {max(v):.1f} | {100.0 * sum(v) / total:.2f}% |")
    print(f"\nKernel source sha256 (first 16 hex digits) of csrc/dm_kernels.hip plus csrc/dm_common.hpp: "
          f"`{kernel_source_hash()}`")


def _per_dispatch(path: str) -> dict[str, list[float]]:
    out: dict[str, list[float]] = {}
    for r in csv.DictReader(open(path)):
        out.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def _match(table: dict[str, list[float]], key: str) -> list[float]:
    hits = [v for k, v in table.items() if key in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel name '{key}' matches {len(hits)} entries: {sorted(table)}")
    return hits[0]


def traffic(args) -> None:
    fetch, write = _per_dispatch(args.fetch), _per_dispatch(args.write)
    cf = max(_match(fetch, args.calib_kernel))  # the large copy (the runtime may add tiny ones)
    cw = max(_match(write, args.calib_kernel))
    f_scale = args.calib_bytes / (cf * 1024.0)
    w_scale = args.calib_bytes / (cw * 1024.0)
    kf = _match(fetch, args.kernel)
    kw = _match(write, args.kernel)
    fetch_b = statistics.mean(kf) * 1024.0 * f_scale
    write_b = statistics.mean(kw) * 1024.0 * w_scale
    total = fetch_b + write_b
    rec = {
        "kernel": args.kernel,
        "workload": args.workload,
        "fetch_kib_per_dispatch": [round(x, 1) for x in kf],
        "write_kib_per_dispatch": [round(x, 1) for x in kw],
        "calibration": {"kernel": args.calib_kernel, "bytes": args.calib_bytes, "fetch_kib": cf, "write_kib": cw,
                        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5)},
        "hbm_read_bytes_per_launch": round(fetch_b),
        "hbm_write_bytes_per_launch": round(write_b),
        "hbm_bytes_per_launch": round(total),
        "algorithmic_bytes_per_launch": args.alg_bytes,
        "traffic_over_algorithmic": round(total / args.alg_bytes, 4) if args.alg_bytes else None,
        "kernel_source_sha256_16": kernel_source_hash(args.kernel),
        "kernel_source_hashed": f"the {args.kernel} section of csrc/dm_kernels.hip plus csrc/dm_common.hpp",
        "command": args.command,
    }
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    print(f"# HBM traffic of `{args.kernel}`, {args.workload}\n")
    print(f"Commands (from the repository root, one run per counter):\n\n```\n{args.command}\n```\n")
    print(f"Calibration: `{args.calib_kernel}` copies {args.calib_bytes} bytes.  The counters read "
          f"FETCH_SIZE {cf:.1f} KiB and WRITE_SIZE {cw:.1f} KiB, so the scale factors are "
          f"{f_scale:.4f} (read) and {w_scale:.4f} (write).\n")
    print("| quantity | per launch |")
    print("|---|---|")
    print(f"| FETCH_SIZE (KiB, raw, per dispatch) | {', '.join(f'{x:.1f}' for x in kf)} |")
    print(f"| WRITE_SIZE (KiB, raw, per dispatch) | {', '.join(f'{x:.1f}' for x in kw)} |")
    print(f"| HBM read bytes (scaled) | {fetch_b:,.0f} |")
    print(f"| HBM write bytes (scaled) | {write_b:,.0f} |")
    print(f"| HBM bytes total | {total:,.0f} |")
    print(f"| algorithmic bytes | {args.alg_bytes:,} |")
    if args.alg_bytes:
        print(f"| traffic / algorithmic | {total / args.alg_bytes:.4f} |")
    print(f"\nSource sha256 (first 16 hex digits) of the `{args.kernel}` section of csrc/dm_kernels.hip plus "
          f"csrc/dm_common.hpp: `{kernel_source_hash(args.kernel)}`")


def counters(args) -> None:
    per: dict[str, list[float]] = {}
    dur: dict[str, float] = {}
    for r in csv.DictReader(open(args.csv)):
        if args.kernel not in _short(r["Kernel_Name"]):
            continue
        per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        dur[r["Dispatch_Id"]] = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9
    if not per:
        raise SystemExit(f"no dispatch of {args.kernel} in {args.csv}")
    t = statistics.mean(dur.values())
    print(f"# {args.title}\n")
    print(f"Command (from the repository root):\n\n```\n{args.command}\n```\n")
    print(f"Dispatches of `{args.kernel}`: {len(dur)}; mean duration under counter collection {t * 1e6:.1f} us.\n")
    print("| counter | mean per dispatch |")
    print("|---|---|")
    for name in sorted(per):
        print(f"| {name} | {statistics.mean(per[name]):,.2f} |")
    if "MfmaFlopsBF16" in per:
        fl = statistics.mean(per["MfmaFlopsBF16"])
        print(f"| bf16 matrix-core rate (MfmaFlopsBF16 / duration) | {fl / t / 1e12:,.1f} TFLOP/s |")
    print(f"\nSource sha256 (first 16 hex digits) of the `{args.kernel}` section of csrc/dm_kernels.hip plus "
          f"csrc/dm_common.hpp: `{kernel_source_hash(args.kernel)}`")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", required=True)
    k = sub.add_parser("trace")
    k.add_argument("csv")
    k.add_argument("--warmup", type=int, required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--title", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--title", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--alg-bytes", type=int, required=True)
    t.add_argument("--calib-kernel", default="__amd_rocclr_copyBuffer")
    t.add_argument("--calib-bytes", type=int, default=1 << 30)
    t.add_argument("--command", required=True)
    t.add_argument("--json", default=None)
    a = ap.parse_args(argv)
    {"stats": stats, "trace": trace, "counters": counters, "traffic": traffic}[a.cmd](a)


if __name__ == "__main__":
    main(sys.argv[1:])
