"""Summaries of rocprofv3 output for the verify kernels.

Two offline commands turn the CSV files rocprofv3 writes into the short text
summaries kept next to the code:

  python -m rejection_sampling_verify_sv_amd.prof trace DIR --command CMD
      per-kernel table (calls, mean and total duration) from a
      ``--kernel-trace --stats`` run, as markdown on stdout;

  python -m rejection_sampling_verify_sv_amd.prof counters \\
      --fetch DIR --write DIR --kernel rowpass_kernel --bench-log LOG \\
      --command-fetch CMD --command-write CMD
      HBM bytes per launch of one kernel from a ``--pmc FETCH_SIZE`` run and a
      ``--pmc WRITE_SIZE`` run, each scaled by what the same counter reads for
      the 1 GiB device-to-device copies ``bench.py --calibrate-copy 1024``
      runs at the end (known bytes / counted bytes), as JSON on stdout.

Nothing here is imported by the library itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def trace_table(d: str, command: str) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    out = ["# Kernel trace", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | mean us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def _counter_rows(d: str):
    return list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))


def _calibration(rows, copy_bytes: int):
    """Counted KiB per calibration copy: the copy dispatches of copy_bytes."""
    big = [float(r["Counter_Value"]) for r in rows
           if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) * 1024 > copy_bytes / 8]
    if not big:
        raise SystemExit("no calibration copy found in the counter file")
    return sum(big) / len(big), len(big)


def _bench_line(log: str) -> dict:
    for line in open(log, errors="replace"):
        line = line.strip()
        if line.startswith('{"metric"'):
            return json.loads(line)
    raise SystemExit(f"no bench JSON line in {log}")


def counters(fetch_dir, write_dir, kernel, bench_log, cmd_fetch, cmd_write) -> dict:
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402

    line = _bench_line(bench_log)
    copy_bytes = int(line["calibration_copy_bytes"])
    out = {"kernel": kernel, "workload": line["config"]["workload"],
           "kernel_source_hash": bench.kernel_source_hash(),
           "alg_bytes_per_launch": line["roofline"]["alg_bytes_per_launch"]}
    total = 0.0
    for name, d, cmd in (("FETCH_SIZE", fetch_dir, cmd_fetch), ("WRITE_SIZE", write_dir, cmd_write)):
        rows = _counter_rows(d)
        cal_kib, ncal = _calibration(rows, copy_bytes)
        factor = copy_bytes / (cal_kib * 1024.0)
        vals = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"kernel {kernel} not found in {d}")
        mean_kib = sum(vals) / len(vals)
        scaled = mean_kib * 1024.0 * factor
        total += scaled
        out[name] = {"mean_kib_per_dispatch": round(mean_kib, 1), "dispatches": len(vals),
                     "calibration_copy_bytes": copy_bytes,
                     "calibration_counted_kib": round(cal_kib, 1), "calibration_copies": ncal,
                     "scale": round(factor, 4), "bytes_per_launch": int(scaled),
                     "command": cmd}
    out["hbm_bytes_per_launch"] = int(total)
    out["traffic_over_algorithmic"] = round(total / out["alg_bytes_per_launch"], 4)
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--kernel", default="rowpass_kernel")
    c.add_argument("--bench-log", required=True)
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    a = ap.parse_args()
    if a.what == "trace":
        sys.stdout.write(trace_table(a.dir, a.command))
    else:
        json.dump(counters(a.fetch, a.write, a.kernel, a.bench_log, a.command_fetch,
                           a.command_write), sys.stdout, indent=1)
        sys.stdout.write("\n")


if __name__ == "__main__":
    main()
