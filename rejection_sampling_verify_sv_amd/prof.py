"""Summaries of rocprofv3 output for the verify kernels.

Offline commands that turn the CSV files rocprofv3 writes into the short text
summaries kept under profiles/ (the library never imports this module):

  python -m rejection_sampling_verify_sv_amd.prof trace DIR --command CMD
      per-kernel table (calls, mean and total duration) from a
      ``--kernel-trace --stats`` run, as markdown on stdout;

  python -m rejection_sampling_verify_sv_amd.prof counters \\
      --fetch DIR --write DIR --bench-log LOG \\
      --command-fetch CMD --command-write CMD
      HBM bytes per dispatch of every kernel of the verify step from a
      ``--pmc FETCH_SIZE`` run and a ``--pmc WRITE_SIZE`` run of
      ``bench.py --no-extras --calibrate-copy 1024``, each counter scaled by
      what it reads for the 1 GiB device-to-device copies that run ends with
      (known bytes / counted bytes); plus the bytes of one whole step
      (per-dispatch bytes x dispatches per verify call), as JSON on stdout.
      The JSON carries the workload and a hash of the kernel sources: bench.py
      uses it only for that workload and only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def kernel_source_hash() -> str:
    """Hash of every kernel source file: counters taken on other sources are
    not reported."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


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


def _short(name: str) -> str:
    """sv::rowpass_kernel<0, true>(...) -> rowpass_kernel."""
    m = re.search(r"sv::(\w+)", name)
    return m.group(1) if m else name


def counters(fetch_dir, write_dir, bench_log, cmd_fetch, cmd_write) -> dict:
    line = _bench_line(bench_log)
    copy_bytes = int(line["calibration_copy_bytes"])
    calls = int(line["verify_calls"])
    out = {"workload": line["config"]["workload"], "kernel_source_hash": kernel_source_hash(),
           "verify_calls": calls, "alg_bytes_per_step": line["whole_step"]["alg_bytes"],
           "rowpass_alg_bytes_per_launch": line["roofline"]["alg_bytes_per_launch"],
           "commands": {"FETCH_SIZE": cmd_fetch, "WRITE_SIZE": cmd_write}, "calibration": {},
           "kernels": {}}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        cal_kib, ncal = _calibration(rows, copy_bytes)
        factor = copy_bytes / (cal_kib * 1024.0)
        out["calibration"][name] = {"copy_bytes": copy_bytes, "counted_kib": round(cal_kib, 1),
                                    "copies": ncal, "scale": round(factor, 4)}
        per = {}
        for r in rows:
            if "sv::" not in r["Kernel_Name"]:
                continue
            per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        for k, vals in per.items():
            e = out["kernels"].setdefault(k, {})
            e[name.lower() + "_bytes_per_dispatch"] = int(sum(vals) / len(vals) * 1024.0 * factor)
            e["dispatches"] = len(vals)
    step = 0.0
    for k, e in out["kernels"].items():
        e["bytes_per_dispatch"] = e.get("fetch_size_bytes_per_dispatch", 0) + \
            e.get("write_size_bytes_per_dispatch", 0)
        e["dispatches_per_step"] = round(e["dispatches"] / calls, 3)
        step += e["bytes_per_dispatch"] * e["dispatches"] / calls
    out["step_bytes"] = int(step)
    out["step_traffic_over_alg"] = round(step / out["alg_bytes_per_step"], 4)
    rp = out["kernels"].get("rowpass_kernel")
    if rp:
        out["rowpass_traffic_over_alg"] = round(
            rp["bytes_per_dispatch"] / out["rowpass_alg_bytes_per_launch"], 4)
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
    c.add_argument("--bench-log", required=True)
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    a = ap.parse_args()
    if a.what == "trace":
        sys.stdout.write(trace_table(a.dir, a.command))
    else:
        json.dump(counters(a.fetch, a.write, a.bench_log, a.command_fetch, a.command_write),
                  sys.stdout, indent=1)
        sys.stdout.write("\n")


if __name__ == "__main__":
    main()
