#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

One step = one sv_verify call over a whole batch of the mixed-sampler
workload (V=151936, B=1024 rows, K=3 drafts, fp32 logits, per-row T, top_k,
top_p), inputs already resident in HBM.  Prints one JSON line:

  value      verified rows/s (B / mean step time, hipEvent timing)
  roofline   the row-pass kernel (the HBM-bound step): algorithmic bytes
             per launch / its mean launch time, against 8 TB/s
  cpu_baseline  the fp64 oracle on the host cores over one full batch

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

With --op accept_stats it measures sv_accept_stats instead (the acceptance
statistics of position 0 of the same workload) and adds the study: the mean
of each statistic per sampler class and the expected tokens per step for
K = 1..4 that each implies.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified rows/s and achieved HBM GB/s (% of MI355X peak), V=151936"
PEAK_HBM_GBPS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_rowpass_mixed_samplers_b1024.json")
KERNEL_SOURCES = ["sv_device.h", "sv_rowpass.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rejection_sampling_verify_sv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Hip:
    """Minimal hipEvent access (the library records the events itself)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = ev.value
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        self.lib.hipEventSynchronize(ctypes.c_void_p(b))
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, arr):
        for e in arr:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))


def algorithmic_rows(acc, draft_len, params):
    """Logits rows the method must read for each batch row: target rows at
    positions 0..f and draft rows at positions 0..min(f, L-1) on sampling
    rows, f = the position of the emitted non-draft token (= accept length).
    Rows reported invalid or unsupported count zero."""
    acc = np.asarray(acc)
    L = np.asarray(draft_len)
    greedy = np.asarray(params["temperature"]) == 0
    ok = acc >= 0
    f = np.where(ok, acc, 0)
    tgt = np.where(ok, f + 1, 0)
    drf = np.where(ok & ~greedy, np.minimum(f, L - 1) + 1, 0)
    return int(tgt.sum()), int(drf.sum())


def rows_at_position(acc, draft_len, params, K):
    """Logits rows (target + draft) the method reads at each position k."""
    acc = np.asarray(acc)
    L = np.asarray(draft_len)
    greedy = np.asarray(params["temperature"]) == 0
    ok = acc >= 0
    f = np.where(ok, acc, -1)
    out = []
    for k in range(K + 1):
        tgt = ok & (k <= f)
        drf = ok & ~greedy & (k <= np.minimum(f, L - 1))
        out.append(int(tgt.sum() + drf.sum()))
    return out


def cpu_baseline(wl):
    import oracle

    oracle.build(force=False)
    t0 = time.perf_counter()
    out = oracle.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params, wl.uniforms,
                        dtype=wl.dtype)
    dt = time.perf_counter() - t0
    return {"value": wl.B / dt, "unit": "rows/s", "cores": int(out[4]), "kind": "oracle",
            "sample": f"one full step of the workload ({wl.B} rows), timed once, wall clock "
                      f"{dt:.2f} s, OpenMP over rows"}, out


STAT_NAMES = ["sum_min_p_q", "sum_p_q", "sum_min_p~_q", "sum_min_p~_q~"]


def expected_tokens(alpha, K):
    """Tokens per verify step (accepted drafts + the one drawn token) when
    every draft is accepted with probability alpha independently: the sum of
    alpha^j for j = 0..K."""
    alpha = np.asarray(alpha, np.float64)
    return np.sum([alpha ** j for j in range(K + 1)], axis=0)


def bench_accept_stats(args, wl, dev):
    import torch

    import rejection_sampling_verify_sv_amd as sv
    from rejection_sampling_verify_sv_amd import workloads

    B, V = wl.B, wl.V
    t, d, _, _, prm, _ = workloads.to_torch(wl, dev)
    t0, d0 = t[:, 0, :], d[:, 0, :]
    code = sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16
    ws = torch.empty(sv.workspace_bytes(B, 1, V, code) + 256, dtype=torch.uint8, device=dev)
    out = torch.empty((B, 4), dtype=torch.float64, device=dev)
    for _ in range(args.warmup):
        sv.accept_stats(t0, d0, prm, workspace=ws, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        sv.accept_stats(t0, d0, prm, workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    st = out.cpu().numpy()
    # two reads of both rows are what the method needs: the normalisers and
    # cuts, then the sums
    alg_bytes = 2 * 2 * B * V * wl.elem_size
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    P = wl.params
    cls = np.where(P["temperature"] == 0, "greedy",
                   np.where(P["top_k"] > 0, "top_k", np.where(P["top_p"] < 1, "nucleus", "full")))
    study = {}
    for c in ["greedy", "top_k", "full", "nucleus", "all"]:
        m = (cls == c) if c != "all" else np.ones(B, bool)
        m &= np.isfinite(st).all(axis=1)
        if not m.any():
            continue
        study[c] = {"rows": int(m.sum()),
                    "mean": {n: round(float(st[m, j].mean()), 4) for j, n in enumerate(STAT_NAMES)},
                    "tokens_per_step": {f"K={K}": {n: round(float(expected_tokens(st[m, j], K).mean()), 3)
                                                   for j, n in enumerate(STAT_NAMES)}
                                        for K in range(1, 5)}}
    line = {
        "metric": "acceptance-statistics rows/s, V=%d" % V,
        "value": round(B / (ms * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload + " position 0", "vocab": V, "batch": B,
                   "logits": wl.dtype},
        "roofline": {"bound": "hbm", "kernel": "whole call (7 launches)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "alg_bytes_per_call": int(alg_bytes)},
        "study": study,
    }
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        rows = np.arange(0, B, 16)
        tc = time.perf_counter()
        ref, _ = oracle.accept_stats(wl.target[rows, 0], wl.draft[rows, 0], P[rows],
                                     dtype=wl.dtype)
        dt = time.perf_counter() - tc
        line["cpu_baseline"] = {"value": len(rows) / dt, "unit": "rows/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{len(rows)} rows (every 16th), one thread, {dt:.2f} s"}
        ok = np.isfinite(ref).all(axis=1)
        line["oracle_max_abs_diff"] = float(np.abs(ref[ok] - st[rows][ok]).max())
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed_samplers_b1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", default="verify", choices=["verify", "accept_stats"])
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the measurement, run 5 device-to-device copies of MIB MiB "
                         "(the reference kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the verify step "
              "shards by batch rows with no communication, so N GPUs run N independent "
              "copies of this measurement.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rejection_sampling_verify_sv_amd as sv
    from rejection_sampling_verify_sv_amd import _lib, workloads

    dev = torch.device("cuda:0")
    lib = sv.load()
    log(f"[bench] generating {args.workload}")
    wl = workloads.make(args.workload)
    if args.op == "accept_stats":
        bench_accept_stats(args, wl, dev)
        return
    esz = wl.elem_size
    t, d, tok, dl, prm, uni = workloads.to_torch(wl, dev)
    B, K, V = wl.B, wl.K, wl.V
    code = sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16
    ws = torch.empty(sv.workspace_bytes(B, K, V, code) + 256, dtype=torch.uint8, device=dev)
    out_tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    out_acc = torch.empty((B,), dtype=torch.int32, device=dev)

    def step(events=None):
        sv.verify(t, d, tok, dl, prm, uni, workspace=ws, out_tokens=out_tok,
                  out_accept_len=out_acc, events=events)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # per-kernel times from events the library records between its launches
    hip = Hip()
    names = _lib.launch_names(K)
    nl = len(names)
    per_kernel = {}
    rowpass_ms = []
    evsets = [hip.events(nl + 1) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(events=evsets[s])
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i, n in enumerate(names):
            ms = hip.elapsed_ms(evsets[s][i], evsets[s][i + 1])
            per_kernel[n] = per_kernel.get(n, 0.0) + ms / args.steps
            if n == "rowpass":
                rowpass_ms.append(ms)
        hip.destroy(evsets[s])
    rowpass_launches = names.count("rowpass")
    rowpass_mean_ms = float(np.mean(rowpass_ms))
    by_pos_ms = np.mean(np.asarray(rowpass_ms).reshape(args.steps, rowpass_launches), axis=0)

    acc = out_acc.cpu().numpy()
    n_tgt, n_drf = algorithmic_rows(acc, wl.draft_len, wl.params)
    row_bytes = V * esz
    pos_bytes = [r * row_bytes for r in rows_at_position(acc, wl.draft_len, wl.params, K)]
    alg_bytes_step = (n_tgt + n_drf) * row_bytes
    alg_bytes_launch = alg_bytes_step / rowpass_launches
    achieved = alg_bytes_launch / (rowpass_mean_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as fh:
            c = json.load(fh)
        if c.get("kernel_source_hash") == kernel_source_hash():
            traffic = c.get("hbm_bytes_per_launch")

    value = B / (ms_per_step * 1e-3)
    unsupported = int((acc == -2).sum())
    served = acc >= 0
    L = wl.draft_len
    acc_rate = float(acc[served].sum() / max(1, L[served].sum()))
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "vocab": V, "batch": B, "max_draft": K,
                   "logits": wl.dtype, "rows_unsupported": unsupported},
        "roofline": {
            "bound": "hbm",
            "kernel": "rowpass",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": int(alg_bytes_launch),
            "launch_ms": round(rowpass_mean_ms, 4),
        },
        "kernels_ms_per_step": {k: round(v, 4) for k, v in per_kernel.items()},
        "rowpass_by_position": [{"ms": round(float(m), 4), "GBps": round(b / (m * 1e-3) / 1e9, 1)}
                                for m, b in zip(by_pos_ms, pos_bytes)],
        "useful_GBps_whole_step": round(alg_bytes_step / (ms_per_step * 1e-3) / 1e9, 1),
        "acceptance_rate": round(acc_rate, 4),
    }
    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on host cores)")
        cb, ref = cpu_baseline(wl)
        line["cpu_baseline"] = cb
        same = int(((ref[1] == acc) | (acc == -2)).sum())
        line["oracle_agreement_rows"] = same
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
