#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

One step = one sv_verify call over a whole batch, inputs already resident in
HBM.  The headline workload is the mixed-sampler batch (V=151936, B=1024
rows, K=3 drafts, fp32 logits, per-row T, top_k, top_p).  Prints one JSON
line:

  value         verified rows/s (B / mean step time, hipEvent timing)
  roofline      the row-pass kernel (the HBM-bound step): algorithmic bytes
                per launch / its mean launch time, against 8 TB/s; traffic =
                FETCH_SIZE + WRITE_SIZE per launch from the rocprofv3 counter
                summary of this workload (null when the sources changed since)
  whole_step    the whole step: algorithmic bytes / step time (useful rate),
                and the counted HBM bytes of every kernel / summed kernel time
  read_ceiling  a plain streaming read with the row pass's tiling: the
                sustainable read rate, the second denominator
  cpu_baseline  the fp64 oracle on the host cores: median of 3 runs over one
                full batch on all threads, plus a one-thread figure
  configs       the other workloads, each with its own figures: the
                untruncated ragged batch (V=248320), the small mixed-greedy
                batch (inputs rotated over replicas larger than the 256 MB
                last-level cache), the one-row decode step and the tiny
                V=1000 case (latency at B=1, throughput at B=10,000)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-extras] [--no-cpu-baseline] [--calibrate-copy MIB]

With --op accept_stats it measures sv_accept_stats instead (the acceptance
statistics of position 0 of the same workload) and adds the study: the mean
of each statistic per sampler class and the expected tokens per step for
K = 1..4 that each implies.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
HEADLINE = "mixed_samplers_b1024"
BAND = 1e-5


def metric_for(V: int) -> str:
    return f"verified rows/s and achieved HBM GB/s (% of MI355X peak), V={V}"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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


def dense_rows(draft_len, params):
    """Rows a verify that reads every drafted position would read."""
    L = np.asarray(draft_len)
    greedy = np.asarray(params["temperature"]) == 0
    return int((L + 1).sum() + np.where(greedy, 0, L).sum())


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


def counters_for(workload: str):
    """The rocprofv3 counter summary of this workload, if it was taken on the
    current kernel sources (else None)."""
    from rejection_sampling_verify_sv_amd import prof

    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        c = json.load(fh)
    if c.get("workload") != workload or c.get("kernel_source_hash") != prof.kernel_source_hash():
        return None
    return c


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(wl, acc_gpu, tok_gpu):
    """The oracle as it stands, on the host: median of 3 runs over the whole
    batch on all host threads, one run on one thread over every 32nd row;
    plus the agreement of the GPU's outputs with the oracle's."""
    import oracle

    oracle.build(force=False)
    runs, out = [], None
    for _ in range(3):
        t0 = time.perf_counter()
        out = oracle.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params, wl.uniforms,
                            dtype=wl.dtype)
        runs.append(time.perf_counter() - t0)
    dt = statistics.median(runs)
    rows1 = np.arange(0, wl.B, 32)
    t0 = time.perf_counter()
    oracle.verify(wl.target[rows1], wl.draft[rows1], wl.tokens[rows1], wl.draft_len[rows1],
                  wl.params[rows1], wl.uniforms[rows1], dtype=wl.dtype, nthreads=1)
    dt1 = time.perf_counter() - t0
    o_tok, o_acc, o_diag = out[0], out[1], out[2]
    same = (o_acc == acc_gpu) & (o_tok == tok_gpu).all(axis=1)
    m = o_diag[:, :, 3]
    in_band = np.array([bool((r[~np.isnan(r)] < BAND).any()) for r in m]) & (o_acc >= 0)
    cb = {"value": round(wl.B / dt, 1), "unit": "rows/s", "cores": int(out[4]), "kind": "oracle",
          "sample": (f"one full batch of the workload ({wl.B} rows), median of 3 runs "
                     f"({', '.join(f'{r:.2f}' for r in runs)} s), OpenMP over rows; "
                     f"one-thread run over every 32nd row ({len(rows1)} rows, {dt1:.2f} s)"),
          "one_thread_rows_per_s": round(len(rows1) / dt1, 2),
          "cpu_model": cpu_model()}
    agree = {"rows": int(wl.B), "identical_tokens_and_accept_len": int(same.sum()),
             "differing": int((~same).sum()), "differing_in_band": int((~same & in_band).sum()),
             "in_band": int(in_band.sum())}
    return cb, agree


def read_ceiling(dev, nbytes=2 << 30, reps=10):
    """Sustainable read rate: sv_stream_read over nbytes, mean of reps."""
    import torch

    import rejection_sampling_verify_sv_amd as sv

    buf = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    buf.fill_(0.5)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        sv.stream_read(buf, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        sv.stream_read(buf, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    torch.cuda.empty_cache()
    return {"GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": int(nbytes),
            "ms": round(ms, 4), "kernel": "sv_stream_read (row-pass tiling, max per element)"}


def measure(wl, dev, steps, warmup, replicas=1, ceiling=None, step_mode="auto"):
    """Time sv_verify on a workload; per-kernel times from the events the
    library records between its launches.  With replicas > 1 the step
    rotates over that many copies of the inputs in HBM."""
    import torch

    import rejection_sampling_verify_sv_amd as sv
    from rejection_sampling_verify_sv_amd import _lib, workloads

    B, K, V = wl.B, wl.K, wl.V
    esz = wl.elem_size
    ins = [workloads.to_torch(wl, dev) for _ in range(replicas)]
    code = sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16
    ws = torch.empty(sv.workspace_bytes(B, K, V, code) + 256, dtype=torch.uint8, device=dev)
    out_tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    out_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    calls = [0]

    def step(i, events=None):
        sv.verify(*ins[i % replicas], workspace=ws, out_tokens=out_tok, out_accept_len=out_acc,
                  events=events, step_mode=step_mode)
        calls[0] += 1

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps

    hip = Hip()
    names = _lib.launch_names(B, K, step_mode)
    nl = len(names)
    per_kernel = {}
    rowpass_ms = []
    cut_ms = []
    evsets = [hip.events(nl + 1) for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        step(s, events=evsets[s])
    torch.cuda.synchronize()
    for s in range(steps):
        for i, n in enumerate(names):
            ms = hip.elapsed_ms(evsets[s][i], evsets[s][i + 1])
            per_kernel[n] = per_kernel.get(n, 0.0) + ms / steps
            if n == "rowpass":
                rowpass_ms.append(ms)
            elif n == "cut_decide":
                cut_ms.append(ms)
        hip.destroy(evsets[s])
    rowpass_launches = names.count("rowpass")
    rowpass_mean_ms = float(np.mean(rowpass_ms))
    by_pos_ms = np.mean(np.asarray(rowpass_ms).reshape(steps, rowpass_launches), axis=0)
    cut_by_pos_ms = np.mean(np.asarray(cut_ms).reshape(steps, -1), axis=0)
    kernel_ms_step = float(sum(per_kernel.values()))

    acc = out_acc.cpu().numpy()
    tok = out_tok.cpu().numpy()
    n_tgt, n_drf = algorithmic_rows(acc, wl.draft_len, wl.params)
    row_bytes = V * esz
    pos_bytes = [r * row_bytes for r in rows_at_position(acc, wl.draft_len, wl.params, K)]
    alg_bytes_step = (n_tgt + n_drf) * row_bytes
    alg_bytes_launch = alg_bytes_step / rowpass_launches
    achieved = alg_bytes_launch / (rowpass_mean_ms * 1e-3) / 1e9
    useful = alg_bytes_step / (ms_per_step * 1e-3) / 1e9

    c = counters_for(wl.name)
    traffic = None
    whole = {"useful_GBps": round(useful, 1), "useful_frac": round(useful / PEAK_HBM_GBPS, 4),
             "alg_bytes": int(alg_bytes_step),
             "dense_bytes": int(dense_rows(wl.draft_len, wl.params) * row_bytes),
             "kernel_ms": round(kernel_ms_step, 4), "traffic_bytes": None,
             "traffic_over_alg": None, "achieved_hbm_GBps": None}
    if c is not None:
        traffic = c["kernels"].get("rowpass_kernel", {}).get("bytes_per_dispatch")
        tb = c.get("step_bytes")
        if tb:
            whole["traffic_bytes"] = int(tb)
            whole["traffic_over_alg"] = round(tb / alg_bytes_step, 4)
            whole["achieved_hbm_GBps"] = round(tb / (kernel_ms_step * 1e-3) / 1e9, 1)
    if ceiling:
        whole["useful_frac_of_read_ceiling"] = round(useful / ceiling, 4)
    served = acc >= 0
    L = wl.draft_len
    res = {
        "metric": metric_for(V),
        "value": round(B / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "ms_per_step": round(ms_per_step, 4),
        "steps": steps,
        "warmup": warmup,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "config": {"workload": wl.name, "vocab": V, "batch": B, "max_draft": K,
                   "logits": wl.dtype, "input_replicas": replicas, "step_mode": step_mode,
                   "launches": len(names),
                   "rows_unsupported": int((acc == -2).sum())},
        "roofline": {
            "bound": "hbm", "kernel": "rowpass", "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic, "alg_bytes_per_launch": int(alg_bytes_launch),
            "launch_ms": round(rowpass_mean_ms, 4),
        },
        "whole_step": whole,
        "kernels_ms_per_step": {k: round(v, 4) for k, v in per_kernel.items()},
        "rowpass_by_position": [{"ms": round(float(m), 4), "GBps": round(b / (m * 1e-3) / 1e9, 1)}
                                for m, b in zip(by_pos_ms, pos_bytes)],
        "cut_decide_ms_by_launch": [round(float(m), 4) for m in cut_by_pos_ms],
        "acceptance_rate": round(float(acc[served].sum() / max(1, L[served].sum())), 4),
        "verify_calls": calls[0],
    }
    if ceiling:
        res["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling, 4)
    if c is not None:
        # every kernel of the step: its counted HBM bytes per step (rocprofv3
        # FETCH_SIZE + WRITE_SIZE, calibrated) over its time per step (events)
        kh = {}
        for n, ms in per_kernel.items():
            e = c["kernels"].get(n + "_kernel")
            if not e or ms <= 0:
                continue
            b = e["bytes_per_dispatch"] * e["dispatches_per_step"]
            kh[n] = {"bytes_per_step": int(b), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                     "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        res["kernels_hbm"] = kh
    del ins, ws
    torch.cuda.empty_cache()
    return res, acc, tok


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


# Extra workloads of the default run: name, batch, input replicas.  The
# small batches rotate over copies whose total exceeds the 256 MB last-level
# cache, so that every step reads its logits from HBM.
EXTRAS = [
    ("fullvocab_ragged_b256", None, 1),
    ("mixed_greedy_b64", None, 4),
    ("decode_b1", None, 512),
    ("tiny_v1000", 1, 1),
    ("tiny_v1000", None, 1),
]


def _timed(fn, steps, warmup):
    """Mean ms per call of fn over `steps` calls after `warmup`, torch events
    on the current stream around the timed calls."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _op_line(args, metric, value, ms, dtype, config, alg_bytes, kernel_note):
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    return {
        "metric": metric, "value": round(value, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic", "config": config,
        "roofline": {"bound": "hbm", "kernel": kernel_note, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "alg_bytes_per_call": int(alg_bytes)},
    }


def bench_sample(args, wl, dev):
    """The plain sampler (sv_sample) over position 0's target rows of a
    recipe: one draw per row from its truncated distribution.  Algorithmic
    bytes: each row read once (the draw's second pass over a full-vocabulary
    row is not counted)."""
    import torch

    import rejection_sampling_verify_sv_amd as sv
    from rejection_sampling_verify_sv_amd import workloads

    B, V = wl.B, wl.V
    t, _, _, _, prm, uni = workloads.to_torch(wl, dev)
    rows, u = t[:, 0, :], uni[:, 0].contiguous()
    out = sv.sample(rows, prm, u)
    code = sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16
    ws = torch.empty(sv.workspace_bytes(B, 0, V, code) + 256, dtype=torch.uint8, device=dev)
    ms = _timed(lambda: sv.sample(rows, prm, u, out_tokens=out[0], out_status=out[1],
                                  workspace=ws), args.steps, args.warmup)
    line = _op_line(args, "sampled rows/s, V=%d" % V, B / (ms * 1e-3), ms,
                    "f32" if wl.dtype == "f32" else "bf16",
                    {"workload": args.workload + " position 0 targets", "vocab": V, "batch": B,
                     "logits": wl.dtype},
                    B * V * wl.elem_size, "whole call (sv_sample)")
    g_tok = out[0].cpu().numpy()
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        sel = np.arange(0, B, 16)
        tc = time.perf_counter()
        ref, _, _ = oracle.sample(wl.target[sel, 0], wl.params[sel], wl.uniforms[sel, 0],
                                  dtype=wl.dtype, nthreads=1)
        dt = time.perf_counter() - tc
        line["cpu_baseline"] = {"value": round(len(sel) / dt, 2), "unit": "rows/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{len(sel)} rows (every 16th), one thread, {dt:.2f} s"}
        line["oracle_agreement"] = {"rows": int(len(sel)),
                                    "identical_tokens": int((ref == g_tok[sel]).sum())}
    print(json.dumps(line), flush=True)


def bench_tree(args, dev):
    """The tree / multi-candidate verify (sv_verify_tree) on the tree recipe:
    256 rows, a Medusa-shaped tree of 12 candidates each.  Algorithmic bytes:
    each needed row read once, i.e. the target row of every node the walk
    reaches, and the draft row of every reached node with children on a
    sampling row."""
    import torch

    import rejection_sampling_verify_sv_amd as sv
    from rejection_sampling_verify_sv_amd import workloads

    log("[bench] generating the tree recipe")
    wl, par = workloads.make_tree()
    B, K, V = wl.B, wl.K, wl.V
    t, d, tok, nc, prm, uni = workloads.to_torch(wl, dev)
    par_t = torch.from_numpy(np.ascontiguousarray(par)).to(dev)
    depth = np.zeros(K + 1, np.int64)
    for c in range(1, K + 1):
        depth[c] = depth[par[0, c - 1]] + 1
    max_depth = int(depth.max())
    max_kids = int(np.bincount(par[0], minlength=K + 1).max())
    out = sv.verify_tree(t, d, tok, par_t, nc, prm, uni, max_depth=max_depth,
                         max_children=max_kids)
    code = sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16
    ws = torch.empty(sv.workspace_bytes(B, K, V, code) + 256, dtype=torch.uint8, device=dev)
    ms = _timed(lambda: sv.verify_tree(t, d, tok, par_t, nc, prm, uni, max_depth=max_depth,
                                       max_children=max_kids, workspace=ws, out_tokens=out[0],
                                       out_accept_len=out[1], out_path=out[2]),
                args.steps, args.warmup)
    g_tok, g_len, g_path = (x.cpu().numpy() for x in out[:3])
    has_kids = np.bincount(par[0], minlength=K + 1) > 0
    greedy = wl.params["temperature"] == 0
    n_tgt = n_drf = 0
    for b in range(B):
        if g_len[b] < 0:
            continue
        nodes = [0] + [int(v) for v in g_path[b, :g_len[b]]]
        n_tgt += len(nodes)
        if not greedy[b]:
            n_drf += sum(1 for v in nodes if v < K and has_kids[v])
    alg = (n_tgt + n_drf) * V * wl.elem_size
    line = _op_line(args, "tree-verified rows/s, V=%d" % V, B / (ms * 1e-3), ms,
                    "f32" if wl.dtype == "f32" else "bf16",
                    {"workload": wl.name, "vocab": V, "batch": B, "candidates": K,
                     "tree": "medusa 3-2-1", "logits": wl.dtype, "max_depth": max_depth,
                     "max_children": max_kids},
                    alg, "whole call (sv_verify_tree)")
    line["mean_accepted"] = round(float(g_len[g_len >= 0].mean()), 3)
    line["rows_read"] = {"target": int(n_tgt), "draft": int(n_drf)}
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        sel = np.arange(0, B, 16)
        tc = time.perf_counter()
        r_tok, r_len, r_path, _, used = oracle.verify_tree(
            wl.target[sel], wl.draft[sel], wl.tokens[sel], par[sel], wl.draft_len[sel],
            wl.params[sel], wl.uniforms[sel], dtype=wl.dtype, nthreads=1)
        dt = time.perf_counter() - tc
        line["cpu_baseline"] = {"value": round(len(sel) / dt, 2), "unit": "rows/s",
                                "cores": int(used), "kind": "oracle",
                                "sample": f"{len(sel)} rows (every 16th), one thread, {dt:.2f} s"}
        same = (r_len == g_len[sel]) & (r_tok == g_tok[sel]).all(axis=1)
        line["oracle_agreement"] = {"rows": int(len(sel)), "identical": int(same.sum())}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--replicas", type=int, default=1,
                    help="copies of the headline inputs to rotate over")
    ap.add_argument("--no-extras", action="store_true", help="measure the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", default="verify", choices=["verify", "accept_stats", "sample", "tree"])
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
    from rejection_sampling_verify_sv_amd import workloads

    dev = torch.device("cuda:0")
    sv.load()
    if args.op == "tree":
        bench_tree(args, dev)
        return
    log(f"[bench] generating {args.workload}")
    wl = workloads.make(args.workload)
    if args.op == "accept_stats":
        bench_accept_stats(args, wl, dev)
        return
    if args.op == "sample":
        bench_sample(args, wl, dev)
        return
    log("[bench] streaming-read ceiling")
    ceil = read_ceiling(dev)
    log(f"[bench] ceiling {ceil['GBps']} GB/s; timing {args.workload}: warmup {args.warmup}, "
        f"{args.steps} steps")
    res, acc, tok = measure(wl, dev, args.steps, args.warmup, replicas=args.replicas,
                            ceiling=ceil["GBps"])
    line = {
        "metric": res["metric"],
        "value": res["value"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic",
        "config": res["config"],
        "roofline": res["roofline"],
        "whole_step": res["whole_step"],
        "read_ceiling": ceil,
        "kernels_ms_per_step": res["kernels_ms_per_step"],
        "rowpass_by_position": res["rowpass_by_position"],
        "cut_decide_ms_by_launch": res["cut_decide_ms_by_launch"],
        "acceptance_rate": res["acceptance_rate"],
        "verify_calls": res["verify_calls"],
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
        torch.cuda.empty_cache()
    if not args.no_extras:
        configs = []
        for name, batch, reps in EXTRAS:
            log(f"[bench] extra workload {name} batch={batch or 'full'} replicas={reps}")
            w = workloads.make(name, batch=batch)
            r, _, _ = measure(w, dev, args.steps, args.warmup, replicas=reps,
                              ceiling=ceil["GBps"])
            r["latency_us"] = round(r["ms_per_step"] * 1e3, 1)
            configs.append(r)
            del w
        line["configs"] = configs
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on host cores)")
        cb, agree = cpu_baseline(wl, acc, tok)
        line["cpu_baseline"] = cb
        line["oracle_agreement"] = agree
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
