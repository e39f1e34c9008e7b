"""GPU parity of the acceptance statistics of one draft position
(sv_accept_stats) against the fp64 oracle (oracle.accept_stats).

Bar: the four sums agree within 2e-6 absolute.  The GPU forms every weight
from one fp32 exp2 (relative error about 2.4e-7) and adds in fp64, and each
sum is at most 1.  NaN on exactly the oracle's NaN rows, and on rows with a
top_k this build does not serve.  A row whose truncation the oracle reports
within 1e-6 of a tie in mass (its cut margin) may keep one token more or less
on the GPU; such rows are counted and skipped for the truncated sums.
"""
import sys
import zlib

import numpy as np
import pytest

from rejection_sampling_verify_sv_amd import workloads
from rejection_sampling_verify_sv_amd.workloads import PARAMS_DTYPE

pytestmark = pytest.mark.gpu

TOL = 2e-6


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need cuda:0"
    import rejection_sampling_verify_sv_amd as sv

    sv.load()
    return torch.device("cuda:0")


def _t(rows, dtype, dev):
    import torch

    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(rows)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(torch.bfloat16)


def _gpu(t, d, params, dev):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    out = sv.accept_stats(t, d, sv.params_tensor(params, dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(g, ref, margin, params, label, V):
    unsup = (params["top_k"] > sv_max_top_k()) & (params["top_k"] < V) & (params["temperature"] > 0)
    near = margin < 1e-6
    n_cmp = 0
    for b in range(len(params)):
        if unsup[b]:
            assert np.isnan(g[b]).all(), (label, b, g[b])
            continue
        if np.isnan(ref[b]).any():
            assert np.isnan(g[b]).all(), (label, b, g[b], ref[b])
            continue
        cols = [2, 3] if near[b] else [0, 1, 2, 3]
        err = np.abs(g[b, cols] - ref[b, cols])
        assert (err <= TOL).all(), (label, b, g[b], ref[b], params[b])
        n_cmp += 1
    _say(f"[gpu] {label}: {n_cmp} rows compared, {int(near.sum())} near a cut tie, "
         f"{int(unsup.sum())} unsupported")
    return n_cmp


def sv_max_top_k():
    import rejection_sampling_verify_sv_amd as sv

    return sv.SV_MAX_TOP_K


SAMPLERS = [
    (0.0, 0, 1.0), (1.0, 20, 0.95), (0.7, 50, 0.9), (1.0, 0, 1.0), (1.2, 0, 1.0),
    (1.0, 0, 0.8), (0.6, 0, 0.95), (1.0, 1, 1.0), (1.0, 64, 1.0), (1.0, 300, 1.0),
]


def _mixed(seed, B, V, dtype):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 2.0, (B, V))
    d = 0.8 * t + rng.normal(0, 1.2, (B, V))
    prm = np.zeros(B, PARAMS_DTYPE)
    pick = rng.integers(0, len(SAMPLERS), B)
    for b in range(B):
        prm[b]["temperature"], prm[b]["top_k"], prm[b]["top_p"] = SAMPLERS[pick[b]]
    if dtype == "f32":
        return t.astype(np.float32), d.astype(np.float32), prm
    bf = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bf(t), bf(d), prm


@pytest.mark.parametrize("dtype,V", [("f32", 30011), ("bf16", 20011), ("f32", 4096),
                                     ("f32", 1000), ("bf16", 2048), ("f32", 61)])
def test_mixed_samplers(oracle_mod, dev, dtype, V):
    B = 96
    t, d, prm = _mixed(zlib.crc32(f"acc{dtype}{V}".encode()), B, V, dtype)
    _say(f"[gpu] accept_stats mixed {dtype} B={B} V={V}")
    g = _gpu(_t(t, dtype, dev), _t(d, dtype, dev), prm, dev)
    ref, margin = oracle_mod.accept_stats(t, d, prm, dtype=dtype)
    assert _check(g, ref, margin, prm, f"mixed_{dtype}_V{V}", V) > B // 2


def test_many_rows(oracle_mod, dev):
    """2500 rows: the plan splits them over three classifying workgroups."""
    B, V = 2500, 257
    t, d, prm = _mixed(zlib.crc32(b"acc_many_rows"), B, V, "f32")
    g = _gpu(_t(t, "f32", dev), _t(d, "f32", dev), prm, dev)
    ref, margin = oracle_mod.accept_stats(t, d, prm, dtype="f32")
    assert _check(g, ref, margin, prm, "many_rows_f32", V) > B // 2


def test_one_workgroup_per_unit(oracle_mod, dev):
    """160 nucleus rows (320 units): the cut runs one workgroup per unit."""
    B, V = 160, 8192
    rng = np.random.default_rng(5)
    t = rng.normal(0, 2.0, (B, V)).astype(np.float32)
    d = (0.8 * t + rng.normal(0, 1.2, (B, V))).astype(np.float32)
    prm = np.zeros(B, PARAMS_DTYPE)
    prm["temperature"], prm["top_k"], prm["top_p"] = 1.0, 0, 0.9
    g = _gpu(_t(t, "f32", dev), _t(d, "f32", dev), prm, dev)
    ref, margin = oracle_mod.accept_stats(t, d, prm)
    assert _check(g, ref, margin, prm, "nucleus_one_wg_per_unit", V) > B - 4


def test_full_size_position_0(oracle_mod, dev):
    """The 1024-row mix at V = 151936: position 0 of its target and draft
    tensors (strided rows), every row on the GPU, a sample on the oracle."""
    import torch

    wl = workloads.make("mixed_samplers_b1024")
    t, d, _, _, _, _ = workloads.to_torch(wl, dev)
    g = _gpu(t[:, 0, :], d[:, 0, :], wl.params, dev)
    rows = np.sort(np.random.default_rng(17).choice(wl.B, size=24, replace=False))
    ref, margin = oracle_mod.accept_stats(wl.target[rows, 0], wl.draft[rows, 0], wl.params[rows])
    _check(g[rows], ref, margin, wl.params[rows], "mixed_samplers_b1024_pos0", wl.V)
    finite = np.isfinite(g).all(axis=1)
    assert finite.sum() == wl.B
    assert (g[:, 0] <= 1 + 1e-9).all() and (g >= -1e-12).all()
    del torch


def test_edges(oracle_mod, dev):
    """Invalid parameters, a side with no finite logit, greedy ties (lowest
    id), identical rows, and rows that are not 16-byte aligned."""
    B, V = 12, 5003
    rng = np.random.default_rng(8)
    t = rng.normal(0, 1.0, (B, V)).astype(np.float32)
    d = t.copy()
    d[1::2] += rng.normal(0, 0.5, (B // 2, V)).astype(np.float32)
    prm = np.zeros(B, PARAMS_DTYPE)
    prm["temperature"], prm["top_k"], prm["top_p"] = 1.0, 0, 0.9
    prm["temperature"][0] = -1.0
    prm["top_p"][1] = 0.0
    t[2, :] = -np.inf
    prm["temperature"][3] = 0.0
    t[3, :] = 0.0
    d[3, :] = 0.0          # all tied: both argmaxes are id 0
    prm["temperature"][5] = 0.0
    t[5, 7] = 50.0
    d[5, 9] = 50.0          # argmaxes differ
    prm["top_k"][6] = 20
    g = _gpu(_t(t, "f32", dev), _t(d, "f32", dev), prm, dev)
    ref, margin = oracle_mod.accept_stats(t, d, prm)
    _check(g, ref, margin, prm, "edges", V)
    assert np.isnan(g[0]).all() and np.isnan(g[1]).all() and np.isnan(g[2]).all()
    assert (g[3] == 1.0).all() and (g[5] == 0.0).all()
    assert abs(g[4, 0] - 1.0) < TOL  # identical rows
    # not 16-byte aligned: rows start one element into a padded buffer
    import torch

    pad_t = torch.zeros((B, V + 1), dtype=torch.float32, device=dev)
    pad_d = torch.zeros((B, V + 1), dtype=torch.float32, device=dev)
    pad_t[:, 1:] = _t(t, "f32", dev)
    pad_d[:, 1:] = _t(d, "f32", dev)
    g2 = _gpu(pad_t[:, 1:], pad_d[:, 1:], prm, dev)
    np.testing.assert_array_equal(np.isnan(g2), np.isnan(g))
    np.testing.assert_allclose(g2[~np.isnan(g)], g[~np.isnan(g)], atol=1e-12)
