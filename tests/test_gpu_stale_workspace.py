"""Workspace reuse: a call's outputs depend on its inputs only, never on what
an earlier call left in the workspace.

Each case runs one batch on a zeroed workspace, then a different batch of the
same shape (its rows rolled by a few places, so every row slot changes its
sampler class, draft length and logits) on that same workspace, then the
first batch again: the last run must match the first bit for bit, and the
middle one the rolled batch's own run on a zeroed workspace.  The stale
contents are what a real call of that shape writes, so every list index and
count the kernels could read is one a call of that shape produces.
"""
import dataclasses
import sys

import numpy as np
import pytest

from rejection_sampling_verify_sv_amd import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _rolled(wl, s):
    r = lambda x: np.roll(x, s, axis=0)
    return dataclasses.replace(wl, target=r(wl.target), draft=r(wl.draft), tokens=r(wl.tokens),
                               draft_len=r(wl.draft_len), params=r(wl.params),
                               uniforms=r(wl.uniforms), name=wl.name + f"_roll{s}")


def _run(wl, dev, ws, mode):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    tok, acc, dg = sv.verify(*workloads.to_torch(wl, dev), diag=True, workspace=ws,
                             step_mode=mode)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), acc.cpu().numpy(), dg.cpu().numpy()


def _same(x, y, what):
    for i, (p, q) in enumerate(zip(x, y)):
        if not np.array_equal(p, q, equal_nan=True):
            bad = np.nonzero(~((p == q) | (np.isnan(p) & np.isnan(q))))[0]
            raise AssertionError(f"{what}: output {i} differs in rows {np.unique(bad)[:8]}")


CASES = [
    ("mixed_samplers_b1024", 96, 20011, "auto"),       # dense step
    ("mixed_samplers_b1024", 96, 20011, "positions"),
    ("mixed_samplers_b1024", 1100, 3001, "auto"),      # merged launch, plan of two workgroups
    ("fullvocab_ragged_b256", 64, 20011, "auto"),
    ("fullvocab_ragged_b256", 600, 2047, "positions"),
    ("mixed_greedy_b64", 64, 9000, "auto"),
    ("mixed_samplers_b1024", 300, 1000, "auto"),       # short rows, one wave per unit
]


@pytest.mark.parametrize("name,batch,vocab,mode", CASES,
                         ids=[f"{n}_b{b}_v{v}_{m}" for n, b, v, m in CASES])
def test_verify_on_a_stale_workspace(dev, name, batch, vocab, mode):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl = workloads.make(name, batch=batch, vocab=vocab)
    other = _rolled(wl, 3)
    code = sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16
    need = sv.workspace_bytes(wl.B, wl.K, wl.V, code) + 256
    _say(f"[gpu] stale workspace: {name} B={wl.B} V={wl.V} {wl.dtype} {mode}")
    fresh = _run(wl, dev, torch.zeros(need, dtype=torch.uint8, device=dev), mode)
    fresh_other = _run(other, dev, torch.zeros(need, dtype=torch.uint8, device=dev), mode)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    _same(_run(wl, dev, ws, mode), fresh, "first run")
    _same(_run(other, dev, ws, mode), fresh_other, "rolled batch after the first")
    _same(_run(wl, dev, ws, mode), fresh, "first batch after the rolled one")


def test_tree_on_a_stale_workspace(dev):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl, par = workloads.make_tree(batch=24, vocab=20011, K=12, shape="medusa", dtype="bf16")
    other = _rolled(wl, 5)
    par_o = np.roll(par, 5, axis=0)
    need = sv.workspace_bytes(wl.B, wl.K, wl.V, sv.SV_BF16) + 256
    depth = np.zeros(wl.K + 1, np.int64)
    for c in range(1, wl.K + 1):
        depth[c] = depth[par[0, c - 1]] + 1
    max_depth = int(depth.max())
    max_kids = int(np.bincount(par[0], minlength=wl.K + 1).max())

    def run(w, p, ws):
        t, d, tok, _, prm, uni = workloads.to_torch(w, dev)
        out = sv.verify_tree(t, d, tok, torch.from_numpy(np.ascontiguousarray(p)).to(dev),
                             torch.from_numpy(np.ascontiguousarray(w.draft_len)).to(dev), prm, uni,
                             max_depth=max_depth, max_children=max_kids, diag=True, workspace=ws)
        torch.cuda.synchronize()
        return tuple(x.cpu().numpy() for x in out)

    _say(f"[gpu] stale workspace: tree B={wl.B} K={wl.K} V={wl.V}")
    fresh = run(wl, par, torch.zeros(need, dtype=torch.uint8, device=dev))
    fresh_o = run(other, par_o, torch.zeros(need, dtype=torch.uint8, device=dev))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    _same(run(wl, par, ws), fresh, "tree first run")
    _same(run(other, par_o, ws), fresh_o, "tree rolled batch")
    _same(run(wl, par, ws), fresh, "tree first batch again")


def test_sample_on_a_stale_workspace(dev):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl = workloads.make("mixed_samplers_b1024", batch=200, vocab=20011)
    other = _rolled(wl, 7)
    need = sv.workspace_bytes(wl.B, 0, wl.V, sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16) + 256

    def run(w, ws):
        t, _, _, _, prm, uni = workloads.to_torch(w, dev)
        out = sv.sample(t[:, 0], prm, uni[:, 0].contiguous(), diag=True, workspace=ws)
        torch.cuda.synchronize()
        return tuple(x.cpu().numpy() for x in out)

    _say(f"[gpu] stale workspace: sample B={wl.B} V={wl.V}")
    fresh = run(wl, torch.zeros(need, dtype=torch.uint8, device=dev))
    fresh_o = run(other, torch.zeros(need, dtype=torch.uint8, device=dev))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    _same(run(wl, ws), fresh, "sample first run")
    _same(run(other, ws), fresh_o, "sample rolled batch")
    _same(run(wl, ws), fresh, "sample first batch again")


def test_accept_stats_on_a_stale_workspace(dev):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl = workloads.make("mixed_samplers_b1024", batch=150, vocab=20011)
    other = _rolled(wl, 11)
    code = sv.SV_F32 if wl.dtype == "f32" else sv.SV_BF16
    need = sv.workspace_bytes(wl.B, 1, wl.V, code) + 256

    def run(w, ws):
        t, d, _, _, prm, _ = workloads.to_torch(w, dev)
        out = sv.accept_stats(t[:, 0], d[:, 0], prm, workspace=ws)
        torch.cuda.synchronize()
        return (out.cpu().numpy(),)

    _say(f"[gpu] stale workspace: accept_stats B={wl.B} V={wl.V}")
    fresh = run(wl, torch.zeros(need, dtype=torch.uint8, device=dev))
    fresh_o = run(other, torch.zeros(need, dtype=torch.uint8, device=dev))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    _same(run(wl, ws), fresh, "accept_stats first run")
    _same(run(other, ws), fresh_o, "accept_stats rolled batch")
    _same(run(wl, ws), fresh, "accept_stats first batch again")
