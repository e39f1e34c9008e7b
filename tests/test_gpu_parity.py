"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test builds seeded inputs with the shared input module, runs libsv.so on
cuda:0 and the oracle on the host, and applies the bar of tests/parity.py:
identical tokens and accept lengths except where the GPU's outcome is what the
rule gives for uniforms within 1e-5 of the ones passed in (counted per sampler
class; never on greedy or top-k rows), diagnostics within 1e-5.  Every row is
compared, the five recipes at their full sizes included.
"""
import sys
import zlib

import numpy as np
import pytest

from rejection_sampling_verify_sv_amd import _lib, workloads
from rejection_sampling_verify_sv_amd.workloads import PARAMS_DTYPE
from tests.parity import compare, subset

pytestmark = pytest.mark.gpu


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


def modes_for(B, K):
    """Step modes a batch shape is served in: position by position always,
    the dense step when 2 B (K+1) <= 1024."""
    return ["positions", "dense"] if 2 * B * (K + 1) <= 1024 else ["positions"]


def run_gpu(wl, dev, diag=True, step_mode="auto"):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    tok, acc, dg = sv.verify(*workloads.to_torch(wl, dev), diag=diag, step_mode=step_mode)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), acc.cpu().numpy(),
            dg.cpu().numpy() if dg is not None else None)


def run_oracle(oracle_mod, wl, rows=None):
    if rows is None:
        return oracle_mod.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params,
                                 wl.uniforms, dtype=wl.dtype)
    rows = np.asarray(rows)
    return oracle_mod.verify(wl.target[rows], wl.draft[rows], wl.tokens[rows],
                             wl.draft_len[rows], wl.params[rows], wl.uniforms[rows],
                             dtype=wl.dtype)


def check(oracle_mod, wl, dev, rows=None, label="", step_mode="auto"):
    label = f"{label or wl.name}[{step_mode}]"
    _say(f"[gpu] {label}: B={wl.B} K={wl.K} V={wl.V} {wl.dtype}")
    g_tok, g_acc, g_diag = run_gpu(wl, dev, step_mode=step_mode)
    ref = run_oracle(oracle_mod, wl, rows)
    rep = compare(g_tok, g_acc, g_diag, ref, rows,
                  inputs=wl if rows is None else subset(wl, rows), oracle_mod=oracle_mod)
    _say(f"[gpu] {label}: {rep.describe()}")
    assert rep.tight_ok, rep.describe()
    # greedy and top-k rows decide in fp64 from exact selections: no outcome
    # may differ there, in band or not
    assert rep.mismatch_in_band_by_class.get("top_k", 0) == 0, rep.describe()
    return rep, g_tok, g_acc


RECIPES = ["tiny_v1000", "decode_b1", "mixed_greedy_b64", "fullvocab_ragged_b256",
           "mixed_samplers_b1024"]


@pytest.mark.parametrize("name", RECIPES)
def test_recipe_parity(oracle_mod, dev, name):
    # every row of each recipe at its full size (tiny_v1000: 10,000 steps), in
    # the mode the library picks (dense for the two small batches)
    wl = workloads.make(name, poison=(name == "fullvocab_ragged_b256"))
    rep, _, _ = check(oracle_mod, wl, dev)
    assert rep.compared == wl.B
    assert rep.unsupported == 0


@pytest.mark.parametrize("name", ["decode_b1", "mixed_greedy_b64"])
def test_small_recipes_position_by_position(oracle_mod, dev, name):
    wl = workloads.make(name)
    rep, _, _ = check(oracle_mod, wl, dev, step_mode="positions")
    assert rep.compared == wl.B


@pytest.mark.parametrize("name,batch,vocab", [("mixed_samplers_b1024", 120, 30011),
                                              ("fullvocab_ragged_b256", 100, 20011),
                                              ("mixed_greedy_b64", None, None),
                                              ("decode_b1", None, None)])
def test_dense_matches_positions(dev, name, batch, vocab):
    """The dense step and the position-by-position step give bitwise the same
    outputs and diagnostics (the records they merge are the same: per (tile,
    wave) for untruncated rows, exact keys and fixed-point histograms
    otherwise).  At these batches the decision launch has a workgroup for
    every row, so the dense step decides each row's positions side by side
    and walks them in order afterwards; the position-by-position step never
    does."""
    wl = workloads.make(name, batch=batch, vocab=vocab)
    a = run_gpu(wl, dev, step_mode="positions")
    b = run_gpu(wl, dev, step_mode="dense")
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    _say(f"[gpu] dense == positions on {name} B={wl.B} V={wl.V}")


@pytest.mark.parametrize("name,batch,vocab,d0", [("mixed_samplers_b1024", 700, 4099, 2),
                                                 ("fullvocab_ragged_b256", 300, 5003, 1)])
def test_merged_matches_positions(dev, name, batch, vocab, d0):
    """Larger batches merge their last positions into one launch pair (from
    position d0 on); that step and the position-by-position one give bitwise
    the same outputs and diagnostics, like the dense step."""
    wl = workloads.make(name, batch=batch, vocab=vocab)
    auto = _lib.launch_names(wl.B, wl.K, "auto")
    assert auto.count("rowpass") == d0 + 1  # the merge applies at this shape
    a = run_gpu(wl, dev, step_mode="positions")
    b = run_gpu(wl, dev, step_mode="auto")
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    _say(f"[gpu] merged from {d0} == positions on {name} B={wl.B} V={wl.V}")


@pytest.mark.parametrize("name", ["mixed_greedy_b64", "fullvocab_ragged_b256",
                                  "mixed_samplers_b1024"])
def test_recipe_small_vocab_every_row(oracle_mod, dev, name):
    # same recipes at a vocabulary the oracle finishes quickly on every row;
    # 20011 is not a multiple of any tile, so the ragged tail is exercised
    wl = workloads.make(name, batch=96, vocab=20011)
    check(oracle_mod, wl, dev, label=f"{name}@V=20011")


def test_unit_aligned_grid_every_row(oracle_mod, dev):
    # 160 rows of the mix at V = 151936: position 0 holds about 290 units of
    # 38 tiles, so the row pass (1024 resident workgroups) takes the
    # unit-aligned grid (three workgroups per unit, one piece each); every
    # row is compared, of every sampler class
    wl = workloads.make("mixed_samplers_b1024", batch=160)
    rep, _, _ = check(oracle_mod, wl, dev, label="unit_aligned_b160")
    assert rep.compared > 100


def _random_case(rng, B, K, V, dtype, T, top_k, top_p, scale=2.0, quant=None, draft_len=None,
                 noise=0.6):
    t = rng.normal(0, scale, (B, K + 1, V))
    d = t[:, :K] * 0.8 + rng.normal(0, scale * noise, (B, K, V))
    if quant:
        t, d = np.round(t * quant) / quant, np.round(d * quant) / quant
    prm = np.zeros(B, PARAMS_DTYPE)
    prm["temperature"], prm["top_k"], prm["top_p"] = T, top_k, top_p
    L = np.full(B, K, np.int32) if draft_len is None else draft_len
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        for k in range(K):
            tok[b, k] = int(np.argmax(d[b, k] / max(T, 1e-3) + rng.gumbel(size=V)))
    u = rng.random((B, K + 1), dtype=np.float32)
    return workloads.custom(t, d, tok, L, prm, u, dtype=dtype)


def test_split_units_on_a_dirty_workspace(oracle_mod, dev):
    """A dense step of 8 nucleus rows at K = 7 holds 120 nucleus units in one
    launch; each is cut by several workgroups, which count their arrivals in
    per-unit counters indexed by the unit's place in the list (up to 119, past
    2 B).  The workspace comes in filled with a byte pattern: the plan clears
    every counter a launch can use, so the outputs match the oracle and, bit
    for bit, a run on a zeroed workspace."""
    import torch

    import rejection_sampling_verify_sv_amd as sv

    rng = np.random.default_rng(8107)
    wl = _random_case(rng, 8, 7, 20011, "f32", 1.0, 0, 0.9)
    code = sv.SV_F32
    need = sv.workspace_bytes(wl.B, wl.K, wl.V, code) + 256
    outs = []
    for fill in (1, 0):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=dev)
        tok, acc, dg = sv.verify(*workloads.to_torch(wl, dev), diag=True, workspace=ws,
                                 step_mode="dense")
        torch.cuda.synchronize()
        outs.append((tok.cpu().numpy(), acc.cpu().numpy(), dg.cpu().numpy()))
    for x, y in zip(*outs):
        assert np.array_equal(x, y, equal_nan=True)
    rep = compare(*outs[0], run_oracle(oracle_mod, wl), None, inputs=wl, oracle_mod=oracle_mod)
    _say(f"[gpu] dirty workspace, 120 split nucleus units: {rep.describe()}")
    assert rep.tight_ok, rep.describe()
    assert rep.compared == wl.B


def _mixed_case(seed, wide=False, short=False):
    """A seeded batch whose rows each draw their own sampler (greedy, top-k up
    to 64, top-k above 64 (not served), untruncated, nucleus), temperature,
    draft length and logit scale; drafts are sampled from the untruncated
    tempered draft, so some fall outside q.  wide: larger batches, drafts
    and vocabularies, more nucleus rows, and logits rounded to a grid on some
    batches (many ties).  short: rows that fit one wave's loads (up to 1024
    fp32 or 2048 bf16 tokens) and a token past either limit, batches from
    one row to 1100."""
    rng = np.random.default_rng((9001 if wide else 7707 if short else 5150) + seed)
    if short:
        B = int(rng.choice([1, 9, 64, 300, 1100], p=[0.15, 0.2, 0.2, 0.25, 0.2]))
        K = int(rng.integers(1, 5))
        dtype = "bf16" if rng.random() < 0.5 else "f32"
        V = int(rng.choice([2, 7, 64, 333, 1000, 1021, 1024, 1025] if dtype == "f32"
                           else [5, 64, 999, 2047, 2048, 2049]))
        probs = [0.2, 0.3, 0.05, 0.2, 0.25]
    elif wide:
        B = int(rng.choice([3, 64, 130, 300, 600], p=[0.1, 0.2, 0.25, 0.25, 0.2]))
        K = int(rng.integers(1, 8))
        V = int(rng.choice([2048, 30011, 65543]))
        while B * (K + 1) * V > 40_000_000:
            V = 2048 if V == 30011 else 30011
        probs = [0.1, 0.2, 0.05, 0.2, 0.45]
    else:
        B = int(rng.choice([5, 37, 90, 150, 260], p=[0.15, 0.25, 0.2, 0.2, 0.2]))
        K = int(rng.integers(1, 7))
        V = int(rng.choice([3001, 9000, 20011]))
        probs = [0.2, 0.3, 0.05, 0.2, 0.25]
    if not short:
        dtype = "bf16" if rng.random() < 0.5 else "f32"
    scale = float(rng.choice([1.0, 3.0]))
    t = rng.normal(0, scale, (B, K + 1, V))
    d = t[:, :K] * 0.8 + rng.normal(0, scale * 0.6, (B, K, V))
    if wide and rng.random() < 0.3:
        t, d = np.round(t * 4) / 4, np.round(d * 4) / 4
    prm = np.zeros(B, PARAMS_DTYPE)
    kind = rng.choice(5, size=B, p=probs)
    for b in range(B):
        T = float(rng.uniform(0.3, 1.6))
        if kind[b] == 0:
            prm[b] = (0.0, 0, 1.0, 0)
        elif kind[b] == 1:
            prm[b] = (T, int(rng.integers(1, 65)), float(rng.choice([1.0, 0.9, 0.6])), 0)
        elif kind[b] == 2 and V > 66:
            prm[b] = (T, int(rng.integers(65, V)), 1.0, 0)
        elif kind[b] == 2:
            prm[b] = (T, int(rng.integers(1, V + 1)), 1.0, 0)
        elif kind[b] == 3:
            prm[b] = (T, int(rng.choice([0, V])), 1.0, 0)
        else:
            prm[b] = (T, 0, float(rng.uniform(0.5, 0.99)), 0)
    L = rng.integers(0, K + 1, size=B).astype(np.int32)
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        T = max(float(prm["temperature"][b]), 1e-3)
        for k in range(K):
            tok[b, k] = int(np.argmax(d[b, k] / T + rng.gumbel(size=V)))
    u = rng.random((B, K + 1), dtype=np.float32)
    tag = "wide_" if wide else "short_" if short else ""
    return workloads.custom(t, d, tok, L, prm, u, dtype=dtype, name=f"mixed_sweep_{tag}{seed}")


@pytest.mark.parametrize("seed", range(12))
def test_mixed_rows_sweep(oracle_mod, dev, seed):
    """Every sampler class, draft length and temperature mixed in one batch,
    at batch shapes that take the dense, merged and position-by-position
    steps; every row against the oracle in the library's own mode and
    position by position."""
    wl = _mixed_case(seed)
    for mode in ("auto", "positions"):
        rep, _, _ = check(oracle_mod, wl, dev, label=wl.name, step_mode=mode)
        assert rep.compared + rep.unsupported == wl.B


@pytest.mark.parametrize("seed", range(16))
def test_mixed_rows_sweep_wide(oracle_mod, dev, seed):
    """The same at up to 600 rows, seven drafts and V = 65543, with more
    nucleus rows and, on some batches, logits on a grid of 1/4 (ties)."""
    wl = _mixed_case(seed, wide=True)
    modes = ["auto", "positions"] + (["dense"] if 2 * wl.B * (wl.K + 1) <= 1024 else [])
    for mode in modes:
        rep, _, _ = check(oracle_mod, wl, dev, label=wl.name, step_mode=mode)
        assert rep.compared + rep.unsupported == wl.B


@pytest.mark.parametrize("seed", range(12))
def test_short_rows_sweep(oracle_mod, dev, seed):
    """Rows short enough for one wave's loads, where the row pass gives each
    wave a unit of its own (nucleus units keep the whole workgroup), with
    every sampler class mixed in, in every step mode the batch takes."""
    wl = _mixed_case(seed, short=True)
    modes = ["auto", "positions"] + (["dense"] if 2 * wl.B * (wl.K + 1) <= 1024 else [])
    for mode in modes:
        rep, _, _ = check(oracle_mod, wl, dev, label=f"{wl.name} V={wl.V} {wl.dtype}",
                          step_mode=mode)
        assert rep.compared + rep.unsupported == wl.B


EDGE = [
    # label, B, K, V, dtype, T, top_k, top_p, extra
    ("tiny_vocab_topk", 64, 2, 7, "f32", 1.0, 3, 0.9, {}),
    ("vocab_below_tile_bf16", 64, 3, 5000, "bf16", 0.8, 20, 0.95, {}),
    ("ragged_tail_f32", 64, 2, 12345, "f32", 1.0, 50, 0.9, {}),
    ("top_k_64", 48, 2, 30000, "f32", 1.0, 64, 1.0, {}),
    ("top_k_1", 48, 2, 30000, "bf16", 0.7, 1, 0.5, {}),
    ("heavy_ties_bf16", 48, 3, 40000, "bf16", 1.0, 20, 0.95, {"quant": 2}),
    ("all_equal_logits", 16, 2, 9000, "f32", 1.0, 10, 1.0, {"scale": 0.0}),
    ("full_vocab_untruncated_f32", 48, 3, 30011, "f32", 0.9, 0, 1.0, {}),
    ("full_vocab_top_k_ge_V", 32, 2, 3000, "bf16", 1.1, 3000, 1.0, {}),
    ("greedy_rows", 64, 4, 50000, "bf16", 0.0, 20, 0.95, {"quant": 4}),
    ("nucleus_f32", 64, 3, 30011, "f32", 1.0, 0, 0.9, {}),
    ("nucleus_bf16_ties", 64, 2, 50000, "bf16", 0.7, 0, 0.95, {"quant": 4}),
    ("nucleus_low_T", 48, 2, 20000, "f32", 0.3, 0, 0.8, {}),
    ("nucleus_tiny_top_p", 32, 2, 10000, "f32", 1.0, 0, 1e-3, {}),
    ("nucleus_all_equal", 16, 2, 3000, "f32", 1.0, 0, 0.5, {"scale": 0.0}),
    ("nucleus_top_k_ge_V", 32, 2, 4000, "bf16", 1.2, 5000, 0.7, {}),
    # boundary buckets beyond the LDS collect capacity: the radix-select path
    ("nucleus_wide_all_equal", 16, 2, 20011, "f32", 1.0, 0, 0.6, {"scale": 0.0}),
    ("nucleus_wide_flat_f32", 24, 2, 151936, "f32", 2.0, 0, 0.8, {"scale": 0.1}),
    ("nucleus_wide_ties_bf16", 24, 2, 90000, "bf16", 8.0, 0, 0.8, {"scale": 0.5, "quant": 64}),
    ("nucleus_wide_T50", 24, 3, 90001, "f32", 50.0, 0, 0.9, {}),
]


EDGE_MODES = [e + (m,) for e in EDGE for m in modes_for(e[1], e[2])]


@pytest.mark.parametrize("label,B,K,V,dtype,T,top_k,top_p,extra,mode", EDGE_MODES,
                         ids=[f"{e[0]}-{e[-1]}" for e in EDGE_MODES])
def test_edge_cases(oracle_mod, dev, label, B, K, V, dtype, T, top_k, top_p, extra, mode):
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    wl = _random_case(rng, B, K, V, dtype, T, top_k, top_p, **extra)
    rep, _, _ = check(oracle_mod, wl, dev, label=label, step_mode=mode)
    assert rep.unsupported == 0 and rep.compared == B


@pytest.mark.parametrize("mode", ["positions", "dense"])
def test_ragged_draft_len_and_zero(oracle_mod, dev, mode):
    rng = np.random.default_rng(5)
    L = rng.integers(0, 4, 80).astype(np.int32)
    wl = _random_case(rng, 80, 3, 20000, "bf16", 1.0, 20, 0.9, draft_len=L)
    wl.params["top_k"][::3] = 0   # and nucleus rows
    wl.params["top_p"][1::6] = 1.0
    wl.params["temperature"][2::5] = 0.0
    check(oracle_mod, wl, dev, label="ragged_draft_len", step_mode=mode)


@pytest.mark.parametrize("mode", ["positions", "dense"])
def test_invalid_rows(oracle_mod, dev, mode):
    rng = np.random.default_rng(6)
    wl = _random_case(rng, 12, 2, 3000, "f32", 1.0, 20, 0.9)
    wl.params["temperature"][1] = -1.0
    wl.params["temperature"][2] = np.nan
    wl.params["top_p"][3] = 0.0
    wl.draft_len[4] = 3
    wl.tokens[5, 1] = 3000
    wl.tokens[6, 0] = -4
    wl.draft_len[7] = -1
    wl.target[8, :, :] = -np.inf
    rep, g_tok, g_acc = check(oracle_mod, wl, dev, label="invalid_rows", step_mode=mode)
    assert g_acc[1:9].tolist() == [-1] * 8
    assert (g_tok[1:9] == -1).all()


@pytest.mark.parametrize("mode", ["auto", "positions"])
def test_plan_of_several_workgroups(oracle_mod, dev, mode):
    """3000 rows (the plan's rows split over three classifying workgroups,
    each counting the units of the rows before its own): every sampler
    class, unsupported rows and invalid rows spread over the batch, each
    row's list position checked through its outcome against the oracle."""
    rng = np.random.default_rng(61)
    B, K, V = 3000, 2, 333
    t = rng.normal(0, 2.0, (B, K + 1, V))
    d = t[:, :K] * 0.8 + rng.normal(0, 1.2, (B, K, V))
    prm = np.zeros(B, PARAMS_DTYPE)
    kind = rng.integers(0, 5, B)
    for b in range(B):
        T = float(rng.uniform(0.4, 1.4))
        prm[b] = [(0.0, 0, 1.0, 0), (T, int(rng.integers(1, 65)), 0.9, 0), (T, 100, 1.0, 0),
                  (T, 0, 1.0, 0), (T, 0, float(rng.uniform(0.5, 0.99)), 0)][kind[b]]
    L = rng.integers(0, K + 1, size=B).astype(np.int32)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    bad = rng.choice(B, size=60, replace=False)
    for i, b in enumerate(bad):  # invalid rows, in every workgroup's share
        if i % 4 == 0:
            prm[b]["temperature"] = -1.0
        elif i % 4 == 1:
            prm[b]["top_p"] = 0.0
        elif i % 4 == 2:
            L[b] = K + 1
        else:
            L[b] = K
            tok[b, K - 1] = V
    u = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.custom(t, d, tok, L, prm, u, dtype="f32", name="plan_3000_rows")
    rep, g_tok, g_acc = check(oracle_mod, wl, dev, label="plan_3000_rows", step_mode=mode)
    assert rep.compared + rep.unsupported == B
    assert (g_acc[bad] == -1).all()
    assert (g_acc[kind == 2] == -2).sum() == int(((kind == 2) & ~np.isin(np.arange(B), bad)).sum())


@pytest.mark.parametrize("case", ["bf16_zipf", "f32_grid_jitter"])
def test_boundary_sub_bucket_crowded(oracle_mod, dev, case):
    """Nucleus rows whose boundary sub-bucket holds hundreds to thousands of
    tokens: of one rounded value (bf16 Zipf rows; the cut ranks them by a
    radix select over their ids), or of many nearly equal values (fp32
    logits on a grid of 1/4 plus a jitter of 1e-6; ranked by a sort)."""
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    B, K = 40, 2
    if case == "bf16_zipf":
        wl0 = workloads.make("mixed_samplers_b1024", batch=B)
        t, d = wl0.target[:, :K + 1], wl0.draft[:, :K]
        dtype = "bf16"
    else:
        V = 30011
        t = np.round(rng.normal(0, 1.0, (B, K + 1, V)) * 4) / 4
        d = np.round((0.8 * t[:, :K] + rng.normal(0, 0.6, (B, K, V))) * 4) / 4
        t = t + rng.uniform(0, 1e-6, t.shape)
        d = d + rng.uniform(0, 1e-6, d.shape)
        dtype = "f32"
    V = t.shape[-1]
    prm = np.zeros(B, PARAMS_DTYPE)
    for b in range(B):
        prm[b] = (float(rng.choice([0.6, 1.0, 1.3])), 0, float(rng.choice([0.8, 0.9, 0.95])), 0)
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        for k in range(K):
            tok[b, k] = int(np.argmax(d[b, k] / prm["temperature"][b] + rng.gumbel(size=V)))
    u = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.custom(t, d, tok, np.full(B, K, np.int32), prm, u, dtype=dtype,
                          name=f"crowded_{case}")
    for mode in ("auto", "positions"):
        rep, _, _ = check(oracle_mod, wl, dev, label=wl.name, step_mode=mode)
        assert rep.compared == B and rep.error_rows == 0


def test_deterministic(dev):
    wl = workloads.make("mixed_samplers_b1024", batch=128, vocab=30011)
    a = run_gpu(wl, dev)
    b = run_gpu(wl, dev)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def _to_padded(x, pad, offset, fill):
    """Copy device tensor x [B, R, V] into the columns offset..offset+V of a
    wider [B, R, V + pad] tensor whose other columns hold `fill`; returns the
    strided view (row stride V + pad, base shifted by `offset` elements)."""
    import torch

    B, R, V = x.shape
    base = torch.full((B, R, V + pad), fill, dtype=x.dtype, device=x.device)
    view = base[:, :, offset:offset + V]
    view.copy_(x)
    return view


@pytest.mark.parametrize("dtype,V,pad,offset", [
    ("f32", 30008, 8, 0),     # aligned rows wider than V: the tail reads stop at V
    ("f32", 30011, 13, 1),    # base and stride off the 16-byte grid
    ("bf16", 50000, 16, 0),
    ("bf16", 20011, 5, 3),
], ids=["f32_aligned", "f32_unaligned", "bf16_aligned", "bf16_unaligned"])
@pytest.mark.parametrize("mode", ["positions", "dense"])
def test_strided_rows(oracle_mod, dev, dtype, V, pad, offset, mode):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    rng = np.random.default_rng(V + pad + offset)
    B = 48
    wl = _random_case(rng, B, 3, V, dtype, 1.0, 20, 0.9)
    prm = wl.params
    prm["top_k"][::3] = 0            # nucleus rows
    prm["top_p"][1::6] = 1.0         # and untruncated full-vocab rows
    prm["temperature"][2::5] = 0.0   # and greedy rows
    t, d, tok, dl, pt, uni = workloads.to_torch(wl, dev)
    # +inf in the padding wins every comparison if a kernel ever reads it
    tp = _to_padded(t, pad, offset, float("inf"))
    dp = _to_padded(d, pad, offset, float("inf"))
    assert tp.stride(1) == V + pad and tp.data_ptr() % 16 == (offset * tp.element_size()) % 16
    _say(f"[gpu] strided rows {dtype} V={V} stride={V + pad} offset={offset}")
    g_tok, g_acc, g_dg = sv.verify(tp, dp, tok, dl, pt, uni, diag=True, step_mode=mode)
    torch.cuda.synchronize()
    rep = compare(g_tok.cpu().numpy(), g_acc.cpu().numpy(), g_dg.cpu().numpy(),
                  run_oracle(oracle_mod, wl), inputs=wl, oracle_mod=oracle_mod)
    _say(f"[gpu] strided rows: {rep.describe()}")
    assert rep.tight_ok, rep.describe()
    assert rep.unsupported == 0 and rep.error_rows == 0
    # the same inputs packed densely give the same bits
    c_tok, c_acc, c_dg = run_gpu(wl, dev, step_mode=mode)
    assert np.array_equal(c_tok, g_tok.cpu().numpy())
    assert np.array_equal(c_acc, g_acc.cpu().numpy())
    assert np.array_equal(c_dg, g_dg.cpu().numpy(), equal_nan=True)


def test_side_stream(dev):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl = workloads.make("mixed_samplers_b1024", batch=96, vocab=20011)
    ref = run_gpu(wl, dev)
    ins = workloads.to_torch(wl, dev)
    s = torch.cuda.Stream(device=dev)  # default priority
    s.wait_stream(torch.cuda.current_stream(dev))
    _say("[gpu] verify on a side stream")
    tok, acc, dg = sv.verify(*ins, diag=True, stream=s)
    s.synchronize()
    got = (tok.cpu().numpy(), acc.cpu().numpy(), dg.cpu().numpy())
    for x, y in zip(ref, got):
        if not np.array_equal(x, y, equal_nan=True):
            same = (x == y) | (np.isnan(x) & np.isnan(y)) if x.dtype.kind == "f" else x == y
            rows = np.unique(np.nonzero(~same.reshape(len(x), -1))[0])
            detail = [(int(b), ref[0][b].tolist(), int(ref[1][b]), got[0][b].tolist(), int(got[1][b]),
                       wl.params[b].tolist(), int(wl.draft_len[b])) for b in rows[:6]]
            raise AssertionError(f"current and side stream differ in rows {rows.tolist()}: "
                                 f"(row, tokens, accept length on the current stream, on the side "
                                 f"stream, params, draft length) {detail}")


def test_side_stream_other_entry_points(dev):
    """The sampler, the tree verify and the acceptance statistics on a side
    stream give what they give on the current one."""
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl, par = workloads.make_tree(batch=24, vocab=4099, K=6, shape="wide", dtype="f32")
    ins = workloads.to_torch(wl, dev)
    t, d, tok, nc, prm, uni = ins
    par_t = torch.from_numpy(np.ascontiguousarray(par)).to(dev)
    runs = [
        lambda **kw: sv.sample(t[:, 0, :], prm, uni[:, 0], diag=True, **kw),
        lambda **kw: sv.verify_tree(t, d, tok, par_t, nc, prm, uni, max_depth=1, max_children=6,
                                    diag=True, **kw),
        lambda **kw: (sv.accept_stats(t[:, 0, :], d[:, 0, :], prm, **kw),),
    ]
    for run in runs:
        ref = [x.cpu().numpy() for x in run() if x is not None]
        s = torch.cuda.Stream(device=dev)  # default priority
        s.wait_stream(torch.cuda.current_stream(dev))
        out = run(stream=s)
        s.synchronize()
        got = [x.cpu().numpy() for x in out if x is not None]
        for x, y in zip(ref, got):
            assert np.array_equal(x, y, equal_nan=True)


@pytest.mark.parametrize("mode", ["positions", "dense"])
def test_top_k_above_limit_unsupported(oracle_mod, dev, mode):
    import rejection_sampling_verify_sv_amd as sv

    rng = np.random.default_rng(11)
    V = 3000
    wl = _random_case(rng, 24, 2, V, "f32", 1.0, 20, 0.9)
    bad = [1, 4, 9, 17]
    wl.params["top_k"][bad] = [sv.SV_MAX_TOP_K + 1, 100, V - 1, 2 * sv.SV_MAX_TOP_K]
    wl.params["top_k"][[2, 3]] = [sv.SV_MAX_TOP_K, V]   # served: the limit itself, and top_k = V
    rep, g_tok, g_acc = check(oracle_mod, wl, dev, label="top_k_above_limit", step_mode=mode)
    assert g_acc[bad].tolist() == [-2] * len(bad)
    assert (g_tok[bad] == -1).all()
    assert rep.unsupported == len(bad)
    assert rep.compared == wl.B - len(bad)


@pytest.mark.parametrize("mode", ["positions", "dense"])
@pytest.mark.parametrize("dtype,K,top_k,top_p", [
    ("bf16", 8, 20, 0.9),
    ("f32", 7, 0, 0.8),
    ("bf16", 8, 0, 1.0),
], ids=["topk_K8", "nucleus_K7", "untruncated_K8"])
def test_long_drafts(oracle_mod, dev, dtype, K, top_k, top_p, mode):
    rng = np.random.default_rng(K * 100 + top_k)
    B, V = 40, 20011
    L = rng.integers(K - 2, K + 1, B).astype(np.int32)
    wl = _random_case(rng, B, K, V, dtype, 1.0, top_k, top_p, draft_len=L)
    # drafts close to the target so that acceptance runs deep into the draft
    wl_close = _random_case(rng, B, K, V, dtype, 1.0, top_k, top_p, draft_len=L, noise=0.1)
    for case, lab in ((wl, "random"), (wl_close, "close")):
        rep, _, g_acc = check(oracle_mod, case, dev, label=f"long_drafts_{lab}_{dtype}_K{K}",
                              step_mode=mode)
        assert rep.unsupported == 0


EXTREME_T = [
    # label, V, dtype, T, top_k, top_p, scale
    ("topk_T50", 20000, "f32", 50.0, 50, 0.95, 2.0),
    ("topk_T1e-3", 20000, "bf16", 1e-3, 20, 0.9, 2.0),
    ("greedy_equiv_top_k_1_T4", 20000, "f32", 4.0, 1, 1.0, 2.0),
    ("untruncated_T8", 30011, "f32", 8.0, 0, 1.0, 2.0),
    ("untruncated_T1e-3", 30011, "bf16", 1e-3, 0, 1.0, 2.0),
    ("nucleus_T4", 30011, "f32", 4.0, 0, 0.9, 2.0),
    ("nucleus_T1e-3", 30011, "bf16", 1e-3, 0, 0.9, 2.0),
    ("nucleus_T1e-2_f32", 30011, "f32", 1e-2, 0, 0.95, 2.0),
]


@pytest.mark.parametrize("mode", ["positions", "dense"])
@pytest.mark.parametrize("label,V,dtype,T,top_k,top_p,scale", EXTREME_T,
                         ids=[e[0] for e in EXTREME_T])
def test_extreme_temperature(oracle_mod, dev, label, V, dtype, T, top_k, top_p, scale, mode):
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    wl = _random_case(rng, 32, 2, V, dtype, T, top_k, top_p, scale=scale)
    rep, _, _ = check(oracle_mod, wl, dev, label=label, step_mode=mode)
    assert rep.unsupported == 0 and rep.error_rows == 0


@pytest.mark.parametrize("mode", ["positions", "dense"])
def test_nucleus_anchor_cases(oracle_mod, dev, mode):
    """Nucleus rows measured against the anchor window: rows whose max lies
    far above the largest of the first 64 vectors (second histogram pass),
    rows whose first vectors are all -inf, and ordinary rows, in one batch."""
    rng = np.random.default_rng(zlib.crc32(b"nucleus_anchor"))
    B, K, V = 36, 2, 30011
    wl = _random_case(rng, B, K, V, "f32", 0.5, 0, 0.9)
    T = 0.5
    for b in range(0, B, 3):       # a spike 40 T above everything else, late in the row
        for k in range(K + 1):
            row = wl.target[b, k]
            row[V - 7 - b] = row.max() + 40 * T
        for k in range(K):
            row = wl.draft[b, k]
            row[V - 11 - b] = row.max() + 40 * T
    for b in range(1, B, 3):       # the anchor's vectors hold no finite logit
        wl.target[b, :, :512] = -np.inf
        wl.draft[b, :, :512] = -np.inf
    rep, _, g_acc = check(oracle_mod, wl, dev, label="nucleus_anchor_cases", step_mode=mode)
    assert rep.unsupported == 0 and rep.error_rows == 0 and rep.compared == B


@pytest.mark.parametrize("mode", ["positions", "dense"])
@pytest.mark.parametrize("B", [8, 80], ids=["split_units", "one_workgroup_per_unit"])
def test_nucleus_boundary_in_one_wave(oracle_mod, dev, B, mode):
    """A boundary bucket of 2000 equal logits, all at offsets that one wave
    of a 4096-element tile reads: with one workgroup per unit (80 rows, 160
    nucleus units) that wave's share of the collect buffer overflows and the
    cut takes the wide path; with few rows the unit is split into slices and
    each slice's keys fit."""
    rng = np.random.default_rng(zlib.crc32(b"boundary_one_wave") + B)
    K, V = 2, 20480
    pos = np.flatnonzero(np.arange(V) % 1024 < 256)

    def row():
        r = rng.normal(-5.0, 0.3, V)
        r[rng.choice(pos, size=2000, replace=False)] = 0.0
        return r

    t = np.stack([np.stack([row() for _ in range(K + 1)]) for _ in range(B)])
    d = np.stack([np.stack([row() for _ in range(K)]) for _ in range(B)])
    prm = np.zeros(B, PARAMS_DTYPE)
    prm["temperature"], prm["top_k"], prm["top_p"] = 1.0, 0, 0.5
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        for k in range(K):
            tok[b, k] = int(np.argmax(d[b, k] + rng.gumbel(size=V)))
    u = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.custom(t, d, tok, np.full(B, K, np.int32), prm, u, dtype="f32")
    rep, _, _ = check(oracle_mod, wl, dev, label=f"nucleus_boundary_in_one_wave_B{B}",
                      step_mode=mode)
    assert rep.unsupported == 0 and rep.error_rows == 0 and rep.compared == B
