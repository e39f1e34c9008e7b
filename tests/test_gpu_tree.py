"""GPU parity of the tree / multi-candidate verify (sv_verify_tree) against the
fp64 oracle (oracle.verify_tree), through the C ABI, under the band rule of
tests/parity.py (compare_tree): identical paths, tokens and lengths except
outcomes a uniform within 1e-5 of the given one would give; probabilities
within 1e-5.  A tree that is a path must give exactly what sv_verify gives.
"""
import sys
import zlib

import numpy as np
import pytest

from rejection_sampling_verify_sv_amd import workloads
from rejection_sampling_verify_sv_amd.workloads import PARAMS_DTYPE
from tests.parity import compare_tree, tree_inputs

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


def _parents(rng, K, shape):
    if shape == "path":
        return np.arange(K, dtype=np.int32)
    if shape == "wide":  # every candidate at the root
        return np.zeros(K, np.int32)
    if shape == "medusa":  # 3 at the root, 2 under each, then 1 under those
        par = []
        for c in range(1, K + 1):
            if c <= 3:
                par.append(0)
            elif c <= 9:
                par.append((c - 4) // 2 + 1)
            else:
                par.append(c - 6)
        return np.array(par, np.int32)
    return np.array([rng.integers(0, c) for c in range(1, K + 1)], np.int32)


def tree_case(rng, B, K, V, dtype, T, top_k, top_p, shape="random", noise=0.5, n_cand=None):
    t = rng.normal(0, 2.0, (B, K + 1, V))
    d = t[:, :K] * 0.9 + rng.normal(0, 2.0 * noise, (B, K, V))
    par = np.stack([_parents(rng, K, shape) for _ in range(B)])
    tok = np.zeros((B, K), np.int32)
    Te = max(T, 1e-3)
    for b in range(B):
        for c in range(1, K + 1):
            row = d[b, par[b, c - 1]]
            tok[b, c - 1] = int(np.argmax(row / Te + rng.gumbel(size=V)))
    prm = np.zeros(B, PARAMS_DTYPE)
    prm["temperature"], prm["top_k"], prm["top_p"] = T, top_k, top_p
    nc = np.full(B, K, np.int32) if n_cand is None else n_cand
    u = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.custom(t, d, tok, nc, prm, u, dtype=dtype)
    return wl, par


def run_tree(wl, par, dev, max_depth, max_children):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    t, d, tok, nc, prm, uni = workloads.to_torch(wl, dev)
    out = sv.verify_tree(t, d, tok, torch.from_numpy(np.ascontiguousarray(par)).to(dev), nc, prm,
                         uni, max_depth=max_depth, max_children=max_children, diag=True)
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in out)


def check_tree(oracle_mod, wl, par, dev, label, max_depth=None, max_children=None):
    K = wl.K
    if max_depth is None:
        depth = np.zeros((wl.B, K + 1), np.int32)
        for c in range(1, K + 1):
            depth[:, c] = depth[np.arange(wl.B), par[:, c - 1]] + 1
        max_depth = int(depth.max())
    if max_children is None:
        max_children = max(1, int(max(np.bincount(p, minlength=K + 1).max() for p in par)))
    _say(f"[gpu] tree {label}: B={wl.B} K={K} V={wl.V} {wl.dtype} depth<={max_depth} "
         f"children<={max_children}")
    g_tok, g_len, g_path, g_dg = run_tree(wl, par, dev, max_depth, max_children)
    ref = oracle_mod.verify_tree(wl.target, wl.draft, wl.tokens, par, wl.draft_len, wl.params,
                                 wl.uniforms, dtype=wl.dtype)
    inp = tree_inputs(wl.target, wl.draft, wl.tokens, par, wl.draft_len, wl.params, wl.uniforms,
                      wl.dtype)
    rep = compare_tree(g_tok, g_len, g_path, g_dg, ref, inputs=inp, oracle_mod=oracle_mod)
    _say(f"[gpu] tree {label}: {rep.describe()} mean_path_len="
         f"{float(np.mean(g_len[g_len >= 0])) if (g_len >= 0).any() else 0:.2f}")
    assert rep.tight_ok, rep.describe()
    assert rep.mismatch_in_band_by_class.get("top_k", 0) == 0, rep.describe()
    return rep, g_len


@pytest.mark.parametrize("name", ["mixed_samplers_b1024", "fullvocab_ragged_b256",
                                  "mixed_greedy_b64"])
def test_path_tree_is_the_chain(oracle_mod, dev, name):
    """Every recipe (smaller vocabulary), as a path tree: bitwise the same
    outputs as sv_verify on the same inputs, and the path is 1..accept_len."""
    import rejection_sampling_verify_sv_amd as sv

    wl = workloads.make(name, batch=96, vocab=20011)
    B, K = wl.B, wl.K
    par = np.broadcast_to(np.arange(K, dtype=np.int32), (B, K)).copy()
    g_tok, g_len, g_path, g_dg = run_tree(wl, par, dev, K, 1)
    import torch

    c_tok, c_acc, c_dg = sv.verify(*workloads.to_torch(wl, dev), diag=True)
    torch.cuda.synchronize()
    assert np.array_equal(g_len, c_acc.cpu().numpy())
    assert np.array_equal(g_tok, c_tok.cpu().numpy())
    assert np.array_equal(g_dg, c_dg.cpu().numpy(), equal_nan=True)
    for b in range(B):
        if g_len[b] >= 0:
            assert g_path[b, :g_len[b]].tolist() == list(range(1, g_len[b] + 1))
            assert (g_path[b, g_len[b]:] == -1).all()
    _say(f"[gpu] path tree {name}: identical to sv_verify on {B} rows")


TREES = [
    # label, B, K, V, dtype, T, top_k, top_p, shape, noise
    ("topk_random", 64, 8, 20011, "f32", 1.0, 20, 0.95, "random", 0.5),
    ("topk_wide_bf16", 64, 6, 30011, "bf16", 0.8, 50, 1.0, "wide", 0.4),
    ("topk_medusa", 64, 12, 20011, "f32", 0.7, 20, 0.9, "medusa", 0.3),
    ("greedy_random", 64, 10, 20011, "bf16", 0.0, 20, 0.95, "random", 0.2),
    ("greedy_wide", 48, 6, 20011, "f32", 0.0, 0, 1.0, "wide", 0.2),
    ("untruncated_random_f32", 48, 8, 30011, "f32", 1.0, 0, 1.0, "random", 0.4),
    ("untruncated_wide_bf16", 48, 5, 20011, "bf16", 1.0, 0, 1.0, "wide", 0.5),
    ("untruncated_medusa", 32, 12, 20011, "f32", 0.9, 0, 1.0, "medusa", 0.3),
    ("nucleus_random", 48, 8, 30011, "f32", 1.0, 0, 0.9, "random", 0.4),
    ("nucleus_wide_bf16", 48, 5, 20011, "bf16", 0.8, 0, 0.8, "wide", 0.5),
    ("topk_1_is_greedy", 32, 6, 20011, "f32", 1.3, 1, 1.0, "random", 0.3),
]


@pytest.mark.parametrize("label,B,K,V,dtype,T,top_k,top_p,shape,noise", TREES,
                         ids=[t[0] for t in TREES])
def test_tree_parity(oracle_mod, dev, label, B, K, V, dtype, T, top_k, top_p, shape, noise):
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    wl, par = tree_case(rng, B, K, V, dtype, T, top_k, top_p, shape, noise)
    rep, g_len = check_tree(oracle_mod, wl, par, dev, label)
    assert rep.compared == B and rep.error_rows == 0 and rep.unsupported == 0


def test_tree_mixed_classes_ragged(oracle_mod, dev):
    """Every sampler class in one batch, ragged candidate counts (0..K), and
    nodes with many children (child rounds on full-vocab rows)."""
    rng = np.random.default_rng(zlib.crc32(b"tree_mixed"))
    B, K, V = 96, 9, 30011
    nc = rng.integers(0, K + 1, B).astype(np.int32)
    wl, par = tree_case(rng, B, K, V, "f32", 1.0, 20, 0.95, "random", 0.3, n_cand=nc)
    P = wl.params
    P["temperature"] = rng.choice([0.0, 0.6, 1.0, 1.5], B)
    P["top_k"] = rng.choice([0, 5, 20, 64], B)
    P["top_p"] = rng.choice([0.8, 0.95, 1.0], B)
    par[::4] = 0  # a quarter of the rows put every candidate at the root
    rep, g_len = check_tree(oracle_mod, wl, par, dev, "mixed_classes_ragged")
    assert rep.compared == B and rep.error_rows == 0


@pytest.mark.parametrize("seed", range(14))
def test_tree_sweep(oracle_mod, dev, seed):
    """Seeded trees: shape (random, wide, medusa, path), size, candidate
    counts, dtype, and each row's sampler class and temperature drawn at
    random; every row against the oracle.  Seeds from 10 on take rows short
    enough for one wave's loads (one unit per wave in the row pass)."""
    rng = np.random.default_rng(7300 + seed)
    B = int(rng.choice([7, 64, 200]))
    shape = str(rng.choice(["random", "wide", "medusa", "path"]))
    K = int(rng.integers(2, 13)) if shape != "medusa" else 12
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    if seed < 10:
        V = int(rng.choice([4099, 20011]))
    else:
        V = int(rng.choice([97, 1000, 1024] if dtype == "f32" else [500, 2048]))
    nc = rng.integers(0, K + 1, B).astype(np.int32)
    wl, par = tree_case(rng, B, K, V, dtype, 1.0, 20, 0.95, shape, float(rng.uniform(0.2, 0.7)),
                        n_cand=nc)
    P = wl.params
    P["temperature"] = rng.choice([0.0, 0.5, 1.0, 1.4], B)
    P["top_k"] = rng.choice([0, 1, 20, 64, V], B)
    P["top_p"] = rng.choice([0.7, 0.95, 1.0], B)
    rep, g_len = check_tree(oracle_mod, wl, par, dev, f"sweep_{seed}_{shape}")
    assert rep.compared == B and rep.error_rows == 0


def test_tree_full_vocab_many_rejections(oracle_mod, dev):
    """Candidates the target dislikes (drawn from the draft's tail), so that
    full-vocab rows reject child after child and the residual of residuals is
    both tested and drawn from."""
    rng = np.random.default_rng(zlib.crc32(b"tree_reject"))
    B, K, V = 40, 6, 20011
    wl, par = tree_case(rng, B, K, V, "f32", 1.0, 0, 1.0, "wide", 1.0)
    wl.params["top_p"][::2] = 0.9  # half nucleus, half untruncated
    t32 = workloads.as_f32(wl.target, "f32")
    for b in range(B):  # tokens among the target's 200 lowest at the root
        low = np.argsort(t32[b, 0])[:200]
        wl.tokens[b] = rng.choice(low, K)
    rep, g_len = check_tree(oracle_mod, wl, par, dev, "full_vocab_many_rejections")
    # many rows reject every candidate at the root (all child rounds run)
    assert rep.compared == B and (g_len == 0).sum() >= B // 4


def test_tree_invalid_rows(oracle_mod, dev):
    rng = np.random.default_rng(3)
    B, K, V = 10, 6, 3000
    wl, par = tree_case(rng, B, K, V, "f32", 1.0, 20, 0.9, "random", 0.5)
    par[1, 2] = 3         # node 3's parent is itself
    par[2, 0] = -1        # negative parent
    wl.tokens[3, 4] = V   # token out of range
    wl.draft_len[4] = K + 1
    par[5] = np.arange(K)  # a path of depth 6 > max_depth = 4 below
    par[6] = 0             # 6 children at the root > max_children = 5 below
    wl.params["temperature"][7] = -1.0
    g_tok, g_len, g_path, _ = run_tree(wl, par, dev, 4, 5)
    assert g_len[1:8].tolist() == [-1] * 7
    assert (g_tok[1:8] == -1).all() and (g_path[1:8] == -1).all()
    # the others are served and agree with the oracle
    ok = np.array([0, 8, 9])
    ref = oracle_mod.verify_tree(wl.target[ok], wl.draft[ok], wl.tokens[ok], par[ok],
                                 wl.draft_len[ok], wl.params[ok], wl.uniforms[ok])
    inp = tree_inputs(wl.target[ok], wl.draft[ok], wl.tokens[ok], par[ok], wl.draft_len[ok],
                      wl.params[ok], wl.uniforms[ok], "f32")
    rep = compare_tree(g_tok[ok], g_len[ok], g_path[ok], None, ref, inputs=inp,
                       oracle_mod=oracle_mod)
    assert rep.tight_ok, rep.describe()


def test_tree_full_vocabulary_size(oracle_mod, dev):
    """Medusa-shaped trees at V = 151936 (fp32, every sampler class), every row
    compared."""
    rng = np.random.default_rng(zlib.crc32(b"tree_large"))
    B, K, V = 64, 12, 151936
    wl, par = tree_case(rng, B, K, V, "f32", 1.0, 20, 0.95, "medusa", 0.3)
    P = wl.params
    P["temperature"] = rng.choice([0.0, 0.6, 1.0], B)
    P["top_k"] = rng.choice([0, 20, 50], B)
    P["top_p"] = rng.choice([0.8, 0.95, 1.0], B)
    rep, g_len = check_tree(oracle_mod, wl, par, dev, "medusa_V151936")
    assert rep.compared == B and rep.error_rows == 0
