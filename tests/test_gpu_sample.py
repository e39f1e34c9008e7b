"""GPU parity of the single draw per row (sv_sample, and sv_verify with K = 0)
against the fp64 oracle, and of a full draft-then-verify chain.

Bar as in tests/parity.py: identical tokens except rows whose drawn token was
decided by a uniform within 1e-5 of a CDF bin edge (counted), probabilities in
the diagnostics within 1e-5.
"""
import sys
import zlib

import numpy as np
import pytest

from rejection_sampling_verify_sv_amd import workloads
from tests.parity import compare, draws, subset

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


def _rows_torch(rows, dtype, dev):
    import torch

    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(rows)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(torch.bfloat16)


def _gpu_sample(rows, params, u, dtype, dev):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    tok, st, dg = sv.sample(_rows_torch(rows, dtype, dev), sv.params_tensor(params, dev),
                            torch.from_numpy(u).to(dev), diag=True)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), st.cpu().numpy(), dg.cpu().numpy()


def _oracle_draw(oracle_mod, rows, params, u, dtype):
    B, V = rows.shape
    return oracle_mod.verify(rows.reshape(B, 1, V), None, np.zeros((B, 0), np.int32), None,
                             params, u.reshape(B, 1), dtype=dtype)


SAMPLE_CASES = [
    # recipe, vocab, position
    ("mixed_samplers_b1024", None, 0),
    ("mixed_samplers_b1024", 20011, 2),
    ("fullvocab_ragged_b256", None, 1),
    ("mixed_greedy_b64", None, 0),
    ("decode_b1", None, 0),
]


@pytest.mark.parametrize("name,vocab,k", SAMPLE_CASES,
                         ids=[f"{c[0]}_V{c[1] or 'full'}_k{c[2]}" for c in SAMPLE_CASES])
def test_sample_parity(oracle_mod, dev, name, vocab, k):
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl = workloads.make(name, batch=min(256, workloads.RECIPES[name]["B"]), vocab=vocab)
    rows = np.ascontiguousarray(wl.target[:, k, :])
    u = np.ascontiguousarray(wl.uniforms[:, -1])
    _say(f"[gpu] sample {name} B={wl.B} V={wl.V} {wl.dtype} position {k}")
    g_tok, g_st, g_dg = _gpu_sample(rows, wl.params, u, wl.dtype, dev)
    ref = _oracle_draw(oracle_mod, rows, wl.params, u, wl.dtype)
    rep = compare(g_tok[:, None], g_st, g_dg, ref, inputs=draws(rows, wl.params, u, wl.dtype),
                  oracle_mod=oracle_mod)
    _say(f"[gpu] sample {name}: {rep.describe()}")
    assert rep.mismatch_in_band_by_class.get("top_k", 0) == 0, rep.describe()
    assert rep.tight_ok, rep.describe()
    assert rep.unsupported == 0 and rep.compared == wl.B
    # sv_verify with K = 0 is the same launch sequence: identical bits
    tok0, acc0, dg0 = sv.verify(_rows_torch(rows, wl.dtype, dev)[:, None, :], None, None, None,
                                wl.params, torch.from_numpy(u[:, None]).to(dev), diag=True)
    torch.cuda.synchronize()
    assert np.array_equal(tok0.cpu().numpy()[:, 0], g_tok)
    assert np.array_equal(acc0.cpu().numpy(), g_st)
    assert np.array_equal(dg0.cpu().numpy(), g_dg, equal_nan=True)


@pytest.mark.parametrize("seed", range(12))
def test_sample_sweep(oracle_mod, dev, seed):
    """Seeded batches of up to 700 rows (beyond 512 the draw runs position by
    position), each row with its own sampler class and temperature, both
    dtypes, every row against the oracle.  Seeds from 8 on take rows short
    enough for one wave's loads (one unit per wave in the row pass)."""
    rng = np.random.default_rng(6100 + seed)
    B = int(rng.choice([3, 300, 700]))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    if seed < 8:
        V = int(rng.choice([2048, 20011, 65543]))
    else:
        V = int(rng.choice([3, 100, 1000, 1024] if dtype == "f32" else [100, 2000, 2048]))
    rows = rng.normal(0, float(rng.choice([1.0, 3.0])), (B, V)).astype(np.float32)
    prm = np.zeros(B, workloads.PARAMS_DTYPE)
    prm["temperature"] = rng.choice([0.0, 0.5, 1.0, 1.5], B)
    prm["top_k"] = rng.choice([0, 1, 20, 64, 100, V], B)
    prm["top_p"] = rng.choice([0.5, 0.9, 1.0], B)
    u = rng.random(B, dtype=np.float32)
    stored = rows if dtype == "f32" else workloads.f32_to_bf16_bits(rows)
    g_tok, g_st, g_dg = _gpu_sample(stored, prm, u, dtype, dev)
    ref = _oracle_draw(oracle_mod, stored, prm, u, dtype)
    rep = compare(g_tok[:, None], g_st, g_dg, ref, inputs=draws(stored, prm, u, dtype),
                  oracle_mod=oracle_mod)
    _say(f"[gpu] sample sweep {seed} B={B} V={V} {dtype}: {rep.describe()}")
    assert rep.mismatch_in_band_by_class.get("top_k", 0) == 0, rep.describe()
    assert rep.tight_ok, rep.describe()
    assert rep.compared + rep.unsupported == B


def test_sample_edge_rows(oracle_mod, dev):
    rng = np.random.default_rng(zlib.crc32(b"sample_edges"))
    B, V = 12, 5003
    rows = rng.normal(0, 2, (B, V)).astype(np.float32)
    prm = np.zeros(B, workloads.PARAMS_DTYPE)
    prm["temperature"], prm["top_k"], prm["top_p"] = 1.0, 20, 0.9
    prm["temperature"][1] = 0.0                      # greedy
    rows[2, :] = 0.0                                 # all equal, untruncated
    prm["top_k"][2] = 0
    prm["top_p"][2] = 1.0
    prm["top_k"][3] = 100                            # above the in-register limit
    prm["temperature"][4] = -1.0                     # invalid
    rows[5, :] = -np.inf                             # no finite logit
    rows[6, 1:] = -np.inf                            # one finite logit
    prm["top_k"][7], prm["top_p"][7] = 0, 0.3        # nucleus
    prm["top_k"][8] = 1                              # top_k = 1 is the argmax
    u = rng.random(B, dtype=np.float32)
    u[9] = 0.0
    u[10] = np.float32(1.0) - np.float32(2.0 ** -24)
    g_tok, g_st, g_dg = _gpu_sample(rows, prm, u, "f32", dev)
    ref = _oracle_draw(oracle_mod, rows, prm, u, "f32")
    rep = compare(g_tok[:, None], g_st, g_dg, ref, inputs=draws(rows, prm, u, "f32"),
                  oracle_mod=oracle_mod)
    _say(f"[gpu] sample edges: {rep.describe()}")
    assert rep.tight_ok, rep.describe()
    assert g_st.tolist()[3:6] == [-2, -1, -1]
    assert g_tok[3] == -1 and g_tok[4] == -1 and g_tok[5] == -1
    assert g_tok[1] == int(np.argmax(rows[1])) and g_tok[6] == 0
    assert g_tok[8] == int(np.argmax(rows[8]))


@pytest.mark.parametrize("name,vocab", [("mixed_samplers_b1024", 30011),
                                        ("fullvocab_ragged_b256", 20011)])
def test_draft_then_verify_chain(oracle_mod, dev, name, vocab):
    """Draft tokens drawn on the GPU with the same truncation as the target,
    then verified on the GPU; the oracle runs the same chain on its own."""
    import torch

    import rejection_sampling_verify_sv_amd as sv

    wl = workloads.make(name, batch=128, vocab=vocab)
    B, K, V = wl.B, wl.K, wl.V
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    v = rng.random((B, K), dtype=np.float32)     # uniforms of the draft draws
    g_x = np.zeros((B, K), np.int32)
    o_x = np.zeros((B, K), np.int32)
    same = np.ones(B, bool)
    for k in range(K):
        rows = np.ascontiguousarray(wl.draft[:, k, :])
        gt, gs, _ = _gpu_sample(rows, wl.params, np.ascontiguousarray(v[:, k]), wl.dtype, dev)
        vk = np.ascontiguousarray(v[:, k])
        ref_k = _oracle_draw(oracle_mod, rows, wl.params, vk, wl.dtype)
        ot, oa = ref_k[0], ref_k[1]
        assert (gs == 0).all() and (oa == 0).all()
        g_x[:, k], o_x[:, k] = gt, ot[:, 0]
        diff = gt != ot[:, 0]
        # a differing draw must be the rule's draw for a uniform within the band
        rep_k = compare(gt[:, None], gs, None, ref_k, inputs=draws(rows, wl.params, vk, wl.dtype),
                        oracle_mod=oracle_mod)
        assert rep_k.ok, rep_k.describe()
        same &= ~diff
    _say(f"[gpu] chain {name}: {int(same.sum())}/{B} rows drew identical drafts")
    L = np.where(wl.draft_len >= 0, wl.draft_len, K).astype(np.int32)
    g_x_used = np.where(np.arange(K)[None, :] < L[:, None], g_x, 0).astype(np.int32)
    o_x_used = np.where(np.arange(K)[None, :] < L[:, None], o_x, 0).astype(np.int32)
    t, d, _, dl, prm, uni = workloads.to_torch(wl, dev)
    tok, acc, dg = sv.verify(t, d, torch.from_numpy(g_x_used).to(dev), dl, prm, uni, diag=True)
    torch.cuda.synchronize()
    ref = oracle_mod.verify(wl.target, wl.draft, o_x_used, wl.draft_len, wl.params, wl.uniforms,
                            dtype=wl.dtype)
    rows = np.nonzero(same)[0]
    ref_same = tuple(r[rows] if isinstance(r, np.ndarray) else r for r in ref)
    wl_o = subset(wl, rows)
    wl_o.tokens = o_x_used[rows]
    rep = compare(tok.cpu().numpy(), acc.cpu().numpy(), dg.cpu().numpy(), ref_same, rows,
                  inputs=wl_o, oracle_mod=oracle_mod)
    _say(f"[gpu] chain {name} verify: {rep.describe()}")
    assert rep.tight_ok, rep.describe()
    assert rep.compared == len(rows) and len(rows) >= B - 2
