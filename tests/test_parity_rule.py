"""The comparison rule of tests/parity.py, checked on the CPU with outcomes
planted into copies of the oracle's own outputs (no GPU involved):
identical outputs pass; a changed token far from any threshold fails; an
outcome that a uniform within the band would give passes and is counted per
class; a greedy row may never differ; wrong diagnostics fail."""
import numpy as np
import pytest

from rejection_sampling_verify_sv_amd import workloads
from rejection_sampling_verify_sv_amd.workloads import PARAMS_DTYPE
from tests.parity import BAND, compare


def _case(oracle_mod, seed=0, B=48, K=2, V=300):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 2.0, (B, K + 1, V))
    d = 0.8 * t[:, :K] + rng.normal(0, 0.8, (B, K, V))
    prm = np.zeros(B, PARAMS_DTYPE)
    prm["temperature"] = 1.0
    prm["top_k"] = np.where(np.arange(B) % 3 == 0, 20, 0)
    prm["top_p"] = np.where(np.arange(B) % 3 == 1, 0.9, 1.0)
    prm["temperature"][np.arange(B) % 8 == 7] = 0.0
    tok = rng.integers(0, 30, (B, K)).astype(np.int32)
    # drafts the target likes, so that some rows accept
    for b in range(B):
        for k in range(K):
            tok[b, k] = int(np.argsort(-d[b, k])[rng.integers(0, 3)])
    u = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.custom(t, d, tok, np.full(B, K, np.int32), prm, u)
    ref = oracle_mod.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params,
                            wl.uniforms)
    return wl, ref


def test_identical_outputs_pass(oracle_mod):
    wl, ref = _case(oracle_mod)
    rep = compare(ref[0].copy(), ref[1].copy(), ref[2].copy(), ref, inputs=wl,
                  oracle_mod=oracle_mod)
    assert rep.ok and rep.exact == rep.compared == wl.B and rep.mismatch_in_band == 0


def test_changed_token_out_of_band_fails(oracle_mod):
    wl, ref = _case(oracle_mod, seed=1)
    tok, acc, dg = ref[0].copy(), ref[1].copy(), ref[2].copy()
    K = wl.K
    b = next(b for b in range(wl.B)
             if wl.params["temperature"][b] > 0 and np.nanmin(ref[2][b, :, 3]) > 1e-3)
    a = acc[b]
    ex = oracle_mod.explain(wl.target[b:b + 1], wl.draft[b:b + 1], wl.tokens[b:b + 1],
                            wl.draft_len[b:b + 1], wl.params[b:b + 1], [a], [tok[b, a]])
    # another token of positive weight under the same final distribution
    others = [y for y in range(wl.V) if y != tok[b, a]]
    ex2 = oracle_mod.explain(np.repeat(wl.target[b:b + 1], len(others), 0),
                             np.repeat(wl.draft[b:b + 1], len(others), 0),
                             np.repeat(wl.tokens[b:b + 1], len(others), 0),
                             np.repeat(wl.draft_len[b:b + 1], len(others), 0),
                             np.repeat(wl.params[b:b + 1], len(others), 0),
                             np.full(len(others), a), others)
    y = others[int(np.argmax(ex2["py"]))]
    assert ex["py"][0] > 0
    tok[b, a] = y
    rep = compare(tok, acc, dg, ref, inputs=wl, oracle_mod=oracle_mod)
    assert not rep.ok and rep.mismatch_out_of_band == [b]
    assert K >= 1


def test_outcome_within_band_passes(oracle_mod):
    wl, ref = _case(oracle_mod, seed=2)
    K = wl.K
    # a sampling row; move its final uniform to 0.5 BAND past the upper edge
    # of its drawn token's bin, where the oracle draws the next token
    b = next(b for b in range(wl.B) if wl.params["temperature"][b] > 0
             and ref[2][b, K, 2] < 0.99)
    hi = ref[2][b, K, 2]
    wl.uniforms[b, K] = np.float32(hi + 0.5 * BAND)
    ref2 = oracle_mod.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params,
                             wl.uniforms)
    assert ref2[0][b, ref2[1][b]] != ref[0][b, ref[1][b]]
    # "GPU" = the outcome before the move, diagnostics included
    tok, acc, dg = ref2[0].copy(), ref2[1].copy(), ref2[2].copy()
    tok[b], acc[b], dg[b] = ref[0][b], ref[1][b], ref[2][b]
    rep = compare(tok, acc, dg, ref2, inputs=wl, oracle_mod=oracle_mod)
    assert rep.ok, rep.describe()
    assert rep.mismatch_in_band == 1 and rep.mismatch_in_band_rows == [b]
    # half a band is more than the GPU's arithmetic can move a CDF value
    assert not rep.tight_ok and rep.mismatch_beyond_tight == [b]
    # wrong diagnostics on that row are caught
    dg[b, K, 0] += 1e-3
    rep = compare(tok, acc, dg, ref2, inputs=wl, oracle_mod=oracle_mod)
    assert not rep.ok and rep.diag_bad_rows == [b]
    # the same move by 5 BAND is out of band
    wl.uniforms[b, K] = np.float32(hi + 5 * BAND)
    ref3 = oracle_mod.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params,
                             wl.uniforms)
    tok, acc = ref3[0].copy(), ref3[1].copy()
    tok[b], acc[b] = ref[0][b], ref[1][b]
    rep = compare(tok, acc, None, ref3, inputs=wl, oracle_mod=oracle_mod)
    assert rep.mismatch_out_of_band == [b]


def test_flipped_accept_within_band_passes(oracle_mod):
    wl, ref = _case(oracle_mod, seed=3)
    # a sampling row that rejects its first draft with a < 1: put u just
    # below a (accept) and compare against the outcome of u just above it
    cand = [b for b in range(wl.B) if wl.params["temperature"][b] > 0 and ref[1][b] == 0
            and 0.05 < ref[2][b, 0, 2] < 0.95]
    b = cand[0]
    a0 = ref[2][b, 0, 2]
    wl.uniforms[b, 0] = np.float32(a0 + 0.4 * BAND)  # rejects
    rej = oracle_mod.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params,
                            wl.uniforms)
    wl2 = workloads.custom(workloads.as_f32(wl.target, "f32"), workloads.as_f32(wl.draft, "f32"),
                           wl.tokens, wl.draft_len, wl.params, wl.uniforms.copy())
    wl2.uniforms[b, 0] = np.float32(a0 - 0.4 * BAND)  # accepts
    acc_ = oracle_mod.verify(wl2.target, wl2.draft, wl2.tokens, wl2.draft_len, wl2.params,
                             wl2.uniforms)
    assert acc_[1][b] >= 1 and rej[1][b] == 0
    tok, acc, dg = rej[0].copy(), rej[1].copy(), rej[2].copy()
    tok[b], acc[b], dg[b] = acc_[0][b], acc_[1][b], acc_[2][b]
    rep = compare(tok, acc, dg, rej, inputs=wl, oracle_mod=oracle_mod)
    assert rep.ok and rep.mismatch_in_band_rows == [b], rep.describe()


def test_greedy_row_may_never_differ(oracle_mod):
    wl, ref = _case(oracle_mod, seed=4)
    tok, acc = ref[0].copy(), ref[1].copy()
    b = int(np.flatnonzero(wl.params["temperature"] == 0)[0])
    tok[b, acc[b]] = (tok[b, acc[b]] + 1) % wl.V
    rep = compare(tok, acc, None, ref, inputs=wl, oracle_mod=oracle_mod)
    assert not rep.ok and rep.mismatch_out_of_band == [b]


@pytest.mark.parametrize("field", ["status", "padding", "prefix"])
def test_invalid_or_malformed_outcomes_fail(oracle_mod, field):
    wl, ref = _case(oracle_mod, seed=5)
    tok, acc = ref[0].copy(), ref[1].copy()
    b = next(b for b in range(wl.B) if wl.params["temperature"][b] > 0 and acc[b] == 0)
    if field == "status":
        acc[b] = -1
        tok[b] = -1
    elif field == "padding":
        tok[b, -1] = 5
    else:
        acc[b] = 1
        tok[b, 0] = (wl.tokens[b, 0] + 1) % wl.V
    rep = compare(tok, acc, None, ref, inputs=wl, oracle_mod=oracle_mod)
    assert not rep.ok and b in rep.mismatch_out_of_band


def _tree_case(oracle_mod, seed=0, B=40, K=5, V=200):
    from tests.parity import tree_inputs

    rng = np.random.default_rng(seed)
    t = rng.normal(0, 2.0, (B, K + 1, V))
    d = 0.8 * t[:, :K] + rng.normal(0, 0.8, (B, K, V))
    prm = np.zeros(B, PARAMS_DTYPE)
    prm["temperature"] = np.where(np.arange(B) % 5 == 4, 0.0, 1.0)
    prm["top_k"] = np.where(np.arange(B) % 3 == 0, 20, 0)
    prm["top_p"] = np.where(np.arange(B) % 3 == 1, 0.9, 1.0)
    par = np.zeros((B, K), np.int32)
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        for c in range(1, K + 1):
            par[b, c - 1] = rng.integers(0, c)
            tok[b, c - 1] = int(np.argsort(-d[b, par[b, c - 1]])[rng.integers(0, 3)])
    u = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.custom(t, d, tok, np.full(B, K, np.int32), prm, u)
    inp = tree_inputs(wl.target, wl.draft, wl.tokens, par, wl.draft_len, wl.params,
                      wl.uniforms, "f32")
    ref = oracle_mod.verify_tree(wl.target, wl.draft, wl.tokens, par, wl.draft_len, wl.params,
                                 wl.uniforms)
    return inp, ref


def test_tree_rule(oracle_mod):
    from tests.parity import compare_tree

    inp, ref = _tree_case(oracle_mod)
    tok, ln, path, dg = (x.copy() for x in ref[:4])
    rep = compare_tree(tok, ln, path, dg, ref, inputs=inp, oracle_mod=oracle_mod)
    assert rep.ok and rep.exact == rep.compared
    K = tok.shape[1] - 1
    # a sampling row: move its final uniform just past the top of its drawn
    # token's bin; the outcome before the move is then explained in band,
    # 5 bands away it is not
    b = next(b for b in range(len(ln)) if inp.params["temperature"][b] > 0
             and ref[3][b, K, 2] < 0.99)
    hi = ref[3][b, K, 2]
    for move, explained in ((0.5 * BAND, True), (5 * BAND, False)):
        inp.uniforms[b, K] = np.float32(hi + move)
        ref2 = oracle_mod.verify_tree(inp.target, inp.draft, inp.tokens, inp.parents, inp.n_cand,
                                      inp.params, inp.uniforms)
        assert ref2[0][b, ref2[1][b]] != ref[0][b, ref[1][b]]
        g = [x.copy() for x in ref2[:4]]
        for x, y in zip(g, ref[:4]):
            x[b] = y[b]
        rep = compare_tree(*g, ref2, inputs=inp, oracle_mod=oracle_mod)
        if explained:
            assert rep.ok and rep.mismatch_in_band_rows == [b], rep.describe()
        else:
            assert rep.mismatch_out_of_band == [b]
    # a path that is not made of children, or a greedy row that differs, fails
    g = [x.copy() for x in ref[:4]]
    gb = int(np.flatnonzero(inp.params["temperature"] == 0)[0])
    g[0][gb, g[1][gb]] = (g[0][gb, g[1][gb]] + 1) % inp.target.shape[-1]
    rep = compare_tree(*g, ref, inputs=inp, oracle_mod=oracle_mod)
    assert gb in rep.mismatch_out_of_band and not rep.ok


def test_outcome_within_tight_band(oracle_mod):
    from tests.parity import TIGHT_BAND

    wl, ref = _case(oracle_mod, seed=2)
    K = wl.K
    # as above, with the final uniform moved only 0.5 TIGHT_BAND past the
    # drawn token's bin: a difference the GPU's arithmetic can produce
    b = next(b for b in range(wl.B) if wl.params["temperature"][b] > 0
             and ref[2][b, K, 2] < 0.99 and ref[2][b, K, 2] - ref[2][b, K, 1] > 4 * TIGHT_BAND)
    hi = ref[2][b, K, 2]
    wl.uniforms[b, K] = np.float32(hi + 0.5 * TIGHT_BAND)
    if wl.uniforms[b, K] < hi:  # float32 rounding put it back inside the bin
        wl.uniforms[b, K] = np.nextafter(np.float32(hi), np.float32(1.0))
    ref2 = oracle_mod.verify(wl.target, wl.draft, wl.tokens, wl.draft_len, wl.params,
                             wl.uniforms)
    assert ref2[0][b, ref2[1][b]] != ref[0][b, ref[1][b]]
    tok, acc, dg = ref2[0].copy(), ref2[1].copy(), ref2[2].copy()
    tok[b], acc[b], dg[b] = ref[0][b], ref[1][b], ref[2][b]
    rep = compare(tok, acc, dg, ref2, inputs=wl, oracle_mod=oracle_mod)
    assert rep.tight_ok and rep.mismatch_in_band_rows == [b], rep.describe()
