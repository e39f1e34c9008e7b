"""GPU-vs-oracle comparison with decision-band accounting.

Rules (the bar the GPU path is held to):
* token ids and accept lengths equal the oracle's on every row, except where
  the GPU's outcome is what the rule gives for uniforms within BAND of the
  ones passed in: oracle.explain() evaluates the rule along the GPU's outcome
  (its accepted drafts, its rejection, its final token), and the outcome is
  accepted only if every accept test it passed has u_j < a_j + BAND, the test
  it failed has u_j >= a_j - BAND, and the final uniform lies within BAND of
  the final token's CDF bin [lo, hi) (a bin of positive width).  Such rows are
  counted as mismatch_in_band, per sampler class; greedy rows use no uniform
  and must always match;
* invalid rows (-1) must match exactly; rows the GPU build does not serve
  (-2) are counted and skipped;
* probabilities reported in the diagnostics (p(x), q(x), a, and the drawn
  token's final-distribution probability and bin edges) agree within
  PROB_TOL absolute, on matching rows against the oracle's own diagnostics and
  on in-band rows against explain()'s values along the GPU's outcome.
Margins and probabilities come from the oracle (the definition), never from
the GPU.  in_band_rows counts rows whose own outcome the oracle decided with a
margin below BAND (the rows where a differing outcome can be expected).

BAND alone does not constrain untruncated and nucleus final draws: a token's
CDF bin there is about 1/V wide, narrower than BAND, so any neighbouring
token would pass.  Every in-band mismatch is therefore also checked against
TIGHT_BAND, the error the GPU's arithmetic can make in a probability or a CDF
value: per-token weights are fp32 exp2 terms (within an ulp, 2^-23, of the
exact value), summed in fp32 over a few terms per lane before the fp64 sums,
so any weight sum, normaliser or partial CDF carries a relative error below
about 5e-7, and a normalised CDF value or accept probability an absolute
error below 1e-6; TIGHT_BAND = 2e-6 leaves a factor two.  Rows explained by
BAND but not by TIGHT_BAND are listed in mismatch_beyond_tight (tight_ok).
"""
from __future__ import annotations

import dataclasses

import numpy as np

BAND = 1e-5
TIGHT_BAND = 2e-6
PROB_TOL = 1e-5
CLASSES = ("greedy", "top_k", "full", "nucleus")


@dataclasses.dataclass
class Report:
    rows: int = 0
    compared: int = 0
    exact: int = 0
    in_band_rows: int = 0
    mismatch_in_band: int = 0
    mismatch_out_of_band: list = dataclasses.field(default_factory=list)
    unsupported: int = 0
    error_rows: int = 0
    diag_max_err: float = 0.0
    diag_bad_rows: list = dataclasses.field(default_factory=list)
    min_cut_margin: float = float("inf")
    rows_by_class: dict = dataclasses.field(default_factory=dict)
    in_band_by_class: dict = dataclasses.field(default_factory=dict)
    mismatch_in_band_by_class: dict = dataclasses.field(default_factory=dict)
    mismatch_in_band_rows: list = dataclasses.field(default_factory=list)
    mismatch_beyond_tight: list = dataclasses.field(default_factory=list)

    @property
    def ok(self) -> bool:
        return (not self.mismatch_out_of_band and not self.diag_bad_rows
                and self.mismatch_in_band_by_class.get("greedy", 0) == 0)

    @property
    def tight_ok(self) -> bool:
        """ok, and every in-band mismatch within the GPU's arithmetic error."""
        return self.ok and not self.mismatch_beyond_tight

    def describe(self) -> str:
        by = " ".join(f"{c}:{self.rows_by_class.get(c, 0)}/{self.in_band_by_class.get(c, 0)}"
                      f"/{self.mismatch_in_band_by_class.get(c, 0)}" for c in CLASSES)
        return (f"rows={self.rows} compared={self.compared} exact={self.exact} "
                f"in_band={self.in_band_rows} mismatch_in_band={self.mismatch_in_band} "
                f"mismatch_out_of_band={len(self.mismatch_out_of_band)} "
                f"beyond_tight={len(self.mismatch_beyond_tight)} "
                f"unsupported={self.unsupported} error_rows={self.error_rows} "
                f"diag_max_err={self.diag_max_err:.3g} diag_bad={len(self.diag_bad_rows)} "
                f"min_topp_margin={self.min_cut_margin:.3g} "
                f"[class rows/in_band/mismatch_in_band: {by}]")


def row_class(prm, V: int) -> str:
    T, k, p = float(prm["temperature"]), int(prm["top_k"]), float(prm["top_p"])
    if T == 0.0:
        return "greedy"
    if 0 < k < V:
        return "top_k"
    return "nucleus" if p < 1.0 else "full"


def row_in_band(o_diag_row: np.ndarray) -> bool:
    m = o_diag_row[:, 3]
    m = m[~np.isnan(m)]
    return bool((m < BAND).any())


def _explained(ex, i, u, L, ga, K, band=BAND) -> bool:
    """The GPU outcome (accept length ga) of oracle row i is what the rule
    gives for uniforms within ``band`` of u (see the module docstring)."""
    if ex["status"][i] != 0:
        return False
    a = ex["a"][i]
    for j in range(ga):
        if not u[j] < a[j] + band:
            return False
    if ga < L and not u[ga] >= a[ga] - band:
        return False
    lo, hi, py = ex["lo"][i], ex["hi"][i], ex["py"][i]
    return bool(py > 0.0 and lo - band <= u[K] < hi + band)


def compare(g_tok, g_acc, g_diag, ref, rows=None, *, inputs, oracle_mod) -> Report:
    """Compare GPU outputs (numpy) against oracle outputs ``ref`` (the tuple
    returned by oracle.verify).  ``inputs`` holds the arrays the oracle ran on
    (row i = oracle row i): an object with fields target, draft, tokens,
    draft_len, params, uniforms and dtype (a workloads.Workload).  ``rows``
    maps oracle rows to GPU rows when the oracle ran on a subset."""
    o_tok, o_acc, o_diag, o_cut, _ = ref
    if rows is None:
        rows = np.arange(len(o_acc))
    rows = np.asarray(rows)
    K = o_tok.shape[1] - 1
    V = inputs.target.shape[-1]
    rep = Report(rows=len(rows))
    pending = []  # (oracle row, GPU row) pairs whose outcomes differ
    for i, b in enumerate(rows):
        ga = int(g_acc[b])
        oa = int(o_acc[i])
        if ga == -2:
            rep.unsupported += 1
            continue
        rep.compared += 1
        cls = row_class(inputs.params[i], V)
        rep.rows_by_class[cls] = rep.rows_by_class.get(cls, 0) + 1
        if np.isfinite(o_cut[i]):
            rep.min_cut_margin = min(rep.min_cut_margin, float(o_cut[i]))
        if oa == -1:
            rep.error_rows += 1
        band = oa >= 0 and row_in_band(o_diag[i])
        rep.in_band_rows += band
        if band:
            rep.in_band_by_class[cls] = rep.in_band_by_class.get(cls, 0) + 1
        if ga == oa and np.array_equal(g_tok[b], o_tok[i]):
            rep.exact += 1
            if g_diag is None or oa < 0:
                continue
            od, gd = o_diag[i], g_diag[b]
            ev = ~np.isnan(od[:, 0])
            if not np.array_equal(ev, ~np.isnan(gd[:, 0])):
                rep.diag_bad_rows.append(int(b))
                continue
            err = np.abs(od[ev][:, :3] - gd[ev][:, :3])
            e = float(err.max()) if err.size else 0.0
            rep.diag_max_err = max(rep.diag_max_err, e)
            if e > PROB_TOL:
                rep.diag_bad_rows.append(int(b))
            continue
        if oa < 0 or ga < 0 or cls == "greedy":
            if cls == "greedy" and oa >= 0 and ga >= 0:
                rep.mismatch_in_band_by_class["greedy"] = \
                    rep.mismatch_in_band_by_class.get("greedy", 0) + 1
            rep.mismatch_out_of_band.append(int(b))
            continue
        L = int(inputs.draft_len[i]) if inputs.draft_len is not None else K
        gt = np.asarray(g_tok[b])
        if (ga > L or not np.array_equal(gt[:ga], inputs.tokens[i][:ga])
                or not (gt[ga + 1:] == -1).all()):
            rep.mismatch_out_of_band.append(int(b))
            continue
        pending.append((i, int(b)))
    if pending:
        idx = np.array([p[0] for p in pending])
        gb = np.array([p[1] for p in pending])
        ga = np.asarray(g_acc)[gb].astype(np.int32)
        gy = np.asarray(g_tok)[gb, ga].astype(np.int32)
        ex = oracle_mod.explain(inputs.target[idx], inputs.draft[idx] if K > 0 else None,
                                inputs.tokens[idx],
                                inputs.draft_len[idx] if inputs.draft_len is not None else None,
                                inputs.params[idx], ga, gy, dtype=inputs.dtype)
        for n, (i, b) in enumerate(pending):
            L = int(inputs.draft_len[i]) if inputs.draft_len is not None else K
            cls = row_class(inputs.params[i], V)
            u = np.asarray(inputs.uniforms[i], np.float64)
            if not _explained(ex, n, u, L, int(ga[n]), K):
                rep.mismatch_out_of_band.append(b)
                continue
            if not _explained(ex, n, u, L, int(ga[n]), K, band=TIGHT_BAND):
                rep.mismatch_beyond_tight.append(b)
            rep.mismatch_in_band += 1
            rep.mismatch_in_band_rows.append(b)
            rep.mismatch_in_band_by_class[cls] = rep.mismatch_in_band_by_class.get(cls, 0) + 1
            if g_diag is None:
                continue
            gd = g_diag[b]
            ev = min(int(ga[n]), L - 1) + 1
            want = np.concatenate([np.stack([ex["px"][n, :ev], ex["qx"][n, :ev],
                                             ex["a"][n, :ev]], axis=1).reshape(-1),
                                   [ex["py"][n], ex["lo"][n], ex["hi"][n]]])
            got = np.concatenate([gd[:ev, :3].reshape(-1), gd[K, :3]])
            e = float(np.max(np.abs(want - got))) if want.size else 0.0
            if not np.isfinite(e) or e > PROB_TOL:
                rep.diag_bad_rows.append(b)
            else:
                rep.diag_max_err = max(rep.diag_max_err, e)
    return rep


def draws(rows, params, uniforms, dtype):
    """One draw per row (K = 0) from logits rows [B, V], as an object
    compare() takes."""
    import types

    rows = np.asarray(rows)
    B, V = rows.shape
    return types.SimpleNamespace(target=rows.reshape(B, 1, V), draft=None,
                                 tokens=np.zeros((B, 0), np.int32), draft_len=None,
                                 params=np.asarray(params),
                                 uniforms=np.asarray(uniforms, np.float32).reshape(B, 1),
                                 dtype=dtype, B=B, K=0, V=V)


def subset(wl, rows):
    """The rows ``rows`` of a workload, as an object compare() takes."""
    import copy

    rows = np.asarray(rows)
    s = copy.copy(wl)
    s.target, s.draft = wl.target[rows], wl.draft[rows]
    s.tokens, s.params, s.uniforms = wl.tokens[rows], wl.params[rows], wl.uniforms[rows]
    s.draft_len = wl.draft_len[rows] if wl.draft_len is not None else None
    s.B = len(rows)
    return s


def compare_tree(g_tok, g_len, g_path, g_diag, ref, *, inputs, oracle_mod) -> Report:
    """Tree verify: compare GPU outputs with oracle.verify_tree's ``ref``
    (out_tokens, out_len, out_path, diag, threads) under the same rules as
    compare(): identical tokens, lengths and paths, except outcomes that
    oracle.explain_tree shows the rule gives for uniforms within BAND of the
    given ones (the accepted nodes' tests u < a + BAND, the rejected
    siblings' u >= a - BAND, the final draw within BAND of its bin).
    ``inputs``: target, draft, tokens, parents, n_cand, params, uniforms,
    dtype."""
    o_tok, o_len, o_path, o_diag, _ = ref
    K = o_tok.shape[1] - 1
    V = inputs.target.shape[-1]
    B = len(o_len)
    rep = Report(rows=B)
    pending = []
    for b in range(B):
        gl, ol = int(g_len[b]), int(o_len[b])
        if gl == -2:
            rep.unsupported += 1
            continue
        rep.compared += 1
        cls = row_class(inputs.params[b], V)
        rep.rows_by_class[cls] = rep.rows_by_class.get(cls, 0) + 1
        if ol == -1:
            rep.error_rows += 1
        band = ol >= 0 and row_in_band(o_diag[b])
        rep.in_band_rows += band
        if band:
            rep.in_band_by_class[cls] = rep.in_band_by_class.get(cls, 0) + 1
        if (gl == ol and np.array_equal(g_tok[b], o_tok[b])
                and np.array_equal(g_path[b], o_path[b])):
            rep.exact += 1
            if g_diag is None or ol < 0:
                continue
            od, gd = o_diag[b], g_diag[b]
            ev = ~np.isnan(od[:, 0])
            if not np.array_equal(ev, ~np.isnan(gd[:, 0])):
                rep.diag_bad_rows.append(b)
                continue
            err = np.abs(od[ev][:, :3] - gd[ev][:, :3])
            e = float(err.max()) if err.size else 0.0
            rep.diag_max_err = max(rep.diag_max_err, e)
            if e > PROB_TOL:
                rep.diag_bad_rows.append(b)
            continue
        if ol < 0 or gl < 0 or cls == "greedy":
            if cls == "greedy" and ol >= 0 and gl >= 0:
                rep.mismatch_in_band_by_class["greedy"] = \
                    rep.mismatch_in_band_by_class.get("greedy", 0) + 1
            rep.mismatch_out_of_band.append(b)
            continue
        gp = np.asarray(g_path[b])
        gt = np.asarray(g_tok[b])
        well_formed = (gl <= K and (gp[gl:] == -1).all() and (gt[gl + 1:] == -1).all()
                       and all(0 < gp[i] <= K and gt[i] == inputs.tokens[b][gp[i] - 1]
                               for i in range(gl)))
        if not well_formed:
            rep.mismatch_out_of_band.append(b)
            continue
        pending.append(b)
    if pending:
        idx = np.array(pending)
        ex = oracle_mod.explain_tree(
            inputs.target[idx], inputs.draft[idx] if K > 0 else None, inputs.tokens[idx],
            inputs.parents[idx], inputs.n_cand[idx] if inputs.n_cand is not None else None,
            inputs.params[idx], np.asarray(g_path)[idx], np.asarray(g_len)[idx],
            np.asarray(g_tok)[idx, np.asarray(g_len)[idx]], dtype=inputs.dtype)
        def explained(n, u, band):
            a, need = ex["a"][n], ex["need"][n]
            ok = ex["status"][n] == 0
            for c in range(K):
                if need[c] == 1 and not u[c] < a[c] + band:
                    ok = False
                if need[c] == -1 and not u[c] >= a[c] - band:
                    ok = False
            return bool(ok and ex["py"][n] > 0 and ex["lo"][n] - band <= u[K] < ex["hi"][n] + band)

        for n, b in enumerate(pending):
            u = np.asarray(inputs.uniforms[b], np.float64)
            a, need = ex["a"][n], ex["need"][n]
            cls = row_class(inputs.params[b], V)
            if not explained(n, u, BAND):
                rep.mismatch_out_of_band.append(b)
                continue
            if not explained(n, u, TIGHT_BAND):
                rep.mismatch_beyond_tight.append(b)
            rep.mismatch_in_band += 1
            rep.mismatch_in_band_rows.append(b)
            rep.mismatch_in_band_by_class[cls] = rep.mismatch_in_band_by_class.get(cls, 0) + 1
            if g_diag is None:
                continue
            gd = g_diag[b]
            tested = need != 0
            want = np.concatenate([a[tested], [ex["py"][n], ex["lo"][n], ex["hi"][n]]])
            got = np.concatenate([gd[:K][tested, 2], gd[K, :3]])
            e = float(np.max(np.abs(want - got))) if want.size else 0.0
            if not np.isfinite(e) or e > PROB_TOL:
                rep.diag_bad_rows.append(b)
            else:
                rep.diag_max_err = max(rep.diag_max_err, e)
    return rep


def tree_inputs(target, draft, tokens, parents, n_cand, params, uniforms, dtype):
    """The inputs of a tree verify, as an object compare_tree() takes."""
    import types

    return types.SimpleNamespace(target=target, draft=draft, tokens=np.asarray(tokens),
                                 parents=np.asarray(parents),
                                 n_cand=None if n_cand is None else np.asarray(n_cand),
                                 params=np.asarray(params), uniforms=np.asarray(uniforms),
                                 dtype=dtype)
