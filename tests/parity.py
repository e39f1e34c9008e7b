"""GPU-vs-oracle comparison with decision-band accounting.

Rules (the bar the GPU path is held to):
* token ids and accept lengths must equal the oracle's on every row, except
  rows where a uniform lies within BAND of a decision threshold that fixed the
  row's outcome (an evaluated accept test |u - a|, or the final draw's CDF bin
  edges); those rows are counted as in band and may differ;
* invalid rows (-1) must match exactly; rows the GPU build does not serve
  (-2) are counted and skipped;
* probabilities reported in the diagnostics (p(x), q(x), a, and the drawn
  token's final-distribution probability and bin edges) must agree within
  PROB_TOL absolute on rows whose outcome matches.
Margins come from the oracle (the definition), never from the GPU.
"""
from __future__ import annotations

import dataclasses

import numpy as np

BAND = 1e-5
PROB_TOL = 1e-5


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

    @property
    def ok(self) -> bool:
        return not self.mismatch_out_of_band and not self.diag_bad_rows

    def describe(self) -> str:
        return (f"rows={self.rows} compared={self.compared} exact={self.exact} "
                f"in_band={self.in_band_rows} mismatch_in_band={self.mismatch_in_band} "
                f"mismatch_out_of_band={len(self.mismatch_out_of_band)} "
                f"unsupported={self.unsupported} error_rows={self.error_rows} "
                f"diag_max_err={self.diag_max_err:.3g} diag_bad={len(self.diag_bad_rows)} "
                f"min_topp_margin={self.min_cut_margin:.3g}")


def row_in_band(o_diag_row: np.ndarray, K: int) -> bool:
    m = o_diag_row[:, 3]
    m = m[~np.isnan(m)]
    return bool((m < BAND).any())


def compare(g_tok, g_acc, g_diag, ref, rows=None) -> Report:
    """Compare GPU outputs (numpy) against oracle outputs ``ref`` (the tuple
    returned by oracle.verify).  ``rows`` maps oracle rows to GPU rows when the
    oracle ran on a sample."""
    o_tok, o_acc, o_diag, o_cut, _ = ref
    if rows is None:
        rows = np.arange(len(o_acc))
    rows = np.asarray(rows)
    K = o_tok.shape[1] - 1
    rep = Report(rows=len(rows))
    for i, b in enumerate(rows):
        ga = int(g_acc[b])
        oa = int(o_acc[i])
        if ga == -2:
            rep.unsupported += 1
            continue
        rep.compared += 1
        if np.isfinite(o_cut[i]):
            rep.min_cut_margin = min(rep.min_cut_margin, float(o_cut[i]))
        if oa == -1:
            rep.error_rows += 1
        same = ga == oa and np.array_equal(g_tok[b], o_tok[i])
        band = oa >= 0 and row_in_band(o_diag[i], K)
        rep.in_band_rows += band
        if same:
            rep.exact += 1
        elif band:
            rep.mismatch_in_band += 1
            continue
        else:
            rep.mismatch_out_of_band.append(int(b))
            continue
        if g_diag is None or oa < 0:
            continue
        od, gd = o_diag[i], g_diag[b]
        ev = ~np.isnan(od[:, 0])
        if not np.array_equal(ev, ~np.isnan(gd[:, 0])):
            rep.diag_bad_rows.append(int(b))
            continue
        cols = [0, 1, 2]
        err = np.abs(od[ev][:, cols] - gd[ev][:, cols])
        e = float(err.max()) if err.size else 0.0
        rep.diag_max_err = max(rep.diag_max_err, e)
        if e > PROB_TOL:
            rep.diag_bad_rows.append(int(b))
    return rep
