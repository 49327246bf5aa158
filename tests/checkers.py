"""Independent checks of a top-k result (used on oracle and HIP outputs alike).

Nothing here computes a selection.  The checks use numpy's own float
comparison, with one stated refinement where float comparison is silent:
+0.0 ranks above -0.0 (their bit patterns differ, so they are different keys).
"Equal scores" means identical 32-bit patterns.
"""
from __future__ import annotations

import numpy as np


def _rank_value(x: np.ndarray) -> np.ndarray:
    """float64 copy of x where -0.0 is nudged strictly below +0.0 (NaN-free rows)."""
    v = x.astype(np.float64)
    negzero = (x == 0) & np.signbit(x)
    v[negzero] = -np.finfo(np.float64).tiny  # below +0.0, above every negative fp32
    return v


def check_row(values: np.ndarray, k: int, selected_pos: np.ndarray, n_pad: int) -> None:
    """Assert the invariants of an exact lowest-index top-k of one row.

    ``values``: float32 [n] valid part of the row; ``selected_pos``: positions
    (row-local) the result selected; ``n_pad``: count of -1 slots.
    """
    n = values.shape[0]
    m = min(k, n)
    sel = np.asarray(selected_pos, dtype=np.int64)
    assert sel.shape[0] == m, "expected %d selected, got %d" % (m, sel.shape[0])
    assert n_pad == k - m, "expected %d padding slots, got %d" % (k - m, n_pad)
    if m == 0:
        return
    assert sel.min() >= 0 and sel.max() < n, "selected position out of range"
    assert np.unique(sel).shape[0] == m, "duplicate positions selected"
    if m == n:
        return
    mask = np.zeros(n, dtype=bool)
    mask[sel] = True
    rv = _rank_value(values)
    lo_sel = rv[mask].min()
    hi_uns = rv[~mask].max()
    assert lo_sel >= hi_uns, "an unselected score exceeds a selected one"
    if lo_sel == hi_uns:
        # threshold ties: every unselected equal must come after every selected equal
        bits = values.view(np.uint32)
        tbits = bits[mask][rv[mask] == lo_sel]
        assert np.unique(tbits).shape[0] == 1
        eq = bits == tbits[0]
        sel_eq = np.nonzero(eq & mask)[0]
        uns_eq = np.nonzero(eq & ~mask)[0]
        if uns_eq.size:
            assert sel_eq.max() < uns_eq.min(), "tie at the threshold not broken by lowest index"


def split_output(out_row: np.ndarray):
    """(valid entries, number of -1 slots); -1 must form the tail after sorting."""
    out_row = np.asarray(out_row)
    valid = out_row[out_row != -1]
    return valid, int((out_row == -1).sum())


def recall(got: np.ndarray, want: np.ndarray) -> float:
    g = set(int(v) for v in got if v != -1)
    w = set(int(v) for v in want if v != -1)
    if not w:
        return 1.0 if not g else 0.0
    return len(g & w) / len(w)
