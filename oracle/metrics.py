"""Parity metrics between a GPU bf16 output and the oracle's bf16 output.

Test infrastructure only (see ``oracle/__init__.py``).

The bar: relative L2 error <= 1e-3 over the whole output, and for every
output row m, max_n |Y - Y_ref| <= 2e-2 * max_n |Y_ref|.  Both are computed
in float64 over the two bf16 arrays.  "row" is the oracle's output row
(over n).  Parity: pinned by tests/test_oracle_metrics.py (hand values).
"""
import numpy as np

REL_L2_TOL = 1e-3
ROW_MAXABS_TOL = 2e-2


def rel_l2(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(r)
    num = np.linalg.norm(y - r)
    if den == 0:
        return 0.0 if num == 0 else np.inf
    return float(num / den)


def row_maxabs_ratio(y, y_ref):
    """max over rows of max_n|Y-Y_ref| / max_n|Y_ref| (0/0 -> 0)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    if r.size == 0:
        return 0.0
    num = np.max(np.abs(y - r), axis=-1)
    den = np.max(np.abs(r), axis=-1)
    ratio = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(np.max(ratio))


def check_output(y, y_ref, rel_tol=REL_L2_TOL, row_tol=ROW_MAXABS_TOL):
    """Returns (ok, rel_l2, row_ratio)."""
    rl = rel_l2(y, y_ref)
    rr = row_maxabs_ratio(y, y_ref)
    ok = bool(np.all(np.isfinite(np.asarray(y, dtype=np.float64)))) and rl <= rel_tol and rr <= row_tol
    return ok, rl, rr
