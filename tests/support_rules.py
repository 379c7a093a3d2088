"""Near-tie comparison of a selected index set against the oracle's scores.

A row's set passes when it has exactly k_eff = min(k, units) distinct entries
in ascending order, contains every unit whose score exceeds the oracle's k-th
score by more than ``band``, holds none more than ``band`` below it, and has
no unit beyond the causal range. Units within the band of the k-th score may
go either way (several sets are correct there).
"""
import numpy as np


def check_row(units, count, score, kth, k, band=1e-6):
    """Returns (ok: bool, message: str, n_in_band: int)."""
    n_units = score.shape[0]
    k_eff = min(k, n_units)
    units = np.asarray(units)
    if int(count) != k_eff:
        return False, f"count {count} != {k_eff}", 0
    sel = units[:k_eff]
    pad = units[k_eff:]
    if pad.size and np.any(pad != -1):
        return False, "padding is not -1", 0
    if np.any(sel < 0) or np.any(sel >= n_units):
        return False, f"unit out of causal range: {sel[(sel < 0) | (sel >= n_units)][:5]}", 0
    if np.any(np.diff(sel) <= 0):
        return False, "units not strictly ascending", 0
    if k_eff == n_units:
        return True, "all", 0
    must_in = np.nonzero(score > kth + band)[0]
    must_out = score < kth - band
    missing = np.setdiff1d(must_in, sel)
    if missing.size:
        return False, f"missing must-in units {missing[:8]} (scores {score[missing[:4]]}, kth {kth})", 0
    wrong = sel[must_out[sel]]
    if wrong.size:
        return False, f"selected must-out units {wrong[:8]} (scores {score[wrong[:4]]}, kth {kth})", 0
    in_band = int(np.sum(np.abs(score - kth) <= band))
    return True, "ok", in_band
