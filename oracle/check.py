"""Selection checker: compares a TopK result against oracle scores.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A GPU computes fp32 scores whose head-sum rounding order differs from the
oracle's float64 sum, so near the K-th score two correct implementations may
pick different positions. The tolerance is per score: an implementation is
correct when every score it computes lies within

    e(s) = tol * max(|sigma_s|, m_s),   m_s = sum_h |w_h| ReLU(d_h(s)),

of the oracle's float64 score sigma_s (tol = 1e-5; m_s is the score's own
magnitude, which differs from |sigma_s| only where the heads' terms cancel).
Such an implementation ranks an unselected position s at or below a selected
position s' only if sigma_s - e(s) <= sigma_s' + e(s'). So a selection G is
accepted exactly when it is one that some scores inside those bounds give:

 (i)   max over s not in G of (sigma_s - e(s)) <= min over s' in G of
       (sigma_s' + e(s')): near the K-th score tau the swap band is about
       e(tau) on either side, and nothing farther from tau may swap;
 (ii)  exact ties: if s is selected, s' is not, and their oracle scores are
       identical, then s < s' (index tie-break of the total order);
 (iii) exactly K distinct positions, all inside the window, ascending;
 (iv)  slots are page_table[raw // 64] * 64 + raw % 64, bit-exact.

check_scores() applies the same per-score bound to returned fp32 scores.
Rows with non-finite scores are compared exactly against the oracle's own
selection. Short rows are compared exactly (sequential positions, -1 pad).
"""
from __future__ import annotations

import numpy as np

DEFAULT_TOL = 1e-5


class SelectionMismatch(AssertionError):
    pass


def _fail(msg):
    raise SelectionMismatch(msg)


def score_bound(sigma, mag, tol: float = DEFAULT_TOL) -> np.ndarray:
    """Per-score tolerance e(s) = tol * max(|sigma_s|, m_s)."""
    return tol * np.maximum(np.abs(np.asarray(sigma, np.float64)), np.asarray(mag, np.float64))


def check_scores(got, sigma, mag, tol: float = DEFAULT_TOL, where: str = ""):
    """Every returned fp32 score within its own bound of the oracle's score."""
    got = np.asarray(got, np.float64)
    sigma = np.asarray(sigma, np.float64)
    e = score_bound(sigma, mag, tol)
    err = np.abs(got - sigma)
    bad = ~(err <= e)
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        _fail(f"{where}: score {got[i]!r} vs oracle {sigma[i]!r}: error {err[i]!r} > bound {e[i]!r}")


def expected_slots(raw: np.ndarray, page_table: np.ndarray) -> np.ndarray:
    raw = np.asarray(raw, np.int64)
    out = np.full(raw.shape, -1, np.int64)
    m = raw >= 0
    out[m] = page_table[raw[m] // 64].astype(np.int64) * 64 + raw[m] % 64
    return out


def check_short_row(start, end, K, raw, slot, count, page_table, where=""):
    n = end - start
    exp_raw = np.full(K, -1, np.int64)
    exp_raw[:n] = np.arange(start, end)
    if count != n:
        _fail(f"{where}: short row count {count} != {n}")
    if not np.array_equal(np.asarray(raw, np.int64), exp_raw):
        _fail(f"{where}: short row raw mismatch")
    if not np.array_equal(np.asarray(slot, np.int64), expected_slots(exp_raw, page_table)):
        _fail(f"{where}: short row slot mismatch")


def check_long_row(sigma, mag, start, K, raw, slot, count, page_table, tol=DEFAULT_TOL,
                   oracle_sel=None, where=""):
    """sigma, mag: float64 oracle scores / magnitudes of the window positions
    start..start+len-1. raw/slot/count: the implementation's outputs."""
    sigma = np.asarray(sigma, np.float64)
    n = sigma.shape[0]
    raw = np.asarray(raw, np.int64)
    if count != K:
        _fail(f"{where}: long row count {count} != K={K}")
    G = raw[:K]
    if np.any(G < start) or np.any(G >= start + n):
        _fail(f"{where}: selected position outside the window")
    if np.any(np.diff(G) <= 0):
        _fail(f"{where}: selected positions not strictly ascending")
    if not np.array_equal(np.asarray(slot, np.int64)[:K], expected_slots(G, page_table)):
        _fail(f"{where}: slot mismatch")
    if not np.all(np.isfinite(sigma)):
        if oracle_sel is None:
            _fail(f"{where}: non-finite scores need the oracle selection")
        if not np.array_equal(G, np.asarray(oracle_sel, np.int64)[:K]):
            _fail(f"{where}: selection differs from the oracle on a row with special values")
        return
    e = score_bound(sigma, mag, tol)
    sel = np.zeros(n, bool)
    sel[G - start] = True
    # (i) consistent with some scores inside the per-score bounds
    lo_out = sigma - e
    hi_in = sigma + e
    i_out = int(np.argmax(np.where(sel, -np.inf, lo_out)))
    i_in = int(np.argmin(np.where(sel, hi_in, np.inf)))
    if not sel[i_out] and sel[i_in] and lo_out[i_out] > hi_in[i_in]:
        _fail(f"{where}: position {start + i_out} (score {sigma[i_out]!r}, bound {e[i_out]!r}) not selected "
              f"but position {start + i_in} (score {sigma[i_in]!r}, bound {e[i_in]!r}) is")
    # (ii) exact ties, only for values that straddle the selection boundary
    in_vals = np.unique(sigma[sel])
    out_vals = np.unique(sigma[~sel])
    both = np.intersect1d(in_vals, out_vals)
    for v in both:
        idx = np.flatnonzero(sigma == v)
        s_in = idx[sel[idx]]
        s_out = idx[~sel[idx]]
        if s_in.max() > s_out.min():
            _fail(f"{where}: tie at score {v!r}: selected {start + s_in.max()} after "
                  f"unselected {start + s_out.min()}")
