"""Selection checker: compares a TopK result against oracle scores.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A GPU computes fp32 scores whose head-sum rounding order differs from the
oracle's float64 sum, so near the K-th score two correct implementations may
pick different positions. The checker accepts exactly the selections that an
implementation with per-score error <= E/2 can produce, where
E = 2 * tol * max over the window of max(|score|, sum_h |w_h| ReLU(d_h)):

 (i)   every position whose oracle score exceeds tau + E is selected
       (tau = oracle K-th largest score);
 (ii)  no selected position has an oracle score below tau - E;
 (iii) exact ties: if s is selected, s' is not, and their oracle scores are
       identical, then s < s' (index tie-break of the total order);
 (iv)  exactly K distinct positions, all inside the window, ascending;
 (v)   slots are page_table[raw // 64] * 64 + raw % 64, bit-exact.

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
    mag = np.asarray(mag, np.float64)
    tau = np.partition(sigma, n - K)[n - K]          # K-th largest
    E = 2.0 * tol * float(max(np.abs(sigma).max(), mag.max()))
    sel = np.zeros(n, bool)
    sel[G - start] = True
    must = sigma > tau + E
    if np.any(must & ~sel):
        i = int(np.flatnonzero(must & ~sel)[0])
        _fail(f"{where}: position {start + i} (score {sigma[i]!r}) above tau+E={tau + E!r} not selected")
    bad = sel & (sigma < tau - E)
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        _fail(f"{where}: position {start + i} (score {sigma[i]!r}) below tau-E={tau - E!r} selected")
    # (iii) exact ties, only for values that straddle the selection boundary
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
