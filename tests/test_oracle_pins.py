"""Pins of the CPU oracle against what the pages and mathematics fix.

Every check here is independent of the oracle's own formulas: golden tables
written from the format definitions and the pages' rules, closed forms,
invariants, Python's sort as the textbook total order, and an exact-rational
brute force with its own bit-field decoding.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.check import check_long_row, check_short_row, SelectionMismatch
from fp4_mqa_scoring_amd import synth
import golden_io


def f32(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def one_hot_vec(element: int, code: int) -> np.ndarray:
    v = np.zeros(64, np.uint8)
    v[element // 2] = (code << 4) if element % 2 else code
    return v


# --- decoding -------------------------------------------------------------------

def test_e2m1_table_matches_ocp_fixture_and_bitfields():
    for code, s, e, m, value in golden_io.e2m1_table():
        assert code == (s << 3) | (e << 1) | m
        got = oracle.e2m1_value(code)
        assert got == value and math.copysign(1, got) == math.copysign(1, value), code
        assert Fraction(got) == brute.e2m1_from_bits(code)


def test_ue8m0_powers_of_two():
    assert oracle.ue8m0_value(127) == 1.0
    assert oracle.ue8m0_value(128) == 2.0
    assert oracle.ue8m0_value(125) == 0.25
    assert oracle.ue8m0_value(0) == 2.0 ** -127
    assert oracle.ue8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle.ue8m0_value(255))


# --- per-head dot product: closed forms -----------------------------------------

@pytest.mark.parametrize("element", [0, 1, 30, 31, 32, 33, 64, 95, 96, 127])
def test_head_dot_one_hot_uses_its_own_block_scale(element):
    qs = np.array([120, 125, 130, 133], np.uint8)       # distinct per block
    ks = np.array([131, 126, 122, 128], np.uint8)
    q = one_hot_vec(element, 0x3)       # 1.5
    k = one_hot_vec(element, 0xE)       # -4.0
    b = element // 32
    want = 1.5 * -4.0 * 2.0 ** (int(qs[b]) + int(ks[b]) - 254)
    assert oracle.head_dot(q, qs, k, ks) == want


def test_head_dot_pairs_elements_by_index_only():
    qs = ks = np.full(4, 127, np.uint8)
    # element 2j (low nibble) against element 2j+1 (high nibble) of the same byte
    q = one_hot_vec(10, 0x2)
    k = one_hot_vec(11, 0x2)
    assert oracle.head_dot(q, qs, k, ks) == 0.0
    assert oracle.head_dot(q, qs, one_hot_vec(10, 0x7), ks) == 6.0
    # different elements in different blocks
    assert oracle.head_dot(one_hot_vec(3, 7), qs, one_hot_vec(35, 7), ks) == 0.0


def test_head_dot_all_sixes_is_the_maximum():
    v = np.full(64, 0x77, np.uint8)       # every element 6.0
    s = np.full(4, 127, np.uint8)
    assert oracle.head_dot(v, s, v, s) == 128 * 36.0
    neg = np.full(64, 0xFF, np.uint8)     # every element -6.0
    assert oracle.head_dot(v, s, neg, s) == -128 * 36.0


def test_head_dot_matches_exact_rationals_on_random_vectors():
    rng = np.random.default_rng(5)
    for _ in range(40):
        q = rng.integers(0, 256, 64, dtype=np.uint8)
        k = rng.integers(0, 256, 64, dtype=np.uint8)
        qs = rng.integers(119, 136, 4).astype(np.uint8)     # spans well inside 2^38
        ks = rng.integers(119, 136, 4).astype(np.uint8)
        assert Fraction(oracle.head_dot(q, qs, k, ks)) == brute.head_dot(q, qs, k, ks)


def test_head_dot_wide_scale_spread_is_accurate_to_float64():
    rng = np.random.default_rng(15)
    for _ in range(40):
        q = rng.integers(0, 256, 64, dtype=np.uint8)
        k = rng.integers(0, 256, 64, dtype=np.uint8)
        qs = rng.integers(60, 200, 4).astype(np.uint8)
        ks = rng.integers(60, 200, 4).astype(np.uint8)
        exact = brute.head_dot(q, qs, k, ks)
        bound = sum(Fraction(1152) * brute.ue8m0_exact(qs[b]) * brute.ue8m0_exact(ks[b])
                    for b in range(4))
        assert abs(Fraction(oracle.head_dot(q, qs, k, ks)) - exact) <= Fraction(2) ** -50 * bound


def test_negating_query_bytes_negates_the_dot():
    rng = np.random.default_rng(6)
    q = rng.integers(0, 256, 64, dtype=np.uint8)
    k = rng.integers(0, 256, 64, dtype=np.uint8)
    s = np.full(4, 128, np.uint8)
    assert oracle.head_dot(q ^ 0x88, s, k, s) == -oracle.head_dot(q, s, k, s)


# --- scores ---------------------------------------------------------------------------

def tiny_inputs(seed=1, Q=3, S=256, K=8, **kw):
    rng = np.random.default_rng(seed)
    if "row_start" not in kw:
        st = rng.integers(0, S // 2, Q).astype(np.int32)
        en = (st + rng.integers(K + 1, S // 2, Q)).astype(np.int32)
        kw["row_start"], kw["row_end"] = st, en
    return synth.make_inputs(Q, S, K, seed, **kw)


def test_one_hot_weights_give_relu_of_each_head():
    inp = tiny_inputs(2)
    row, pos = 1, int(inp.row_start[1]) + 3
    page = int(inp.page_table[pos // 64])
    kv, ks = inp.k_pages[page, pos % 64], inp.k_scale[page, pos % 64]
    for h in (0, 17, 63):
        inp.weights[row] = 0
        inp.weights[row, h] = 1.0
        s, m = oracle.row_scores(inp, row, pos, pos + 1)
        d = oracle.head_dot(inp.q[row, h], inp.q_scale[row, h], kv, ks)
        assert s[0] == max(d, 0.0) and m[0] == max(d, 0.0)


def test_all_zero_query_scores_positive_zero():
    inp = tiny_inputs(3)
    inp.q[0] = 0
    s, m = oracle.row_scores(inp, 0)
    assert np.all(s == 0.0) and not np.any(np.signbit(s))
    assert np.all(m == 0.0)


def test_scores_homogeneous_in_weights_and_query_scales():
    inp = tiny_inputs(4)
    base, _ = oracle.row_scores(inp, 2)
    inp.weights[2] *= 2.0
    s2, _ = oracle.row_scores(inp, 2)
    assert np.array_equal(s2, 2.0 * base)
    inp.weights[2] *= 0.5
    inp.q_scale[2] += 3
    s8, _ = oracle.row_scores(inp, 2)
    assert np.array_equal(s8, 8.0 * base)


def test_nonpositive_weights_give_nonpositive_scores():
    inp = tiny_inputs(5)
    inp.weights[0] = -np.abs(inp.weights[0])
    s, _ = oracle.row_scores(inp, 0)
    assert np.all(s <= 0.0)


def test_scores_match_exact_rationals():
    inp = tiny_inputs(7, Q=2, S=128, K=4)
    for row in range(inp.Q):
        s, m = oracle.row_scores(inp, row)
        exact = brute.row_scores(inp, row)
        for a, b, mm in zip(s, exact, m):
            assert abs(Fraction(a) - b) <= Fraction(1e-14) * max(Fraction(mm), Fraction(1))


@pytest.mark.parametrize("seed,K", [(11, 4), (12, 8), (13, 8)])
def test_topk_rows_match_brute_force(seed, K):
    inp = tiny_inputs(seed, Q=3, S=192, K=K)
    for row in range(inp.Q):
        cnt, raw, sl, sc = oracle.topk_row(inp, row, K)
        exact = brute.row_scores(inp, row)
        want = brute.topk(exact, int(inp.row_start[row]), K)
        assert cnt == K and list(raw) == want
        for r, ss in zip(raw, sl):
            assert ss == int(inp.page_table[r // 64]) * 64 + r % 64


def test_duplicate_keys_tie_by_index_in_brute_force_and_oracle():
    inp = tiny_inputs(21, Q=1, S=128, K=4, row_start=np.array([0], np.int32),
                      row_end=np.array([128], np.int32), dup_frac=0.5)
    cnt, raw, _, _ = oracle.topk_row(inp, 0, 4)
    exact = brute.row_scores(inp, 0)
    assert list(raw) == brute.topk(exact, 0, 4)
    assert len(set(exact)) < len(exact)         # the fixture really has ties


# --- total order -------------------------------------------------------------------

def python_rank_key(score: float, index: int):
    """Textbook statement of the order as a Python sort key."""
    if math.isnan(score):
        return (1, 0.0, 0, index)
    return (0, -score, 1 if math.copysign(1.0, score) < 0 else 0, index)


@pytest.mark.parametrize("case", golden_io.total_order_cases(), ids=lambda c: c["name"])
def test_total_order_golden(case):
    scores = [f32(b) for b in case["scores"]]
    idx = list(range(case["start"], case["start"] + len(scores)))
    by_python = [i for _, i in sorted(((python_rank_key(s, i), i) for s, i in zip(scores, idx)))]
    assert by_python == case["order"]
    n = len(scores)
    for a in range(n):
        for b in range(n):
            if a != b:
                before = case["order"].index(idx[a]) < case["order"].index(idx[b])
                assert oracle.ranks_before(scores[a], idx[a], scores[b], idx[b]) == before
    cnt, raw = oracle.select_topk(np.array(scores), case["start"], case["K"])
    assert cnt == case["K"] and list(raw) == case["topk"]


def test_select_matches_python_sort_on_random_arrays_with_ties():
    rng = np.random.default_rng(8)
    for _ in range(20):
        n = int(rng.integers(5, 300))
        vals = rng.choice([-2.0, -0.0, 0.0, 0.5, 1.0, np.inf, -np.inf, np.nan, 3.0], size=n)
        vals = np.where(rng.random(n) < 0.5, rng.standard_normal(n).round(1), vals)
        start = int(rng.integers(0, 1000))
        K = int(rng.integers(1, n))
        order = sorted(range(n), key=lambda i: python_rank_key(vals[i], start + i))
        want = sorted(start + i for i in order[:K])
        cnt, raw = oracle.select_topk(vals, start, K)
        assert cnt == K and list(raw) == want


def test_exact_candidate_union():
    """TopK of a window equals TopK of the union of per-piece TopKs (any split)."""
    rng = np.random.default_rng(9)
    for _ in range(10):
        n, K = int(rng.integers(50, 400)), int(rng.integers(1, 40))
        vals = rng.integers(-5, 6, n).astype(np.float64)      # many exact ties
        start = int(rng.integers(0, 100))
        _, whole = oracle.select_topk(vals, start, K)
        cuts = np.sort(rng.choice(np.arange(1, n), size=int(rng.integers(1, 6)), replace=False))
        bounds = [0, *cuts.tolist(), n]
        cand = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            c, r = oracle.select_topk(vals[a:b], start + a, K)
            cand += [int(x) for x in r[:c]]
        cand = sorted(cand)
        cvals = np.array([vals[i - start] for i in cand])
        # select over the candidate union in rank order (indices are not contiguous)
        order = sorted(range(len(cand)), key=lambda i: python_rank_key(cvals[i], cand[i]))
        merged = sorted(cand[i] for i in order[:K])
        assert merged == list(whole[:K])


# --- short rows, validation, page map ----------------------------------------------------

@pytest.mark.parametrize("start,end,K,expected", golden_io.short_rows())
def test_short_rows_golden(start, end, K, expected):
    cnt, raw = oracle.select_topk(np.zeros(end - start), start, K)
    assert cnt == end - start and list(raw) == expected


def test_validation_codes():
    pt = np.array([3, 0, 7, 2], np.int32)          # P_log = 4, P_phys = 5 -> entry 7 is bad
    L = oracle.lib()
    p = pt.ctypes.data_as(oracle.ctypes.c_void_p)
    assert L.oracle_validate_row(0, 64, p, 4, 5) == 0
    assert L.oracle_validate_row(64, 128, p, 4, 5) == 0
    assert L.oracle_validate_row(100, 129, p, 4, 5) == -2     # touches page 2
    assert L.oracle_validate_row(192, 256, p, 4, 5) == 0
    assert L.oracle_validate_row(128, 128, p, 4, 5) == 0      # empty window touches nothing
    assert L.oracle_validate_row(-1, 10, p, 4, 5) == -1
    assert L.oracle_validate_row(10, 9, p, 4, 5) == -1
    assert L.oracle_validate_row(0, 257, p, 4, 5) == -1
    assert L.oracle_validate_row(256, 256, p, 4, 5) == 0


def test_page_map_closed_form_and_permutation_invariance():
    inp = tiny_inputs(31, Q=2, S=512, K=16, P_phys=11)
    rows = [0, 1]
    cnt, raw, sl, _ = oracle.topk_rows(inp, rows)
    for i, r in enumerate(rows):
        for x, s in zip(raw[i][:cnt[i]], sl[i][:cnt[i]]):
            assert s == oracle.slot(int(x), inp.page_table)
            assert s == int(inp.page_table[x // 64]) * 64 + int(x) % 64
    # move the physical pages around and update the table: raw and count unchanged
    rng = np.random.default_rng(3)
    perm = rng.permutation(inp.P_phys)
    new_pages = np.empty_like(inp.k_pages)
    new_scale = np.empty_like(inp.k_scale)
    new_pages[perm] = inp.k_pages
    new_scale[perm] = inp.k_scale
    moved = synth.Inputs(q=inp.q, q_scale=inp.q_scale, k_pages=new_pages, k_scale=new_scale,
                         weights=inp.weights, page_table=perm[inp.page_table].astype(np.int32),
                         row_start=inp.row_start, row_end=inp.row_end, K=inp.K)
    cnt2, raw2, sl2, _ = oracle.topk_rows(moved, rows)
    assert np.array_equal(cnt, cnt2) and np.array_equal(raw, raw2)
    for i in range(2):
        m = raw2[i] >= 0
        assert np.array_equal(sl2[i][m], perm[inp.page_table[raw2[i][m] // 64]] * 64 + raw2[i][m] % 64)


def test_invalid_rows_fail_closed():
    inp = tiny_inputs(41, Q=3, S=256, K=8)
    inp.row_start[0], inp.row_end[0] = 10, 5
    inp.page_table[1] = 99
    inp.row_start[1], inp.row_end[1] = 60, 70                # touches page 1
    for row, code in ((0, -1), (1, -2)):
        cnt, raw, sl, _ = oracle.topk_row(inp, row)
        assert cnt == code and np.all(raw == -1) and np.all(sl == -1)


def test_all_equal_rows_select_the_first_K_positions():
    inp = tiny_inputs(51, Q=1, S=512, K=16, row_start=np.array([37], np.int32),
                      row_end=np.array([500], np.int32))
    inp.q[0] = 0
    cnt, raw, _, _ = oracle.topk_row(inp, 0)
    assert cnt == 16 and list(raw) == list(range(37, 53))


def test_special_weights_produce_ordered_specials():
    inp = tiny_inputs(61, Q=1, S=128, K=8, row_start=np.array([0], np.int32),
                      row_end=np.array([128], np.int32))
    inp.weights[0] = 0
    inp.weights[0, 5] = np.inf
    s, _ = oracle.row_scores(inp, 0)
    # +inf where head 5's dot is positive, NaN (inf * 0) where it is not
    assert np.all(np.isposinf(s) | np.isnan(s))
    cnt, raw, _, _ = oracle.topk_row(inp, 0)
    pos_inf = np.flatnonzero(np.isposinf(s))
    want = sorted(pos_inf[:8]) if len(pos_inf) >= 8 else sorted(
        list(pos_inf) + list(np.flatnonzero(np.isnan(s))[:8 - len(pos_inf)]))
    assert list(raw) == [int(x) for x in want]


# --- the checker itself (planted mistakes are caught) ---------------------------------

def test_checker_accepts_oracle_and_rejects_planted_mistakes():
    inp = tiny_inputs(71, Q=1, S=1024, K=32, row_start=np.array([5], np.int32),
                      row_end=np.array([1000], np.int32))
    s, m = oracle.row_scores(inp, 0)
    cnt, raw, sl, _ = oracle.topk_row(inp, 0)
    check_long_row(s, m, 5, 32, raw, sl, cnt, inp.page_table)
    # swap a clearly-selected position for a clearly-unselected one
    worst = int(np.argmin(s)) + 5
    bad = raw.copy()
    bad[0] = worst
    bad = np.sort(bad)
    with pytest.raises(SelectionMismatch):
        check_long_row(s, m, 5, 32, bad, oracle.check.expected_slots(bad, inp.page_table), cnt,
                       inp.page_table)
    badslot = sl.copy()
    badslot[3] += 1
    with pytest.raises(SelectionMismatch):
        check_long_row(s, m, 5, 32, raw, badslot, cnt, inp.page_table)
    with pytest.raises(SelectionMismatch):
        check_short_row(3, 6, 8, [3, 4, 5, -1, -1, -1, -1, -1], [0] * 8, 3, inp.page_table)


def test_checker_enforces_index_tie_break():
    sigma = np.array([1.0, 2.0, 2.0, 2.0, 0.5])
    pt = np.arange(4, dtype=np.int32)
    ok = np.array([1, 2])
    check_long_row(sigma, np.abs(sigma), 0, 2, ok, oracle.check.expected_slots(ok, pt), 2, pt)
    wrong = np.array([1, 3])
    with pytest.raises(SelectionMismatch):
        check_long_row(sigma, np.abs(sigma), 0, 2, wrong, oracle.check.expected_slots(wrong, pt), 2, pt)


def _tau_row(n=400, K=32, seed=3, spread=None, mag_factor=1.5):
    """Synthetic oracle scores with known magnitudes, the K-th largest tau, and
    the exact top-K positions (start 0)."""
    rng = np.random.default_rng(seed)
    sigma = rng.normal(100.0, 30.0, n)
    mag = np.abs(sigma) * mag_factor
    if spread is not None:
        sigma[-1] = spread                          # one far-away score that sets the window maximum
        mag[-1] = abs(spread)
    order = np.argsort(-sigma, kind="stable")
    top = np.sort(order[:K])
    tau = sigma[order[K - 1]]
    return sigma, mag, top, order, tau


@pytest.mark.parametrize("mag_factor", [1.0, 1.5])
def test_checker_swap_band_is_per_score(mag_factor):
    """Near the K-th score tau a swap is allowed only within the two scores' own
    bounds e(s) = 1e-5 * max(|s|, m_s): with m = |s| (no cancellation) a selected
    score 2.1e-5 * tau below tau is rejected and one 1.9e-5 * tau below is
    accepted; with m = 1.5 |s| the band scales with m."""
    from oracle.check import score_bound
    pt = np.arange(64, dtype=np.int32)
    K = 32
    sigma, mag, top, order, tau = _tau_row(K=K, mag_factor=mag_factor)
    check_long_row(sigma, mag, 0, K, top, oracle.check.expected_slots(top, pt), K, pt)
    kth, nxt = order[K - 1], order[K]
    for frac, ok in ((0.95, True), (1.05, False)):
        s = sigma.copy()
        m = mag.copy()
        m[nxt] = mag_factor * tau                   # the swapped-in score's magnitude, about tau's
        band = float(score_bound(tau, mag[kth]) + score_bound(tau, m[nxt]))
        if mag_factor == 1.0:
            assert abs(band - 2e-5 * tau) < 1e-12 * tau
        s[nxt] = tau - frac * band                  # |s| < m[nxt], so e(nxt) is 1e-5 * m[nxt]
        swapped = np.sort(np.concatenate([top[top != kth], [nxt]]))
        args = (s, m, 0, K, swapped, oracle.check.expected_slots(swapped, pt), K, pt)
        if ok:
            check_long_row(*args)
        else:
            with pytest.raises(SelectionMismatch):
                check_long_row(*args)


def test_checker_band_does_not_widen_with_the_window_maximum():
    """A window holding one very large score: the old window-wide band (2e-5 *
    the window's maximum magnitude) would allow swaps far below tau; the
    per-score band does not."""
    pt = np.arange(64, dtype=np.int32)
    K = 32
    sigma, mag, top, order, tau = _tau_row(K=K, spread=1e7)
    kth, far = order[K - 1], order[K + 40]            # well below tau, inside 2e-5 * 1e7 = 200
    assert tau - sigma[far] < 2e-5 * 1e7
    swapped = np.sort(np.concatenate([top[top != kth], [far]]))
    with pytest.raises(SelectionMismatch):
        check_long_row(sigma, mag, 0, K, swapped, oracle.check.expected_slots(swapped, pt), K, pt)


def test_check_scores_bound_is_per_score():
    from oracle.check import check_scores, score_bound
    sigma = np.array([1000.0, -5.0, 0.0, 3.0])
    mag = np.array([1000.0, 400.0, 0.0, 3.0])
    e = score_bound(sigma, mag)
    assert np.array_equal(e, 1e-5 * np.array([1000.0, 400.0, 0.0, 3.0]))
    check_scores(sigma + 0.99 * e * np.array([1, -1, 1, 1]), sigma, mag)
    for i in range(4):
        got = sigma.copy()
        got[i] += 1.01 * e[i] if e[i] > 0 else 1e-30     # a zero score must be exact
        with pytest.raises(SelectionMismatch):
            check_scores(got, sigma, mag)


# --- geometry printed on the pages ---------------------------------------------------------

def test_page_geometry_golden():
    pairs, dense = golden_io.geometry()
    for raw, c4 in pairs:
        assert raw // 4 == c4
    assert synth.CONFIGS["H"]["S"] == 196608 and synth.CONFIGS[5]["S"] == 262144
    assert dense["c4"] * 4 == dense["bytes_per_row"]
    assert dense["bytes_per_row"] / 2 ** 20 == dense["mib_per_row"]
    assert dense["rows"] * dense["bytes_per_row"] / 2 ** 20 == dense["mib_total"]
