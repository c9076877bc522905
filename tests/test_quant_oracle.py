"""Pins of the oracle's MXFP4 quantiser (the producer of the path's FP4 inputs).

The oracle follows the OCP MX v1.0 conversion of a vector of scalars into an MX
block (E2M1 elements, UE8M0 scale); these tests pin it to hand-worked cases,
to the definition of "nearest, ties to even" by brute force over all codes, to
the scale rule's closed form, and to the round trip of values that already are
MX blocks.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mx_quant_cases.txt")


def _cases():
    out = []
    for ln in open(GOLDEN):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        name, vals, byte, codes = [f.strip() for f in ln.split("|")]
        v = np.zeros(32, np.float32)
        for i, t in enumerate(vals.split(",")):
            v[i] = np.float32(float(t))
        c = np.zeros(32, np.int64)
        for i, t in enumerate(codes.split(",")):
            c[i] = int(t, 16)
        out.append((name, v, int(byte), c))
    return out


def _elements(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_hand_worked_blocks(case):
    name, v, byte, codes = case
    c, s = oracle.mx_quantize(v)
    assert int(s[0]) == byte, name
    assert np.array_equal(_elements(c), codes), (name, _elements(c), codes)


def test_each_element_is_the_nearest_code_ties_to_even():
    """Brute force over all 16 codes: the chosen code's value is nearest to
    v / X; among equally near ones the mantissa bit is 0; the sign bit is the
    sign of v (so -0 for small negatives)."""
    rng = np.random.default_rng(5)
    table = np.array([oracle.e2m1_value(c) for c in range(16)])   # signed values, code 8 = -0
    for trial in range(400):
        scale = 2.0 ** rng.integers(-20, 20)
        x = (rng.standard_normal(32) * scale * rng.choice([0.01, 1, 5])).astype(np.float32)
        if trial % 7 == 0:      # plant exact ties
            X = 2.0 ** (np.floor(np.log2(np.abs(x).max())) - 2)
            x[:8] = (np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25]) * X).astype(np.float32)
        c, s = oracle.mx_quantize(x)
        X = 2.0 ** (int(s[0]) - 127)
        el = _elements(c)
        for i in range(32):
            t = float(x[i]) / X
            d = np.abs(table - t)
            same_sign = np.array([(cc >= 8) == bool(np.signbit(t)) for cc in range(16)])
            best = d[same_sign].min()
            cand = [cc for cc in range(16) if same_sign[cc] and d[cc] == best]
            want = [cc for cc in cand if (cc & 1) == 0] or cand
            assert el[i] in want and (len(cand) == 1 or el[i] == want[0]), (trial, i, t, el[i], cand)


def test_scale_rule_closed_form():
    """For a finite non-zero block the scale X satisfies 4 X <= max|v| < 8 X
    (the largest element lands in [4, 8) before rounding), unless clamped."""
    rng = np.random.default_rng(6)
    for _ in range(500):
        e = rng.integers(-120, 120)
        x = (rng.uniform(-1, 1, 32) * 2.0 ** e).astype(np.float32)
        amax = float(np.abs(x).max())
        if amax == 0:
            continue
        s = oracle.mx_quantize(x)[1][0]
        X = 2.0 ** (int(s) - 127)
        assert 4 * X <= amax < 8 * X, (e, amax, s)


def test_values_that_are_mx_blocks_round_trip():
    """Dequantised MX blocks (any codes, scale bytes away from the clamp) come
    back with the same values, signed zeros included."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, (300, 64), dtype=np.uint8)
    scales = rng.integers(10, 240, (300, 4), dtype=np.uint8)
    vals = oracle.mx_dequantize(codes, scales).astype(np.float32)
    c2, s2 = oracle.mx_quantize(vals)
    back = oracle.mx_dequantize(c2, s2)
    assert np.array_equal(back, vals.astype(np.float64))
    assert np.array_equal(np.signbit(back), np.signbit(vals))


def test_packing_low_nibble_first():
    x = np.zeros(32, np.float32)
    x[0], x[1] = 6.0, 1.0          # X = 1: codes 7 and 2
    c, _ = oracle.mx_quantize(x)
    assert c[0] == 0x27
