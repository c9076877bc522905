"""Exact-rational brute force for tiny inputs (pins the C oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Independent of ``oracle.c``: E2M1 codes are decoded from their bit fields
(1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 is
subnormal), scales are exact powers of two, weights are converted to exact
fractions, the score sum_h w_h * ReLU(q_h . k) is an exact rational, and TopK
is taken by repeated arg-max under the total order of "[FlyDSL][DSv4]
Prototype FP4 MQA streaming TopK", Changes (score descending, index
ascending). Finite inputs only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def e2m1_from_bits(code: int) -> Fraction:
    sign = -1 if (code >> 3) & 1 else 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = Fraction(man, 2)                      # subnormal: 0 or 0.5
    else:
        mag = Fraction(2) ** (exp - 1) * (1 + Fraction(man, 2))
    return sign * mag


def ue8m0_exact(e: int) -> Fraction:
    return Fraction(2) ** (int(e) - 127)


def unpack(vec_bytes) -> list[int]:
    codes = []
    for b in vec_bytes:
        b = int(b)
        codes.append(b & 15)
        codes.append(b >> 4)
    return codes


# twice the E2M1 value of each code, an exact integer
_TWICE = [int(2 * e2m1_from_bits(c)) for c in range(16)]


def _twice_values(vec_bytes) -> np.ndarray:
    return np.array([_TWICE[c] for c in unpack(vec_bytes)], dtype=np.int64)


def head_dot(q_head, q_scale_head, k_vec, k_scale_vec) -> Fraction:
    """Exact dot product: integer block sums of doubled values, then exact scales."""
    qv, kv = _twice_values(q_head), _twice_values(k_vec)
    total = Fraction(0)
    for b in range(4):
        block = int(np.dot(qv[32 * b:32 * b + 32], kv[32 * b:32 * b + 32]))   # = 4 * sum q_j k_j
        total += Fraction(block, 4) * ue8m0_exact(q_scale_head[b]) * ue8m0_exact(k_scale_vec[b])
    return total


def score(q_row, q_scale_row, w_row, k_vec, k_scale_vec) -> Fraction:
    s = Fraction(0)
    for h in range(len(w_row)):
        d = head_dot(q_row[h], q_scale_row[h], k_vec, k_scale_vec)
        s += Fraction(float(w_row[h])) * max(d, Fraction(0))
    return s


def key_vector(inp, pos: int):
    page = int(inp.page_table[pos // 64])
    return inp.k_pages[page, pos % 64], inp.k_scale[page, pos % 64]


def row_scores(inp, row: int) -> list[Fraction]:
    out = []
    for s in range(int(inp.row_start[row]), int(inp.row_end[row])):
        kv, ks = key_vector(inp, s)
        out.append(score(inp.q[row], inp.q_scale[row], inp.weights[row], kv, ks))
    return out


def topk(scores: list[Fraction], start: int, K: int) -> list[int]:
    """Repeated arg-max: highest score first, the smaller index on equal scores."""
    n = len(scores)
    if n <= K:
        return list(range(start, start + n)) + [-1] * (K - n)
    remaining = list(range(n))
    chosen = []
    for _ in range(K):
        best = remaining[0]
        for i in remaining[1:]:
            if scores[i] > scores[best]:
                best = i
        chosen.append(best)
        remaining.remove(best)
    return sorted(start + i for i in chosen)
