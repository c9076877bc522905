"""CPU oracle for the FP4 paged-MQA prefill indexer with exact TopK.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library and
its Python binding never import, link or call it.

The arithmetic lives in ``oracle.c`` (plain C, float64, OpenMP over
positions); this module builds it with gcc and wraps it with ctypes. The
exact-rational brute force in ``brute.py`` pins it on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a test may point the wrapper at a deliberately broken build of oracle.c
_LOAD = os.environ.get("MQA_ORACLE_LIB", _LIB)

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2 -fopenmp)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if _LOAD == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LOAD)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_ue8m0_value.restype = ctypes.c_double
        L.oracle_ue8m0_value.argtypes = [ctypes.c_int]
        L.oracle_head_dot.restype = ctypes.c_double
        L.oracle_head_dot.argtypes = [P, P, P, P]
        L.oracle_validate_row.restype = ctypes.c_int
        L.oracle_validate_row.argtypes = [i64, i64, P, i64, i64]
        L.oracle_row_scores.restype = ctypes.c_int
        L.oracle_row_scores.argtypes = [P, P, P, P, P, i64, P, i64, i64, i64, P, P, ctypes.c_int]
        L.oracle_ranks_before.restype = ctypes.c_int
        L.oracle_ranks_before.argtypes = [ctypes.c_double, i64, ctypes.c_double, i64]
        L.oracle_select_topk.restype = i64
        L.oracle_select_topk.argtypes = [P, i64, i64, i64, P]
        L.oracle_slot.restype = i64
        L.oracle_slot.argtypes = [i64, P]
        L.oracle_topk_row.restype = i64
        L.oracle_topk_row.argtypes = [P, P, P, P, P, i64, P, i64, P, P, i64, i64, P, P, P,
                                      ctypes.c_int]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_e2m1_encode.restype = ctypes.c_int
        L.oracle_e2m1_encode.argtypes = [ctypes.c_double]
        L.oracle_mx_scale_byte.restype = ctypes.c_int
        L.oracle_mx_scale_byte.argtypes = [P]
        L.oracle_mx_quantize.restype = None
        L.oracle_mx_quantize.argtypes = [P, i64, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def e2m1_value(code: int) -> float:
    return float(lib().oracle_e2m1_value(int(code)))


def ue8m0_value(e: int) -> float:
    return float(lib().oracle_ue8m0_value(int(e)))


def head_dot(q_head, q_scale_head, k_vec, k_scale_vec) -> float:
    arrs = [np.ascontiguousarray(x, dtype=np.uint8) for x in (q_head, q_scale_head, k_vec, k_scale_vec)]
    return float(lib().oracle_head_dot(*[_p(a) for a in arrs]))


def validate_row(inp, row: int) -> int:
    return int(lib().oracle_validate_row(int(inp.row_start[row]), int(inp.row_end[row]),
                                         _p(inp.page_table), inp.P_log, inp.P_phys))


def row_scores(inp, row: int, p0: int | None = None, p1: int | None = None, nthreads: int = 0):
    """float64 scores and magnitudes sum_h |w_h| ReLU(d_h) of ``row`` over
    logical positions [p0, p1) (default: the row's window)."""
    p0 = int(inp.row_start[row]) if p0 is None else int(p0)
    p1 = int(inp.row_end[row]) if p1 is None else int(p1)
    n = max(0, p1 - p0)
    s = np.empty(n, np.float64)
    m = np.empty(n, np.float64)
    if n:
        rc = lib().oracle_row_scores(_p(inp.q[row]), _p(inp.q_scale[row]), _p(inp.weights[row]),
                                     _p(inp.k_pages), _p(inp.k_scale), inp.P_phys,
                                     _p(inp.page_table), inp.P_log, p0, p1, _p(s), _p(m),
                                     int(nthreads))
        if rc != 0:
            raise ValueError("invalid page in range")
    return s, m


def ranks_before(sa: float, ia: int, sb: float, ib: int) -> bool:
    return bool(lib().oracle_ranks_before(float(sa), int(ia), float(sb), int(ib)))


def select_topk(scores, start: int, K: int):
    """Exact TopK of a score array for positions start..start+n-1."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    out = np.empty(K, np.int32)
    cnt = lib().oracle_select_topk(_p(s), s.shape[0], int(start), int(K), _p(out))
    return int(cnt), out


def slot(raw: int, page_table) -> int:
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    return int(lib().oracle_slot(int(raw), _p(pt)))


def topk_row(inp, row: int, K: int | None = None, nthreads: int = 0):
    """The whole operator for one row: (count, raw[K], slot[K], sel_score[K])."""
    K = inp.K if K is None else int(K)
    raw = np.empty(K, np.int32)
    sl = np.empty(K, np.int32)
    sc = np.empty(K, np.float64)
    cnt = lib().oracle_topk_row(_p(inp.q), _p(inp.q_scale), _p(inp.weights), _p(inp.k_pages),
                                _p(inp.k_scale), inp.P_phys, _p(inp.page_table), inp.P_log,
                                _p(inp.row_start), _p(inp.row_end), int(row), K,
                                _p(raw), _p(sl), _p(sc), int(nthreads))
    return int(cnt), raw, sl, sc


def topk_rows(inp, rows, K: int | None = None, nthreads: int = 0):
    K = inp.K if K is None else int(K)
    rows = list(rows)
    cnt = np.empty(len(rows), np.int64)
    raw = np.empty((len(rows), K), np.int32)
    sl = np.empty((len(rows), K), np.int32)
    sc = np.empty((len(rows), K), np.float64)
    for i, r in enumerate(rows):
        cnt[i], raw[i], sl[i], sc[i] = topk_row(inp, r, K, nthreads)
    return cnt, raw, sl, sc


# --- MXFP4 quantisation (OCP MX conversion; see oracle.c) ------------------------

def e2m1_encode(v: float) -> int:
    return int(lib().oracle_e2m1_encode(float(v)))


def mx_quantize(x):
    """float32 [..., 128*k or 32*k] -> (codes uint8 [..., 16*k], scales uint8 [..., k]) per
    32-element block: OCP MX conversion with E2M1 elements and UE8M0 scales."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % 32 == 0
    nb = x.size // 32
    codes = np.empty(nb * 16, np.uint8)
    scales = np.empty(nb, np.uint8)
    if nb:
        lib().oracle_mx_quantize(_p(x), nb, _p(codes), _p(scales))
    lead = x.shape[:-1]
    k = x.shape[-1] // 32
    return codes.reshape(*lead, 16 * k), scales.reshape(*lead, k)


def mx_dequantize(codes, scales):
    """Inverse view for tests: E2M1 codes and UE8M0 scales -> float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = (codes & 15).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    el = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    table = np.array([e2m1_value(c) for c in range(16)])
    vals = table[el]
    sc = np.array([ue8m0_value(e) for e in range(256)])[scales.astype(np.int64)]
    k = scales.shape[-1]
    return (vals.reshape(*vals.shape[:-1], k, 32) * sc[..., None]).reshape(vals.shape)
