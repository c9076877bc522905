"""Binding of the measurement library beside the operator
(``libmqa_fp4_probe.so``, declared in ``include/mqa_fp4_probe.h``): the issue
probe (MXFP4 MFMA waves and fp32 VALU waves per SIMD, timed in shader cycles
per SIMD) and the LDS read probe. Not part of the operator's API; bench.py and
the tests use it to measure the rates the scan kernel is built from."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import PROBE_LIB

FLOP_PER_MFMA = 2 * 32 * 32 * 64      # one v_mfma_scale_f32_32x32x64_f8f6f4
FMA_PER_ITER = 64                     # fp32 FMAs per VALU-wave iteration
MFMA_PER_ITER = 4                     # MFMAs per MFMA-wave iteration

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        try:  # share torch's HIP runtime
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"probe library {PROBE_LIB} is not built; run `python -m fp4_mqa_scoring_amd.build`")
        L = ctypes.CDLL(PROBE_LIB)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        L.mqa_probe_blocks.argtypes = [P]
        L.mqa_probe_issue.argtypes = [i32, i32, i32, P, P, P]
        L.mqa_probe_issue16.argtypes = [i32, i32, i32, P, P, P]
        L.mqa_probe_valu_waves.argtypes = [i32, i32, P, P, P]
        L.mqa_probe_lds.argtypes = [i32, P, i32, i32, P]
        for f in (L.mqa_probe_blocks, L.mqa_probe_issue, L.mqa_probe_issue16, L.mqa_probe_valu_waves,
                  L.mqa_probe_lds):
            f.restype = i32
        _lib = L
    return _lib


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ok(rc, what):
    if rc < 0:
        raise RuntimeError(f"{what} failed with code {rc}")
    return rc


def simd_spans(rec: np.ndarray) -> np.ndarray:
    """Per-SIMD span in shader cycles (latest end - earliest start over the
    waves of one SIMD) from issue-probe records [blocks, waves, 3]."""
    rec = rec.reshape(-1, 3).astype(np.uint64)
    hw = rec[:, 2] & np.uint64(0xFFFFFFFF)
    xcc = (rec[:, 2] >> np.uint64(32)) & np.uint64(0xF)
    simd = (hw >> np.uint64(4)) & np.uint64(3)
    cu = (hw >> np.uint64(8)) & np.uint64(15)
    se = (hw >> np.uint64(13)) & np.uint64(7)
    key = (((xcc * np.uint64(8) + se) * np.uint64(16) + cu) * np.uint64(4) + simd).astype(np.int64)
    order = np.argsort(key, kind="stable")
    k, t0, t1 = key[order], rec[order, 0].astype(np.int64), rec[order, 1].astype(np.int64)
    starts = np.flatnonzero(np.r_[True, k[1:] != k[:-1]])
    lo = np.minimum.reduceat(t0, starts)
    hi = np.maximum.reduceat(t1, starts)
    return (hi - lo).astype(np.float64)


def issue(n_mfma: int, n_valu: int, iters: int, stream=None, shape16: bool = False) -> dict:
    """One issue-probe launch: mean per-SIMD span in cycles and the launch's
    wall time (events on the stream). shape16: the MFMA waves issue 16x16x128
    MFMAs (eight per iteration, the same FLOPs) instead of 32x32x64."""
    import torch
    L = lib()
    fn = L.mqa_probe_issue16 if shape16 else L.mqa_probe_issue
    st = _stream(stream)
    blocks = _ok(L.mqa_probe_blocks(st), "mqa_probe_blocks")
    nw = 4 * (n_mfma + n_valu)
    rec = torch.zeros((blocks, nw, 3), dtype=torch.int64, device="cuda")
    sink = torch.empty(blocks * 64 * nw, dtype=torch.float32, device="cuda")
    args = (n_mfma, n_valu, iters, ctypes.c_void_p(rec.data_ptr()), ctypes.c_void_p(sink.data_ptr()), st)
    _ok(fn(*args), "mqa_probe_issue")                         # warm (clocks, code load)
    s = stream if stream is not None else torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    _ok(fn(*args), "mqa_probe_issue")
    e1.record(s)
    torch.cuda.synchronize()
    spans = simd_spans(rec.cpu().numpy())
    return {"simd_cycles": float(spans.mean()), "simd_cycles_max": float(spans.max()), "simds": int(spans.size),
            "ms": e0.elapsed_time(e1), "blocks": blocks}


def valu_waves(waves_per_simd: int, iters: int = 4096, stream=None) -> float:
    """Cycles per fp32 FMA of one SIMD holding waves_per_simd FMA waves (mean
    per-SIMD span / the SIMD's FMAs), from one launch after a warm one."""
    import torch
    L = lib()
    st = _stream(stream)
    blocks = _ok(L.mqa_probe_blocks(st), "mqa_probe_blocks") * waves_per_simd
    rec = torch.zeros((blocks, 4, 3), dtype=torch.int64, device="cuda")
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    args = (waves_per_simd, iters, ctypes.c_void_p(rec.data_ptr()), ctypes.c_void_p(sink.data_ptr()), st)
    for _ in range(2):
        _ok(L.mqa_probe_valu_waves(*args), "mqa_probe_valu_waves")
    torch.cuda.synchronize()
    spans = simd_spans(rec.cpu().numpy())
    return float(spans.mean()) / (waves_per_simd * iters * FMA_PER_ITER)


def issue_rates(iters: int = 4096, stream=None) -> dict:
    """Cycle rates of one SIMD: MFMAs (one and two MFMA waves), fp32 FMAs (two
    and four VALU waves), and one MFMA wave beside two VALU waves. overlap is
    (alone_sum - together) / min(alone parts): 0 when the two kinds of work
    take the sum of their times, 1 when the shorter one hides entirely."""
    m1 = issue(1, 0, iters, stream)
    m2 = issue(2, 0, iters, stream)
    v2 = issue(0, 2, iters, stream)
    v4 = issue(0, 4, iters, stream)
    mix = issue(1, 2, iters, stream)
    m16 = issue(1, 0, iters, stream, shape16=True)
    mix16 = issue(1, 2, iters, stream, shape16=True)
    n_mfma = iters * MFMA_PER_ITER
    n_fma = iters * FMA_PER_ITER
    alone = m1["simd_cycles"] + v2["simd_cycles"]
    overlap = (alone - mix["simd_cycles"]) / min(m1["simd_cycles"], v2["simd_cycles"])
    blocks = m2["blocks"]
    return {
        "cycles_per_mfma_1wave": m1["simd_cycles"] / n_mfma,
        "cycles_per_mfma_2waves": m2["simd_cycles"] / (2 * n_mfma),
        "cycles_per_fma_2waves": v2["simd_cycles"] / (2 * n_fma),
        "cycles_per_fma_4waves": v4["simd_cycles"] / (4 * n_fma),
        # 1..6 FMA waves per SIMD: how far more resident waves bring the VALU
        # toward one wave64 FMA per 2 cycles
        "cycles_per_fma_by_waves": {k: valu_waves(k, iters, stream) for k in range(1, 7)},
        "mfma_plus_2valu_cycles": mix["simd_cycles"],
        "mfma_alone_plus_2valu_alone_cycles": alone,
        "simd_mfma_valu_overlap": overlap,
        # the same with 16x16x128 MFMAs (cycles per 32x32x64-equivalent, one wave)
        "cycles_per_mfma32_equiv_16x16x128_1wave": m16["simd_cycles"] / n_mfma,
        "mfma16_plus_2valu_cycles": mix16["simd_cycles"],
        "simd_mfma16_valu_overlap": (m16["simd_cycles"] + v2["simd_cycles"] - mix16["simd_cycles"]) /
                                    min(m16["simd_cycles"], v2["simd_cycles"]),
        # sustained MXFP4 rate of the two-wave MFMA launch (wall time by events)
        "mxfp4_tflops_measured": blocks * 4 * 2 * n_mfma * FLOP_PER_MFMA / (m2["ms"] * 1e-3) / 1e12,
    }


def lds_ms(pattern: int, blocks: int = 2048, iters: int = 2000, stream=None) -> float:
    """Mean wall time of an LDS read-probe launch (five timed, after two)."""
    import torch
    L = lib()
    st = _stream(stream)
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    for _ in range(2):
        _ok(L.mqa_probe_lds(pattern, ctypes.c_void_p(out.data_ptr()), blocks, iters, st), "mqa_probe_lds")
    s = stream if stream is not None else torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(5):
        _ok(L.mqa_probe_lds(pattern, ctypes.c_void_p(out.data_ptr()), blocks, iters, st), "mqa_probe_lds")
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 5
