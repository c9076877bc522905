"""MI355X-native FP4 paged-MQA prefill indexer fused with exact TopK.

Thin Python binding of the C ABI in ``include/mqa_fp4_topk.h``: every entry
point below marshals torch tensors (device memory, streams) into pointers and
sizes and calls the HIP library ``libmqa_fp4.so``; all arithmetic runs in the
library's kernels. The library is built in-tree by ``build.build()``; calling
an entry point without it raises.
"""
from __future__ import annotations

import ctypes
import os

from . import synth  # noqa: F401  (seeded input generator)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmqa_fp4.so")

MQA_OK = 0
ERRORS = {
    -1: "MQA_ERR_UNSUPPORTED_K", -2: "MQA_ERR_NULL_POINTER", -3: "MQA_ERR_MISALIGNED",
    -4: "MQA_ERR_BAD_SIZE", -5: "MQA_ERR_DEVICE", -6: "MQA_ERR_CAPTURING", -7: "MQA_ERR_HIP",
    -8: "MQA_ERR_BAD_FLAGS",
}
ROW_BAD_WINDOW, ROW_BAD_PAGE, ROW_UNDERFILL, ROW_SELECTOR = -1, -2, -3, -4
STATUS_BAD_WINDOW, STATUS_BAD_PAGE, STATUS_UNDERFILL, STATUS_SELECTOR = 1, 2, 4, 8
FLAG_SPLITS_MASK = 0xFF
FLAG_NO_PREFILTER = 0x100
FLAG_FORCE_UNDERFILL = 0x200
FLAG_NO_FALLBACK = 0x400
STATIC_SCRATCH_BYTES = 64 << 20          # MQA_STATIC_SCRATCH_BYTES


class MQAError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({_error_string(code)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        try:  # share torch's HIP runtime (same SONAME) so torch streams and memory are valid here
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run "
                               "`python -m fp4_mqa_scoring_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        prefill = [P, P, i64, P, P, i64, P, P, i64, P, P, i32, P, P, P]
        L.mqa_fp4_topk_prefill.argtypes = prefill + [P]
        L.mqa_fp4_topk_prefill_ex.argtypes = prefill + [P, u32, P]
        L.mqa_fp4_topk_prefill_static.argtypes = prefill + [P, u32, P]
        L.mqa_fp4_dense_topk_prefill.argtypes = [P, P, i64, P, P, i64, P, P, i64, P, P, i32, P, P, P, P, P, P]
        L.mqa_fp4_dense_logits.argtypes = [P, P, i64, P, P, i64, P, P, i64, P, P, P, P]
        L.mqa_fp4_logits_topk.argtypes = [P, i64, P, i64, i64, P, P, i32, P, P, P, P, P]
        L.mqa_fp4_supported_k.argtypes = [P, i32, P]
        L.mqa_fp4_topk_scratch_bytes.argtypes = [i64, i32, i32]
        L.mqa_fp4_topk_scratch_bytes.restype = i64
        L.mqa_fp4_status.argtypes = [P, P]
        L.mqa_fp4_error_string.argtypes = [i32]
        L.mqa_fp4_error_string.restype = ctypes.c_char_p
        L.mqa_fp4_abi_version.argtypes = []
        L.mqa_fp4_set_stage_events.argtypes = [P, i32]
        L.mqa_fp4_quantize.argtypes = [P, i64, P, P, P]
        L.mqa_fp4_tiled_topk_prefill.argtypes = prefill[:11] + [i32, i32, P, P, P, P, P]
        L.mqa_fp4_tiled_scratch_bytes.argtypes = [i64, i32, i32]
        L.mqa_fp4_tiled_scratch_bytes.restype = i64
        L.mqa_fp4_topk_decode.argtypes = [P, P, i64, P, P, i64, P, P, i64, i64, P, P, P, i32, P, P, P, P, P, i64,
                                          i32, u32, P]
        L.mqa_fp4_decode_workspace_bytes.argtypes = [i64, i32, i32, i32]
        L.mqa_fp4_decode_workspace_bytes.restype = i64
        L.mqa_fp4_cache_write.argtypes = [P, i64, P, P, i64, i64, P, P, P]
        for name in ("mqa_fp4_topk_prefill", "mqa_fp4_topk_prefill_ex", "mqa_fp4_topk_prefill_static",
                     "mqa_fp4_dense_topk_prefill",
                     "mqa_fp4_dense_logits", "mqa_fp4_logits_topk", "mqa_fp4_supported_k",
                     "mqa_fp4_status", "mqa_fp4_abi_version", "mqa_fp4_set_stage_events",
                     "mqa_fp4_quantize", "mqa_fp4_cache_write",
                     "mqa_fp4_tiled_topk_prefill", "mqa_fp4_topk_decode"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _error_string(code: int) -> str:
    try:
        return lib().mqa_fp4_error_string(int(code)).decode()
    except Exception:  # library missing
        return ""


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(t, name, dtype, ndim=None):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _check_inputs(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end):
    import torch
    _check(q, "q", torch.uint8, 3)
    _check(q_scale, "q_scale", torch.uint8, 3)
    _check(k_pages, "k_pages", torch.uint8, 3)
    _check(k_scale, "k_scale", torch.uint8, 3)
    _check(weights, "weights", torch.float32, 2)
    _check(page_table, "page_table", torch.int32, 1)
    _check(row_start, "row_start", torch.int32, 1)
    _check(row_end, "row_end", torch.int32, 1)
    Q = q.shape[0]
    if tuple(q.shape[1:]) != (64, 64) or tuple(q_scale.shape) != (Q, 64, 4):
        raise ValueError("q must be [Q,64,64] and q_scale [Q,64,4]")
    if tuple(k_pages.shape[1:]) != (64, 64) or tuple(k_scale.shape) != (k_pages.shape[0], 64, 4):
        raise ValueError("k_pages must be [P,64,64] and k_scale [P,64,4]")
    if tuple(weights.shape) != (Q, 64) or row_start.shape[0] != Q or row_end.shape[0] != Q:
        raise ValueError("weights must be [Q,64]; row_start/row_end [Q]")
    return Q, k_pages.shape[0], page_table.shape[0]


def _check_outputs(Q, K, out_raw, out_slot, out_count, out_score):
    import torch
    _check(out_raw, "out_raw", torch.int32, 2)
    _check(out_slot, "out_slot", torch.int32, 2)
    _check(out_count, "out_count", torch.int32, 1)
    _check(out_score, "out_score", torch.float32, 2)
    for t, n in ((out_raw, "out_raw"), (out_slot, "out_slot"), (out_score, "out_score")):
        if t is not None and tuple(t.shape) != (Q, K):
            raise ValueError(f"{n} must be [Q, K] = [{Q}, {K}]")
    if out_count.shape[0] != Q:
        raise ValueError("out_count must be [Q]")


def _rc(code, what):
    if code != MQA_OK:
        raise MQAError(code, what)


def alloc_outputs(Q: int, K: int, device, with_score: bool = False):
    """Output buffers (out_raw, out_slot, out_count[, out_score]) on ``device``."""
    import torch
    out = [torch.empty((Q, K), dtype=torch.int32, device=device),
           torch.empty((Q, K), dtype=torch.int32, device=device),
           torch.empty((Q,), dtype=torch.int32, device=device)]
    if with_score:
        out.append(torch.empty((Q, K), dtype=torch.float32, device=device))
    return tuple(out)


def mqa_fp4_topk_prefill(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end, K,
                         out_raw, out_slot, out_count, stream=None):
    """Fused FP4 indexer scoring + exact TopK + page mapping (see the C header)."""
    return mqa_fp4_topk_prefill_ex(q, q_scale, k_pages, k_scale, weights, page_table, row_start,
                                   row_end, K, out_raw, out_slot, out_count, None, 0, stream)


def mqa_fp4_topk_prefill_ex(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end, K,
                            out_raw, out_slot, out_count, out_score=None, flags=0, stream=None):
    Q, P_phys, P_log = _check_inputs(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end)
    _check_outputs(Q, K, out_raw, out_slot, out_count, out_score)
    rc = lib().mqa_fp4_topk_prefill_ex(
        _ptr(q), _ptr(q_scale), Q, _ptr(k_pages), _ptr(k_scale), P_phys, _ptr(weights),
        _ptr(page_table), P_log, _ptr(row_start), _ptr(row_end), int(K), _ptr(out_raw), _ptr(out_slot),
        _ptr(out_count), _ptr(out_score), int(flags), _stream(stream, q.device))
    _rc(rc, "mqa_fp4_topk_prefill_ex")


def mqa_fp4_topk_prefill_static(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end, K,
                                out_raw, out_slot, out_count, out_score=None, flags=0, stream=None):
    """Allocation-free form of mqa_fp4_topk_prefill_ex: scratch from the library's
    fixed per-device array (STATIC_SCRATCH_BYTES), so the batch is limited to
    1,636 rows at K = 1024 and 2,045 at K = 512; calls on one device must be
    ordered (they share the array). Accepts a capturing stream."""
    Q, P_phys, P_log = _check_inputs(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end)
    _check_outputs(Q, K, out_raw, out_slot, out_count, out_score)
    rc = lib().mqa_fp4_topk_prefill_static(
        _ptr(q), _ptr(q_scale), Q, _ptr(k_pages), _ptr(k_scale), P_phys, _ptr(weights),
        _ptr(page_table), P_log, _ptr(row_start), _ptr(row_end), int(K), _ptr(out_raw), _ptr(out_slot),
        _ptr(out_count), _ptr(out_score), int(flags), _stream(stream, q.device))
    _rc(rc, "mqa_fp4_topk_prefill_static")


def mqa_fp4_dense_topk_prefill(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end, K,
                               logits, out_raw, out_slot, out_count, out_score=None, stream=None):
    """Dense comparator: fp32 logits [Q, S] (caller-owned), then exact TopK."""
    import torch
    Q, P_phys, P_log = _check_inputs(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end)
    _check_outputs(Q, K, out_raw, out_slot, out_count, out_score)
    _check(logits, "logits", torch.float32, 2)
    if tuple(logits.shape) != (Q, 64 * P_log):
        raise ValueError("logits must be [Q, 64 * P_log]")
    rc = lib().mqa_fp4_dense_topk_prefill(
        _ptr(q), _ptr(q_scale), Q, _ptr(k_pages), _ptr(k_scale), P_phys, _ptr(weights),
        _ptr(page_table), P_log, _ptr(row_start), _ptr(row_end), int(K), _ptr(logits), _ptr(out_raw),
        _ptr(out_slot), _ptr(out_count), _ptr(out_score), _stream(stream, q.device))
    _rc(rc, "mqa_fp4_dense_topk_prefill")


def mqa_fp4_tiled_topk_prefill(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end, K,
                               out_raw, out_slot, out_count, out_score=None, tile_positions=0, stream=None):
    """Bounded context-tiled exact TopK (same contract and outputs as the fused path)."""
    Q, P_phys, P_log = _check_inputs(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end)
    _check_outputs(Q, K, out_raw, out_slot, out_count, out_score)
    rc = lib().mqa_fp4_tiled_topk_prefill(
        _ptr(q), _ptr(q_scale), Q, _ptr(k_pages), _ptr(k_scale), P_phys, _ptr(weights),
        _ptr(page_table), P_log, _ptr(row_start), _ptr(row_end), int(K), int(tile_positions), _ptr(out_raw),
        _ptr(out_slot), _ptr(out_count), _ptr(out_score), _stream(stream, q.device))
    _rc(rc, "mqa_fp4_tiled_topk_prefill")


def mqa_fp4_tiled_scratch_bytes(num_rows: int, K: int, tile_positions: int = 0) -> int:
    r = int(lib().mqa_fp4_tiled_scratch_bytes(int(num_rows), int(K), int(tile_positions)))
    if r < 0:
        raise MQAError(r, "mqa_fp4_tiled_scratch_bytes")
    return r


def mqa_fp4_decode_workspace_bytes(num_rows: int, K: int, splits: int = 0, device: int = 0) -> int:
    r = int(lib().mqa_fp4_decode_workspace_bytes(int(num_rows), int(K), int(splits), int(device)))
    if r < 0:
        raise MQAError(r, "mqa_fp4_decode_workspace_bytes")
    return r


def mqa_fp4_topk_decode(q, q_scale, k_pages, k_scale, weights, block_table, seq_of_row, row_start, row_end, K,
                        out_raw, out_slot, out_count, workspace, out_score=None, splits=0, flags=0, stream=None):
    """Decode / multi-sequence form: block_table int32 [n_seq, max_pages], seq_of_row int32 [Q],
    workspace a uint8 device tensor of at least mqa_fp4_decode_workspace_bytes(Q, K, splits) bytes.
    Allocates nothing and does not synchronise (capturable)."""
    import torch
    _check(q, "q", torch.uint8, 3)
    _check(q_scale, "q_scale", torch.uint8, 3)
    _check(k_pages, "k_pages", torch.uint8, 3)
    _check(k_scale, "k_scale", torch.uint8, 3)
    _check(weights, "weights", torch.float32, 2)
    _check(block_table, "block_table", torch.int32, 2)
    for t, n in ((seq_of_row, "seq_of_row"), (row_start, "row_start"), (row_end, "row_end")):
        _check(t, n, torch.int32, 1)
    _check(workspace, "workspace", torch.uint8)
    Q = q.shape[0]
    _check_outputs(Q, K, out_raw, out_slot, out_count, out_score)
    rc = lib().mqa_fp4_topk_decode(
        _ptr(q), _ptr(q_scale), Q, _ptr(k_pages), _ptr(k_scale), k_pages.shape[0], _ptr(weights),
        _ptr(block_table), block_table.shape[0], block_table.shape[1], _ptr(seq_of_row), _ptr(row_start),
        _ptr(row_end), int(K), _ptr(out_raw), _ptr(out_slot), _ptr(out_count), _ptr(out_score), _ptr(workspace),
        workspace.numel(), int(splits), int(flags), _stream(stream, q.device))
    _rc(rc, "mqa_fp4_topk_decode")


def mqa_fp4_dense_logits(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end, logits,
                         stream=None):
    import torch
    Q, P_phys, P_log = _check_inputs(q, q_scale, k_pages, k_scale, weights, page_table, row_start, row_end)
    _check(logits, "logits", torch.float32, 2)
    if tuple(logits.shape) != (Q, 64 * P_log):
        raise ValueError("logits must be [Q, 64 * P_log]")
    rc = lib().mqa_fp4_dense_logits(
        _ptr(q), _ptr(q_scale), Q, _ptr(k_pages), _ptr(k_scale), P_phys, _ptr(weights),
        _ptr(page_table), P_log, _ptr(row_start), _ptr(row_end), _ptr(logits), _stream(stream, q.device))
    _rc(rc, "mqa_fp4_dense_logits")


def mqa_fp4_logits_topk(logits, page_table, num_phys_pages, row_start, row_end, K, out_raw, out_slot,
                        out_count, out_score=None, stream=None):
    """Exact TopK over caller-provided fp32 logits [Q, 64 * P_log]."""
    import torch
    _check(logits, "logits", torch.float32, 2)
    _check(page_table, "page_table", torch.int32, 1)
    _check(row_start, "row_start", torch.int32, 1)
    _check(row_end, "row_end", torch.int32, 1)
    Q, P_log = logits.shape[0], page_table.shape[0]
    if logits.shape[1] != 64 * P_log:
        raise ValueError("logits must be [Q, 64 * P_log]")
    _check_outputs(Q, K, out_raw, out_slot, out_count, out_score)
    rc = lib().mqa_fp4_logits_topk(
        _ptr(logits), Q, _ptr(page_table), P_log, int(num_phys_pages), _ptr(row_start), _ptr(row_end),
        int(K), _ptr(out_raw), _ptr(out_slot), _ptr(out_count), _ptr(out_score),
        _stream(stream, logits.device))
    _rc(rc, "mqa_fp4_logits_topk")


def mqa_fp4_supported_k():
    buf = (ctypes.c_int32 * 8)()
    n = ctypes.c_int32(0)
    _rc(lib().mqa_fp4_supported_k(buf, 8, ctypes.byref(n)), "mqa_fp4_supported_k")
    return [int(buf[i]) for i in range(n.value)]


def mqa_fp4_topk_scratch_bytes(num_rows: int, K: int, device: int = 0) -> int:
    r = int(lib().mqa_fp4_topk_scratch_bytes(int(num_rows), int(K), int(device)))
    if r < 0:
        raise MQAError(r, "mqa_fp4_topk_scratch_bytes")
    return r


def mqa_fp4_status(stream=None, device=None) -> int:
    """Synchronises the stream, returns and clears the sticky status bits."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    st = ctypes.c_int32(0)
    _rc(lib().mqa_fp4_status(_stream(stream, dev), ctypes.byref(st)), "mqa_fp4_status")
    return int(st.value)


def mqa_fp4_abi_version() -> int:
    return int(lib().mqa_fp4_abi_version())


def mqa_fp4_quantize(x, codes=None, scales=None, stream=None):
    """MXFP4 quantisation (OCP MX conversion, E2M1 + UE8M0) of float32 x [..., 128]
    into codes uint8 [..., 64] and scales uint8 [..., 4] (allocated if None)."""
    import torch
    _check(x, "x", torch.float32)
    if x.shape[-1] != 128:
        raise ValueError("x must end in 128 elements")
    lead = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (64,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(lead + (4,), dtype=torch.uint8, device=x.device)
    _check(codes, "codes", torch.uint8)
    _check(scales, "scales", torch.uint8)
    n = x.numel() // 128
    if codes.numel() != n * 64 or scales.numel() != n * 4:
        raise ValueError("codes / scales do not match x")
    _rc(lib().mqa_fp4_quantize(_ptr(x), n, _ptr(codes), _ptr(scales), _stream(stream, x.device)),
        "mqa_fp4_quantize")
    return codes, scales


def mqa_fp4_cache_write(k, positions, page_table, k_pages, k_scale, stream=None) -> None:
    """Quantise float32 keys k [n, 128] into the paged C4 cache at logical
    positions (int32 [n]) through page_table (int32 [P_log])."""
    import torch
    _check(k, "k", torch.float32)
    _check(positions, "positions", torch.int32)
    _check(page_table, "page_table", torch.int32)
    _check(k_pages, "k_pages", torch.uint8)
    _check(k_scale, "k_scale", torch.uint8)
    n = k.numel() // 128
    if positions.numel() != n:
        raise ValueError("positions must have one entry per key vector")
    _rc(lib().mqa_fp4_cache_write(_ptr(k), n, _ptr(positions), _ptr(page_table), page_table.numel(),
                                  k_pages.shape[0], _ptr(k_pages), _ptr(k_scale), _stream(stream, k.device)),
        "mqa_fp4_cache_write")


def mqa_fp4_set_stage_events(events) -> None:
    """Measurement hook: ``events`` is a ctypes array of 5 hipEvent_t handles
    (or None to turn the hook off); see the C header."""
    if events is None:
        _rc(lib().mqa_fp4_set_stage_events(None, 0), "mqa_fp4_set_stage_events")
    else:
        _rc(lib().mqa_fp4_set_stage_events(ctypes.cast(events, ctypes.c_void_p), len(events)),
            "mqa_fp4_set_stage_events")
