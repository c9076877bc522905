"""CPU checks of the C ABI: the HIP library loads, exports every symbol the
public header declares, and rejects bad arguments on the host before any HIP
call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa_fp4_topk.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(mqa_fp4_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    import fp4_mqa_scoring_amd as m
    override = os.environ.get("MQA_ABI_TEST_LIB")   # a sanitizer build of the same sources
    if override:                                     # (tests/test_host_sanitizers.py)
        m.LIB_PATH = override
    elif not os.path.exists(m.LIB_PATH):
        from fp4_mqa_scoring_amd import build
        build.build()
    return m.lib()


def test_header_declares_the_operator_api():
    syms = declared_symbols()
    for name in ("mqa_fp4_topk_prefill", "mqa_fp4_topk_prefill_ex", "mqa_fp4_dense_topk_prefill",
                 "mqa_fp4_logits_topk", "mqa_fp4_supported_k", "mqa_fp4_topk_scratch_bytes",
                 "mqa_fp4_status"):
        assert name in syms


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_capability_probe_and_version(lib):
    import fp4_mqa_scoring_amd as m
    assert m.mqa_fp4_supported_k() == [512, 1024]
    assert m.mqa_fp4_abi_version() == 1
    assert b"unsupported K" in lib.mqa_fp4_error_string(-1)


def _call_prefill(lib, K=512, Q=4, P_phys=2, P_log=2, flags=0, ptr=0x1000, **over):
    args = dict(q=ptr, q_scale=ptr, k_pages=ptr, k_scale=ptr, weights=ptr, page_table=ptr,
                row_start=ptr, row_end=ptr, out_raw=ptr, out_slot=ptr, out_count=ptr, out_score=None)
    args.update(over)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mqa_fp4_topk_prefill_ex(v(args["q"]), v(args["q_scale"]), Q, v(args["k_pages"]),
                                       v(args["k_scale"]), P_phys, v(args["weights"]),
                                       v(args["page_table"]), P_log, v(args["row_start"]),
                                       v(args["row_end"]), K, v(args["out_raw"]), v(args["out_slot"]),
                                       v(args["out_count"]), v(args["out_score"]), flags, None)


@pytest.mark.parametrize("K", [0, 1, 256, 511, 513, 768, 2048, -512])
def test_unsupported_k_rejected_before_any_device_work(lib, K):
    assert _call_prefill(lib, K=K) == -1


def test_bad_flags_sizes_nulls_alignment_rejected_on_host(lib):
    assert _call_prefill(lib, flags=0x800) == -8                # unknown bit
    assert _call_prefill(lib, flags=0x300) == -8                # no prefilter + forced underfill
    assert _call_prefill(lib, flags=0x500) == -8                # no prefilter + no fallback
    assert _call_prefill(lib, Q=-1) == -4
    assert _call_prefill(lib, P_log=(1 << 31) // 64) == -4
    assert _call_prefill(lib, P_phys=(1 << 31) // 64 + 1) == -4
    assert _call_prefill(lib, q=None) == -2
    assert _call_prefill(lib, out_count=None) == -2
    assert _call_prefill(lib, k_pages=0x1008) == -3          # needs 16-byte alignment
    assert _call_prefill(lib, row_end=0x1002) == -3


def test_dense_and_logits_entry_points_check_k_on_host(lib):
    P = ctypes.c_void_p
    p = P(0x1000)
    assert lib.mqa_fp4_dense_topk_prefill(p, p, 1, p, p, 1, p, p, 1, p, p, 7, p, p, p, p, None, None) == -1
    assert lib.mqa_fp4_logits_topk(p, 1, p, 1, 1, p, p, 100, p, p, p, None, None) == -1


def test_stage_event_hook_takes_exactly_five_events(lib):
    # The hook only stores the array (no HIP call): five handles are accepted,
    # other counts are rejected, NULL / zero turns it off.
    arr5 = (ctypes.c_void_p * 5)()
    arr4 = (ctypes.c_void_p * 4)()
    assert lib.mqa_fp4_set_stage_events(ctypes.cast(arr4, ctypes.c_void_p), 4) == -4
    assert lib.mqa_fp4_set_stage_events(ctypes.cast(arr5, ctypes.c_void_p), 5) == 0
    assert lib.mqa_fp4_set_stage_events(None, 0) == 0


PROBE_HEADER = os.path.join(ROOT, "include", "mqa_fp4_probe.h")


@pytest.fixture(scope="module")
def probe_lib():
    from fp4_mqa_scoring_amd import build, probe
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    return probe.lib()


def test_probes_live_in_their_own_library(lib, probe_lib):
    """The measurement probes are not part of the operator's ABI: the operator
    header declares none and its library exports none; the probe header's
    symbols are all exported by the probe library."""
    probe_syms = sorted(set(re.findall(r"^\s*int32_t\s+(mqa_probe_\w+)\s*\(", open(PROBE_HEADER).read(), re.M)))
    assert probe_syms == ["mqa_probe_blocks", "mqa_probe_issue", "mqa_probe_issue16", "mqa_probe_lds",
                          "mqa_probe_valu_waves"]
    for name in probe_syms:
        assert hasattr(probe_lib, name), name
        assert not hasattr(lib, name), name
    assert not hasattr(lib, "mqa_fp4_peak_probe")
    assert not any("probe" in s for s in declared_symbols())


def test_probes_reject_bad_arguments_on_host(probe_lib):
    p = ctypes.c_void_p(0x1000)
    L = probe_lib
    assert L.mqa_probe_issue(0, 0, 8, p, p, None) == -4          # no waves
    assert L.mqa_probe_issue(3, 2, 8, p, p, None) == -4          # more than four waves per SIMD
    assert L.mqa_probe_issue(-1, 2, 8, p, p, None) == -4
    assert L.mqa_probe_issue(1, 1, 0, p, p, None) == -4          # no iterations
    assert L.mqa_probe_issue(1, 1, 8, None, p, None) == -2
    assert L.mqa_probe_issue(1, 1, 8, ctypes.c_void_p(0x1004), p, None) == -3
    assert L.mqa_probe_issue16(3, 2, 8, p, p, None) == -4        # more than four waves per SIMD
    assert L.mqa_probe_issue16(1, 1, 8, None, p, None) == -2
    assert L.mqa_probe_valu_waves(0, 8, p, p, None) == -4         # no waves
    assert L.mqa_probe_valu_waves(7, 8, p, p, None) == -4         # more than six per SIMD
    assert L.mqa_probe_valu_waves(2, 0, p, p, None) == -4         # no iterations
    assert L.mqa_probe_valu_waves(2, 8, p, None, None) == -2
    assert L.mqa_probe_valu_waves(2, 8, ctypes.c_void_p(0x1004), p, None) == -3
    assert L.mqa_probe_lds(3, p, 1, 1, None) == -4               # unknown pattern
    assert L.mqa_probe_lds(0, p, 0, 1, None) == -4               # no blocks
    assert L.mqa_probe_lds(0, None, 1, 1, None) == -2
    assert L.mqa_probe_lds(0, ctypes.c_void_p(0x1002), 1, 1, None) == -3


def test_quantizer_and_cache_writer_reject_bad_arguments_on_host(lib):
    P = ctypes.c_void_p
    a = P(0x1000)
    assert lib.mqa_fp4_quantize(a, -1, a, a, None) == -4
    assert lib.mqa_fp4_quantize(None, 4, a, a, None) == -2
    assert lib.mqa_fp4_quantize(a, 4, None, a, None) == -2
    assert lib.mqa_fp4_quantize(P(0x1004), 4, a, a, None) == -3        # x needs 16-byte alignment
    assert lib.mqa_fp4_quantize(a, 4, P(0x1001), a, None) == -3        # codes need 2-byte alignment
    assert lib.mqa_fp4_cache_write(a, -1, a, a, 1, 1, a, a, None) == -4
    assert lib.mqa_fp4_cache_write(a, 4, a, a, -1, 1, a, a, None) == -4
    assert lib.mqa_fp4_cache_write(a, 4, None, a, 1, 1, a, a, None) == -2
    assert lib.mqa_fp4_cache_write(a, 4, a, a, 1, 1, P(0x1008), a, None) == -3


def test_tiled_path_checks_tile_and_k_on_host(lib):
    import fp4_mqa_scoring_amd as m
    P = ctypes.c_void_p
    p = P(0x1000)
    args = (p, p, 2, p, p, 2, p, p, 2, p, p)
    assert lib.mqa_fp4_tiled_topk_prefill(*args, 512, 300, p, p, p, None, None) == -4     # not a multiple of 256
    assert lib.mqa_fp4_tiled_topk_prefill(*args, 512, -256, p, p, p, None, None) == -4
    assert lib.mqa_fp4_tiled_topk_prefill(*args, 640, 256, p, p, p, None, None) == -1     # unsupported K
    # scratch: O(Q) + Q*2K*8 (the pool) + Q*tile*4, no context argument at all
    q, K, T = 1000, 1024, 4096
    a = lambda x: (x + 255) // 256 * 256
    want = 2 * a(q * 4) + a(q * 8) + a(q * 2 * K * 8) + a(q * T * 4)
    assert m.mqa_fp4_tiled_scratch_bytes(q, K, T) == want
    assert m.mqa_fp4_tiled_scratch_bytes(q, K, 0) == want      # 0 = the 4096 default


def test_decode_entry_checks_arguments_on_host(lib):
    import fp4_mqa_scoring_amd as m
    P = ctypes.c_void_p
    p = P(0x1000)

    def call(K=512, splits=0, ws=p, ws_bytes=1 << 20, flags=0):
        return lib.mqa_fp4_topk_decode(p, p, 2, p, p, 4, p, p, 2, 4, p, p, p, K, p, p, p, None, ws, ws_bytes,
                                       splits, flags, None)
    assert call(K=100) == -1
    assert call(flags=0x3) == -8                     # split bits belong to the splits argument
    assert call(flags=0x300) == -8                   # no prefilter + forced underfill
    assert call(flags=0x500) == -8                   # no prefilter + no fallback
    assert call(flags=0x800) == -8                   # unknown bit
    assert call(splits=65) == -4
    assert call(splits=-1) == -4
    assert call(ws_bytes=-1) == -4
    assert call(ws=None) == -2
    assert call(ws=P(0x1010)) == -3                  # workspace needs 256-byte alignment
    # explicit splits: no device query; O(Q) + Q*splits*(4 + 8K) bytes, the scan plan (Q + 1) * 8, and the
    # gated scan's per-wave candidate regions (3072 waves x (512 + 16) keys), counts and descriptors
    q, K, s = 100, 1024, 5
    a = lambda x: (x + 255) // 256 * 256
    cap = 4096                                       # candidate keys per row at K = 1024
    waves = 3072
    want = (a(q * 4) + a(q * s * 4) + a(q * s * K * 8) + a(q * 8) + a(q * 4) + a(q * cap * 8) + a(q * 4)
            + a(4) + a((q + 1) * 8) + a(waves * 528 * 8) + a(waves * 4) + 4 * a(q * 4) + a(waves * 3 * 8))
    assert m.mqa_fp4_decode_workspace_bytes(q, K, s) == want


def test_allocation_free_entry_point_checks_its_limit_on_host(lib):
    """The allocation-free prefill form takes its scratch from a fixed 64 MiB
    per-device array: 1,636 rows fit at K = 1024 and 2,045 at K = 512, one more
    is rejected with MQA_ERR_BAD_SIZE before any HIP call."""
    import fp4_mqa_scoring_amd as m
    assert m.STATIC_SCRATCH_BYTES == 64 << 20
    p = ctypes.c_void_p(0x1000)

    def call(Q, K, flags=0):
        return lib.mqa_fp4_topk_prefill_static(p, p, Q, p, p, 2, p, p, 2, p, p, K, p, p, p, None, flags, None)
    assert call(1637, 1024) == -4
    assert call(2046, 512) == -4
    assert call(1636, 1024) != -4                   # fits: fails later, at the device checks (no GPU here)
    assert call(2045, 512) != -4
    assert call(10, 700) == -1
    assert call(10, 512, flags=0x500) == -8


def test_binding_rejects_malformed_tensors_before_the_library():
    """The Python binding only marshals pointers, so it refuses any tensor whose
    dtype, contiguity or shape differs from the header's layout (host tensors:
    nothing reaches the library)."""
    import torch
    import fp4_mqa_scoring_amd as mqa
    Q, P, K = 4, 8, 512

    def args(**over):
        a = dict(q=torch.zeros(Q, 64, 64, dtype=torch.uint8), q_scale=torch.zeros(Q, 64, 4, dtype=torch.uint8),
                 k_pages=torch.zeros(P, 64, 64, dtype=torch.uint8), k_scale=torch.zeros(P, 64, 4, dtype=torch.uint8),
                 weights=torch.zeros(Q, 64), page_table=torch.zeros(P, dtype=torch.int32),
                 row_start=torch.zeros(Q, dtype=torch.int32), row_end=torch.zeros(Q, dtype=torch.int32), K=K,
                 out_raw=torch.zeros(Q, K, dtype=torch.int32), out_slot=torch.zeros(Q, K, dtype=torch.int32),
                 out_count=torch.zeros(Q, dtype=torch.int32))
        a.update(over)
        return a

    bad = [
        (TypeError, dict(weights=torch.zeros(Q, 64, dtype=torch.float16))),               # dtype
        (TypeError, dict(q="not a tensor")),
        (ValueError, dict(q=torch.zeros(Q, 64, 128, dtype=torch.uint8)[:, :, ::2])),     # strided view
        (ValueError, dict(weights=torch.zeros(64, Q).t())),                              # transposed
        (ValueError, dict(q_scale=torch.zeros(Q, 64, 2, dtype=torch.uint8))),             # shape
        (ValueError, dict(k_scale=torch.zeros(P + 1, 64, 4, dtype=torch.uint8))),
        (ValueError, dict(row_end=torch.zeros(Q + 1, dtype=torch.int32))),
        (ValueError, dict(out_raw=torch.zeros(Q, K + 1, dtype=torch.int32))),
        (ValueError, dict(out_count=torch.zeros(Q - 1, dtype=torch.int32))),
    ]
    for exc, over in bad:
        with pytest.raises(exc):
            mqa.mqa_fp4_topk_prefill(**args(**over))
