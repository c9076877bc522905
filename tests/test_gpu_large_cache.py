"""A key cache larger than 4 GiB, with every page a window touches above byte
offset 2^32 of k_pages (and 2^28 of k_scale): each address into the cache needs
64-bit arithmetic, which the operators promise ("[AMD][DSv4] Add experimental
AITER FP4 streaming TopK", Memory geometry; "[FlyDSL] Add FP4 LiteTopK prefill
operator", Implementation).

The inputs are a compact seeded workload copied to the top of a 1.1M-page
cache, its page table shifted by the same page offset. Raw indices, counts and
scores must not change; slots move by 64 x the offset. The compact run is
checked against the oracle and the large-cache run against the compact one, bit
for bit, for the fused path (gated, ungated, forced fallback, several splits),
the dense comparator, the tiled path and the decode form. The cache writer is
checked at the same high pages against the oracle's quantiser.
"""
import numpy as np
import pytest

import oracle
import fp4_mqa_scoring_amd as mqa
from fp4_mqa_scoring_amd import synth
import gpu_util as gu
from test_gpu_parity import check_rows
from test_gpu_decode import _dev as decode_dev, run_decode, check_decode

pytestmark = pytest.mark.gpu

BIG_PAGES = 1_100_000                     # 4.51e9 code bytes + 2.8e8 scale bytes


def _need_gpu():
    if not gu.has_gpu():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def big_cache():
    _need_gpu()
    import torch
    kp = torch.empty((BIG_PAGES, 64, 64), dtype=torch.uint8, device="cuda")
    ks = torch.empty((BIG_PAGES, 64, 4), dtype=torch.uint8, device="cuda")
    yield kp, ks
    del kp, ks
    torch.cuda.empty_cache()


def _move_to_top(dev, kp, ks, n_phys):
    """Copies the compact cache into the last n_phys pages of the large one and
    returns the page offset."""
    off = BIG_PAGES - n_phys
    assert off * 64 * 64 > 2**32 and off * 64 * 4 > 2**28
    kp[off:] = dev["k_pages"]
    ks[off:] = dev["k_scale"]
    return off


def _same_but_slots(a, b, off, tag):
    """a, b: (raw, slot, count, score). Everything bit-equal except that b's
    valid slots are a's plus 64 * off."""
    assert np.array_equal(a[0], b[0]), f"{tag}: raw"
    assert np.array_equal(a[2], b[2]), f"{tag}: count"
    if a[3] is not None:
        assert np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32)), f"{tag}: score"
    valid = a[1] >= 0
    assert np.array_equal(b[1][~valid], a[1][~valid]), f"{tag}: padding"
    assert np.array_equal(b[1][valid].astype(np.int64), a[1][valid].astype(np.int64) + 64 * off), f"{tag}: slots"


@pytest.mark.parametrize("K", [512, 1024])
def test_prefill_paths_on_a_cache_beyond_4_gib(big_cache, K):
    _need_gpu()
    import torch
    kp, ks = big_cache
    rng = np.random.default_rng(90 + K)
    Q, S = 24, 8192
    st = rng.integers(0, 2000, Q).astype(np.int32)
    en = np.minimum(st + rng.integers(K + 1, S, Q), S).astype(np.int32)
    st[0], en[0] = 0, S                                   # the whole context
    st[1], en[1] = 100, 100 + K // 2                      # short row
    st[2], en[2] = S - K - 1, S                           # K + 1 positions at the end
    inp = synth.make_inputs(Q, S, K, 9100 + K, row_start=st, row_end=en, P_phys=S // 64 + 5)
    dev = gu.to_device(inp)
    off = _move_to_top(dev, kp, ks, inp.P_phys)
    big = dict(dev, k_pages=kp, k_scale=ks, page_table=dev["page_table"] + off)
    mqa.mqa_fp4_status()                                  # clear bits other tests left

    base = gu.run_fused(dev, K)
    check_rows(inp, range(Q), *base, where=f"compact K={K}")
    for flags in (0, 3, mqa.FLAG_NO_PREFILTER, mqa.FLAG_FORCE_UNDERFILL | 2):
        _same_but_slots(base, gu.run_fused(big, K, flags=flags), off, f"fused K={K} flags={flags:#x}")
    dense = gu.run_dense(big, K)
    _same_but_slots(base, dense[:4], off, f"dense K={K}")
    _same_but_slots(base, gu.run_tiled(big, K, tile=3072), off, f"tiled K={K}")
    assert mqa.mqa_fp4_status() == 0
    torch.cuda.synchronize()


def test_decode_on_a_cache_beyond_4_gib(big_cache):
    _need_gpu()
    kp, ks = big_cache
    K = 1024
    d = synth.make_decode_inputs(6, 2, K // 2, 7000, K, seed=95)
    t = decode_dev(d)
    n_phys = int(d.k_pages.shape[0])
    off = _move_to_top(t, kp, ks, n_phys)
    bt = t["block_table"]
    big = dict(t, k_pages=kp, k_scale=ks, block_table=bt.where(bt < 0, bt + off))
    mqa.mqa_fp4_status()
    base = run_decode(t, K)
    check_decode(d, base, where="compact decode")
    got = run_decode(big, K)
    _same_but_slots(base, got, off, "decode")
    assert mqa.mqa_fp4_status() == 0


def test_cache_writer_beyond_4_gib(big_cache):
    _need_gpu()
    import torch
    kp, ks = big_cache
    rng = np.random.default_rng(97)
    P_log = 48
    page_table = (BIG_PAGES - 1 - rng.permutation(P_log)).astype(np.int32)   # the top 48 pages
    n = 2000
    positions = rng.choice(64 * P_log, n, replace=False).astype(np.int32)
    k = rng.standard_normal((n, 128)).astype(np.float32) * np.float32(3.0)
    kp[BIG_PAGES - P_log:] = 0xAB
    ks[BIG_PAGES - P_log:] = 0xCD
    mqa.mqa_fp4_status()
    mqa.mqa_fp4_cache_write(torch.from_numpy(k).cuda(), torch.from_numpy(positions).cuda(),
                            torch.from_numpy(page_table).cuda(), kp, ks)
    torch.cuda.synchronize()
    assert mqa.mqa_fp4_status() == 0
    want_c, want_s = oracle.mx_quantize(k)
    base = (BIG_PAGES - P_log) * 64
    gc = kp[BIG_PAGES - P_log:].cpu().numpy().reshape(-1, 64)
    gs = ks[BIG_PAGES - P_log:].cpu().numpy().reshape(-1, 4)
    slots = np.array([oracle.slot(int(p), page_table) for p in positions], np.int64) - base
    assert np.array_equal(gc[slots], want_c) and np.array_equal(gs[slots], want_s)
    untouched = np.setdiff1d(np.arange(P_log * 64), slots)
    assert np.all(gc[untouched] == 0xAB) and np.all(gs[untouched] == 0xCD)
