"""The bounded context-tiled exact path ("[FlyDSL][DSv4] Prototype FP4 MQA
streaming TopK", Changes: the correctness / reference fallback) against the
oracle and the fused path, through the C ABI. Bar: outputs identical to the
fused path bit for bit (same exact TopK under bit-identical scores), whatever
the tile size; the oracle's checks on every row of the tiny workload."""
import numpy as np
import pytest

import fp4_mqa_scoring_amd as mqa
from fp4_mqa_scoring_amd import synth
import gpu_util as gu
from test_gpu_parity import check_rows, medium_inputs

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not gu.has_gpu():
        pytest.skip("no GPU")


def _same(a, b, tag):
    for x, y in zip(a, b):
        if x is None:
            continue
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), tag


def test_tiny_tiled_matches_oracle_all_rows():
    _need_gpu()
    inp = synth.make_config(1)
    dev = gu.to_device(inp)
    for tile in (256, 768, 0):
        raw, slot, cnt, score = gu.run_tiled(dev, inp.K, tile)
        check_rows(inp, range(inp.Q), raw, slot, cnt, score, where=f"tiled {tile}")


@pytest.mark.parametrize("K", [512, 1024])
def test_tiled_equals_fused_for_every_tile_size(K):
    _need_gpu()
    inp = medium_inputs(seed=71, K=K, S=4096 if K == 1024 else 2560)
    inp.q[11] = 0                                        # all-equal scores: order by index
    dev = gu.to_device(inp)
    base = gu.run_fused(dev, K)
    for tile in (256, 512, 1280, 4096, 1 << 16):
        _same(base, gu.run_tiled(dev, K, tile), f"K={K} tile={tile}")
    assert mqa.mqa_fp4_status() == 0


def test_tiled_fails_closed_like_fused():
    _need_gpu()
    inp = medium_inputs(seed=61)
    inp.row_start[0], inp.row_end[0] = 10, 5
    inp.row_start[2], inp.row_end[2] = 0, inp.S + 1
    inp.page_table[7] = inp.P_phys + 4
    inp.row_start[8], inp.row_end[8] = 0, 2000
    dev = gu.to_device(inp)
    mqa.mqa_fp4_status()
    base = gu.run_fused(dev, inp.K)
    st_f = mqa.mqa_fp4_status()
    got = gu.run_tiled(dev, inp.K, 512)
    st_t = mqa.mqa_fp4_status()
    assert st_f == st_t == mqa.STATUS_BAD_WINDOW | mqa.STATUS_BAD_PAGE
    _same(base, got, "fail closed")


def test_tiled_full_size_workload_equals_fused():
    """Config 2 at full size (Q=1024, C4=65,536, K=512)."""
    _need_gpu()
    inp = synth.make_config(2)
    dev = gu.to_device(inp)
    base = gu.run_fused(dev, inp.K)
    _same(base, gu.run_tiled(dev, inp.K, 0), "config 2")
    check_rows(inp, [0, 511, inp.Q - 1], *base, where="config 2 tiled")
