"""The allocation-free prefill entry point (mqa_fp4_topk_prefill_static, scratch
from the library's fixed per-device array) against the allocating one
(mqa_fp4_topk_prefill_ex) through the C ABI: every output bit for bit, on calls
in a row with a smaller batch after a larger one (the array keeps the previous
call's contents), with the test flags, at its row limit, and across HIP graph
replays with eager calls in between."""
import numpy as np
import pytest

import fp4_mqa_scoring_amd as mqa
from fp4_mqa_scoring_amd import synth
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not gu.has_gpu():
        pytest.skip("no GPU")


def _run(dev, K, static, flags=0, stream=None):
    import torch
    Q = dev["q"].shape[0]
    outs = mqa.alloc_outputs(Q, K, dev["q"].device, with_score=True)
    for t in outs:
        t.fill_(-7)
    fn = mqa.mqa_fp4_topk_prefill_static if static else mqa.mqa_fp4_topk_prefill_ex
    fn(dev["q"], dev["q_scale"], dev["k_pages"], dev["k_scale"], dev["weights"], dev["page_table"],
       dev["row_start"], dev["row_end"], K, outs[0], outs[1], outs[2], outs[3], flags, stream=stream)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in outs]


def _same(a, b, what):
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), what


def _inputs(Q, S, K, seed):
    """Ragged windows with short rows, an empty row, an invalid window and a page
    out of range (touched by one long row)."""
    rng = np.random.default_rng(seed)
    st = rng.integers(0, S // 4, Q).astype(np.int32)
    en = np.minimum(st + rng.integers(K // 2, S, Q), S).astype(np.int32)
    st[1], en[1] = 7, 7                          # empty
    st[2], en[2] = 100, 100 + K                  # exactly K: short
    st[3], en[3] = 9, 4                          # invalid window
    inp = synth.make_inputs(Q, S, K, seed, row_start=st, row_end=en, P_phys=S // 64 + 2)
    inp.page_table[S // 64 - 1] = inp.P_phys + 3
    inp.row_start[4], inp.row_end[4] = S - 3000, S   # long row through the bad page
    inp.q[5] = 0                                     # all-equal scores
    return inp


def test_two_calls_in_a_row_match_the_allocating_entry_point():
    """A 1,636-row batch (the limit at K = 1024) then a smaller one at K = 512,
    then the first again: each equals mqa_fp4_topk_prefill_ex bit for bit."""
    _need_gpu()
    big = _inputs(1636, 64 * 300, 1024, 11)
    small = _inputs(37, 64 * 90, 512, 12)
    db, ds = gu.to_device(big), gu.to_device(small)
    want_big = _run(db, 1024, static=False)
    want_small = _run(ds, 512, static=False)
    mqa.mqa_fp4_status()
    _same(want_big, _run(db, 1024, static=True), "first call, 1,636 rows")
    _same(want_small, _run(ds, 512, static=True), "second call, 37 rows")
    _same(want_big, _run(db, 1024, static=True), "third call, 1,636 rows again")
    assert mqa.mqa_fp4_status() == mqa.STATUS_BAD_WINDOW | mqa.STATUS_BAD_PAGE


@pytest.mark.parametrize("flags", [3, mqa.FLAG_NO_PREFILTER, mqa.FLAG_FORCE_UNDERFILL | 2,
                                   mqa.FLAG_NO_FALLBACK | mqa.FLAG_FORCE_UNDERFILL])
def test_flags_match_the_allocating_entry_point(flags):
    _need_gpu()
    inp = _inputs(50, 64 * 200, 1024, 13)
    dev = gu.to_device(inp)
    _same(_run(dev, 1024, static=False, flags=flags), _run(dev, 1024, static=True, flags=flags), hex(flags))
    mqa.mqa_fp4_status()


def test_batches_beyond_the_array_are_rejected_and_write_nothing():
    _need_gpu()
    import torch
    inp = _inputs(1637, 64 * 40, 1024, 14)
    dev = gu.to_device(inp)
    outs = mqa.alloc_outputs(inp.Q, 1024, "cuda")
    for t in outs:
        t.fill_(-7)
    with pytest.raises(mqa.MQAError) as e:
        mqa.mqa_fp4_topk_prefill_static(dev["q"], dev["q_scale"], dev["k_pages"], dev["k_scale"], dev["weights"],
                                        dev["page_table"], dev["row_start"], dev["row_end"], 1024, *outs)
    assert e.value.code == -4
    torch.cuda.synchronize()
    for t in outs:
        assert torch.all(t == -7)


def test_graph_replays_match_eager():
    """Captured once on a side stream; replayed four times with the inputs of
    two batches copied into the captured buffers between replays, and an eager
    call of the allocation-free entry point on a third batch (same stream
    order) between replays; every replay equals the allocating entry point's
    result for the inputs it saw."""
    _need_gpu()
    import torch
    K = 1024
    a = _inputs(64, 64 * 160, K, 21)
    b = _inputs(64, 64 * 160, K, 22)
    c = _inputs(20, 64 * 50, 512, 23)
    b.row_start, b.row_end, b.page_table = a.row_start, a.row_end, a.page_table   # same shapes and metadata
    ta, tb, tc = gu.to_device(a), gu.to_device(b), gu.to_device(c)
    want_a, want_b, want_c = _run(ta, K, False), _run(tb, K, False), _run(tc, 512, False)
    mqa.mqa_fp4_status()
    static = {n: v.clone() for n, v in ta.items()}
    outs = mqa.alloc_outputs(a.Q, K, "cuda", with_score=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):        # first call on the device outside capture (symbol address, device info)
        mqa.mqa_fp4_topk_prefill_static(static["q"], static["q_scale"], static["k_pages"], static["k_scale"],
                                        static["weights"], static["page_table"], static["row_start"],
                                        static["row_end"], K, *outs, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mqa.mqa_fp4_topk_prefill_static(static["q"], static["q_scale"], static["k_pages"], static["k_scale"],
                                        static["weights"], static["page_table"], static["row_start"],
                                        static["row_end"], K, *outs)
    for rep, (src, want) in enumerate([(tb, want_b), (ta, want_a), (tb, want_b), (ta, want_a)]):
        for n in static:
            static[n].copy_(src[n])
        for o in outs:
            o.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(want, [o.cpu().numpy() for o in outs], f"replay {rep}")
        _same(want_c, _run(tc, 512, static=True), f"eager call after replay {rep}")
    mqa.mqa_fp4_status()
