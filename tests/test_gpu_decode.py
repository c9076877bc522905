"""Decode / multi-sequence form: per-row page tables, caller workspace, graph
capture. Checked against the oracle row by row through each sequence's own page
table (the oracle's definition is per row), against the prefill path when all
rows share one table, and across HIP graph replays. Bar as for the operator:
slots, counts, padding bit-exact; scores within 1e-5; selections by
oracle/check.py."""
import numpy as np
import pytest

import fp4_mqa_scoring_amd as mqa
from fp4_mqa_scoring_amd import synth
import gpu_util as gu
from test_gpu_parity import check_rows

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not gu.has_gpu():
        pytest.skip("no GPU")


def _dev(d):
    import torch
    return {n: torch.from_numpy(np.ascontiguousarray(getattr(d, n))).cuda()
            for n in ("q", "q_scale", "k_pages", "k_scale", "weights", "block_table", "seq_of_row", "row_start",
                      "row_end")}


def run_decode(t, K, splits=0, with_score=True, flags=0):
    import torch
    Q = t["q"].shape[0]
    outs = mqa.alloc_outputs(Q, K, t["q"].device, with_score=with_score)
    for o in outs:
        o.fill_(-7)
    ws = torch.empty(mqa.mqa_fp4_decode_workspace_bytes(Q, K, splits), dtype=torch.uint8, device="cuda")
    mqa.mqa_fp4_topk_decode(t["q"], t["q_scale"], t["k_pages"], t["k_scale"], t["weights"], t["block_table"],
                            t["seq_of_row"], t["row_start"], t["row_end"], K, outs[0], outs[1], outs[2], ws,
                            out_score=outs[3] if with_score else None, splits=splits, flags=flags)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def check_decode(d, res, rows=None, where=""):
    rows = range(d.Q) if rows is None else rows
    for r in rows:
        check_rows(d.view(int(d.seq_of_row[r])), [r], *res, where=f"{where} seq {d.seq_of_row[r]}")


@pytest.mark.parametrize("K,rps", [(512, 1), (1024, 3)])
def test_multi_sequence_rows_match_the_oracle(K, rps):
    _need_gpu()
    d = synth.make_decode_inputs(10, rps, K // 2, 9000, K, seed=40 + rps)
    d.q[1] = 0                                             # all-equal scores in one row
    res = run_decode(_dev(d), K)
    check_decode(d, res, where=f"decode K={K}")
    assert mqa.mqa_fp4_status() == 0


@pytest.mark.timeout(300)
def test_sequences_of_two_million_positions():
    """Two sequences of 1.5M-2.1M C4 positions, one row each: the gate samples
    a coarser multiple of its page stride there; rows against the oracle through
    their tables, the ungated run bit-equal."""
    _need_gpu()
    K = 1024
    d = synth.make_decode_inputs(2, 1, 1_500_000, 1 << 21, K, seed=2048)
    t = _dev(d)
    res = run_decode(t, K)
    check_decode(d, res, where="2M decode")
    for a, b in zip(res, run_decode(t, K, flags=mqa.FLAG_NO_PREFILTER)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert mqa.mqa_fp4_status() == 0


def test_infinite_and_nan_weights_order_exactly_like_the_oracle():
    """Rows whose scores hold +-inf and NaN (a weight of +-inf gives +-inf where
    the head's dot is positive and NaN where it is 0; a NaN weight makes every
    score NaN, so the selection is the first K positions): the gate, the scan's
    exact key test on NaN classes and the merge order them as the oracle does,
    and the gated, ungated and forced-underfill runs agree bit for bit."""
    _need_gpu()
    K = 1024
    d = synth.make_decode_inputs(6, 1, 3000, 9000, K, seed=515)
    d.weights[0, 3] = np.inf
    d.weights[1, 10] = -np.inf
    d.weights[2, 40] = np.nan
    d.weights[3, 0], d.weights[3, 1] = np.inf, -np.inf
    t = _dev(d)
    base = run_decode(t, K)
    raw, slot, cnt, _ = base
    for r in range(d.Q):
        check_rows(d.view(int(d.seq_of_row[r])), [r], raw, slot, cnt, None, where=f"special weights row {r}")
    for flags in (mqa.FLAG_NO_PREFILTER, mqa.FLAG_FORCE_UNDERFILL):
        got = run_decode(t, K, flags=flags)
        for a, b in zip(base, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), hex(flags)
    assert mqa.mqa_fp4_status() == 0


@pytest.mark.parametrize("K", [512, 1024])
def test_sliding_windows_match_the_oracle(K):
    """Windows that start inside the sequence (sliding windows), most of them
    off a page boundary: 14 sequences x 2 rows, window lengths from just above
    K to 40,000 positions and a few short ones, starts anywhere before the
    end. Every row against the oracle through its sequence's table, and the
    gated, ungated and forced-underfill runs bit for bit equal."""
    _need_gpu()
    d = synth.make_decode_inputs(14, 2, 6000, 60000, K, seed=2600 + K)
    rng = np.random.default_rng(2700 + K)
    for r in range(d.Q):
        end = int(d.row_end[r])
        if r % 7 == 3:
            n = int(rng.integers(1, K + 1))                # short: at most K positions
        else:
            n = int(rng.integers(K + 1, min(40000, end) + 1))
        d.row_start[r] = end - n
    assert np.any(d.row_start % 64 != 0) and np.any(d.row_start > 0)
    t = _dev(d)
    base = run_decode(t, K)
    check_decode(d, base, where=f"sliding K={K}")
    for flags in (mqa.FLAG_NO_PREFILTER, mqa.FLAG_FORCE_UNDERFILL):
        got = run_decode(t, K, flags=flags)
        for a, b in zip(base, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), hex(flags)
    assert mqa.mqa_fp4_status() == 0


def test_splits_do_not_change_outputs():
    _need_gpu()
    d = synth.make_decode_inputs(5, 2, 2000, 12000, 1024, seed=7)
    t = _dev(d)
    base = run_decode(t, 1024, splits=1)
    for s in (3, 7, 64):
        got = run_decode(t, 1024, splits=s)
        for a, b in zip(base, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), s


@pytest.mark.parametrize("K", [512, 1024])
def test_gate_off_and_forced_underfill_give_identical_outputs(K):
    """The calibrated gate, no gate (every row through the exact pool fallback)
    and a forced underfill (gate above every key, then the fallback) agree bit for
    bit; tie rows (all-equal scores) included."""
    _need_gpu()
    d = synth.make_decode_inputs(9, 2, K + 1, 20000, K, seed=91 + K)
    d.q[3] = 0
    d.q[8] = 0
    t = _dev(d)
    base = run_decode(t, K)
    check_decode(d, base, where=f"gated K={K}")
    for flags in (mqa.FLAG_NO_PREFILTER, mqa.FLAG_FORCE_UNDERFILL):
        got = run_decode(t, K, flags=flags)
        for a, b in zip(base, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), hex(flags)
    assert mqa.mqa_fp4_status() == 0


def test_one_sequence_equals_the_prefill_path():
    """All rows in one sequence: identical to mqa_fp4_topk_prefill bit for bit."""
    _need_gpu()
    import torch
    from test_gpu_parity import medium_inputs
    inp = medium_inputs(seed=88, K=512)
    dev = gu.to_device(inp)
    base = gu.run_fused(dev, inp.K)
    t = {"q": dev["q"], "q_scale": dev["q_scale"], "k_pages": dev["k_pages"], "k_scale": dev["k_scale"],
         "weights": dev["weights"], "block_table": dev["page_table"][None, :].contiguous(),
         "seq_of_row": torch.zeros(inp.Q, dtype=torch.int32, device="cuda"),
         "row_start": dev["row_start"], "row_end": dev["row_end"]}
    got = run_decode(t, inp.K)
    for a, b in zip(base, got):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_bad_sequences_and_pages_fail_closed():
    _need_gpu()
    d = synth.make_decode_inputs(6, 1, 700, 3000, 512, seed=9)
    d.seq_of_row[0] = 6                                   # no such sequence
    d.seq_of_row[1] = -1
    d.block_table[2, 3] = d.k_pages.shape[0] + 5          # page 3 of sequence 2 outside the cache
    d.row_start[3], d.row_end[3] = 5, 2                   # end < start
    t = _dev(d)
    mqa.mqa_fp4_status()
    raw, slot, cnt, score = run_decode(t, 512)
    assert mqa.mqa_fp4_status() == mqa.STATUS_BAD_WINDOW | mqa.STATUS_BAD_PAGE
    for r, code in ((0, -1), (1, -1), (2, -2), (3, -1)):
        assert cnt[r] == code and np.all(raw[r] == -1) and np.all(slot[r] == -1), r
    check_decode(d, (raw, slot, cnt, score), rows=[4, 5], where="neighbours")


def test_workspace_too_small_is_rejected():
    _need_gpu()
    import torch
    d = synth.make_decode_inputs(2, 1, 600, 900, 512, seed=3)
    t = _dev(d)
    outs = mqa.alloc_outputs(d.Q, 512, "cuda")
    need = mqa.mqa_fp4_decode_workspace_bytes(d.Q, 512, 4)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mqa.MQAError) as e:
        mqa.mqa_fp4_topk_decode(t["q"], t["q_scale"], t["k_pages"], t["k_scale"], t["weights"], t["block_table"],
                                t["seq_of_row"], t["row_start"], t["row_end"], 512, *outs[:3], ws, splits=4)
    assert e.value.code == -4


def test_graph_capture_and_replays_match_eager():
    """Captured once, replayed several times with different inputs copied into
    the captured buffers eagerly between replays; every replay equals the eager
    result for the inputs it saw."""
    _need_gpu()
    import torch
    K = 1024
    da = synth.make_decode_inputs(8, 2, 800, 6000, K, seed=21)
    db = synth.make_decode_inputs(8, 2, 800, 6000, K, seed=22)
    # same shapes for both sets: share the block table / windows of `a`, new data for `b`
    db.block_table, db.seq_of_row, db.row_start, db.row_end = da.block_table, da.seq_of_row, da.row_start, da.row_end
    db.k_pages, db.k_scale = db.k_pages[:da.k_pages.shape[0]], db.k_scale[:da.k_scale.shape[0]]
    ta, tb = _dev(da), _dev(db)
    assert all(ta[n].shape == tb[n].shape for n in ta)
    want_a, want_b = run_decode(ta, K), run_decode(tb, K)
    static = {n: v.clone() for n, v in ta.items()}
    Q = da.Q
    outs = mqa.alloc_outputs(Q, K, "cuda", with_score=True)
    ws = torch.empty(mqa.mqa_fp4_decode_workspace_bytes(Q, K), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):        # warm the library outside capture (device info, module load)
        mqa.mqa_fp4_topk_decode(static["q"], static["q_scale"], static["k_pages"], static["k_scale"],
                                static["weights"], static["block_table"], static["seq_of_row"], static["row_start"],
                                static["row_end"], K, outs[0], outs[1], outs[2], ws, out_score=outs[3], stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mqa.mqa_fp4_topk_decode(static["q"], static["q_scale"], static["k_pages"], static["k_scale"],
                                static["weights"], static["block_table"], static["seq_of_row"], static["row_start"],
                                static["row_end"], K, outs[0], outs[1], outs[2], ws, out_score=outs[3])
    for rep, (src, want) in enumerate([(tb, want_b), (ta, want_a), (tb, want_b), (ta, want_a)]):
        for n in static:
            static[n].copy_(src[n])
        for o in outs:
            o.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy() for o in outs]
        for a, b in zip(want, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), rep
    assert mqa.mqa_fp4_status() == 0


def test_decode_shape_long_contexts_sampled_rows():
    """64 sequences x 1 row, C4 contexts 30,000..131,072, K = 1024; 6 rows checked."""
    _need_gpu()
    d = synth.make_decode_inputs(64, 1, 30000, 131072, 1024, seed=64)
    res = run_decode(_dev(d), 1024)
    check_decode(d, res, rows=[0, 17, 31, 40, 55, 63], where="decode long")
    n = d.lengths()
    assert np.all(res[2] == np.minimum(n, 1024))


def test_scan_shares_span_many_rows():
    """20,000 rows of 400..720 positions at K = 512: more rows than the gated
    scan has waves, so each wave's equal share of all rows' pages runs over
    several rows, with short rows (no pages to scan) and rows of an invalid
    sequence between them. Bit-equal to the no-prefilter run (the exact fallback,
    which splits every row the same way) on every row; sampled rows against the
    oracle."""
    _need_gpu()
    K = 512
    d = synth.make_decode_inputs(5000, 4, 400, 720, K, seed=4242)
    for r in (3, 4, 5, 777, 19999):
        d.seq_of_row[r] = 5000 + r                            # invalid sequence: code -1
    t = _dev(d)
    mqa.mqa_fp4_status()
    base = run_decode(t, K)
    assert mqa.mqa_fp4_status() == mqa.STATUS_BAD_WINDOW
    n = d.lengths()
    bad = np.zeros(d.Q, bool)
    bad[[3, 4, 5, 777, 19999]] = True
    assert np.all(base[2][bad] == -1)
    assert np.all(base[2][~bad] == np.minimum(n[~bad], K))
    assert (n[~bad] <= K).sum() > 1000 and (n[~bad] > K).sum() > 10000
    got = run_decode(t, K, flags=mqa.FLAG_NO_PREFILTER)
    assert mqa.mqa_fp4_status() == mqa.STATUS_BAD_WINDOW     # read and cleared
    for a, b in zip(base, got):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rows = [r for r in np.random.default_rng(7).choice(d.Q, 48, replace=False) if not bad[r]]
    check_decode(d, base, rows=rows + [0, 1, 2, 6, 19998], where="shares over many rows")


def test_scan_shares_with_more_rows_than_half_the_waves():
    """3,000 long rows (600..1,200 positions, K = 512): more long rows than half
    the gated scan's waves, fewer rows than the plan keeps in LDS, so the plan
    gives the waves equal shares of the concatenated page list (a share runs
    over two or three rows). Bit-equal to the no-prefilter run on every row;
    sampled rows against the oracle."""
    _need_gpu()
    K = 512
    d = synth.make_decode_inputs(1500, 2, 600, 1200, K, seed=3131)
    n = d.lengths()
    assert (n > K).sum() == d.Q == 3000
    t = _dev(d)
    mqa.mqa_fp4_status()
    base = run_decode(t, K)
    got = run_decode(t, K, flags=mqa.FLAG_NO_PREFILTER)
    assert mqa.mqa_fp4_status() == 0
    assert np.all(base[2] == K)
    for a, b in zip(base, got):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rows = sorted(np.random.default_rng(11).choice(d.Q, 40, replace=False).tolist())
    check_decode(d, base, rows=rows + [0, d.Q - 1], where="shares over 3,000 rows")


@pytest.mark.parametrize("K", [512, 1024])
def test_windows_beyond_the_sample_budget(K):
    """Windows of 140,000..300,000 positions (2,188..4,688 pages): the per-row
    gate samples at most 128 pages, so rows beyond 262,144 positions sample every
    64th page instead of every 32nd; every row still matches the oracle."""
    _need_gpu()
    d = synth.make_decode_inputs(3, 1, 140000, 300000, K, seed=65 + K)
    assert d.lengths().max() > 262144
    res = run_decode(_dev(d), K)
    check_decode(d, res, where=f"decode beyond the sample budget K={K}")
    assert np.all(res[2] == K)
    assert mqa.mqa_fp4_status() == 0


@pytest.mark.parametrize("K", [512, 1024])
def test_underfill_without_fallback_fails_closed(K):
    """As for the prefill path: with MQA_FLAG_NO_FALLBACK a forced underfill
    fails every long row closed (all -1, NaN scores, count -3, underfill bit),
    short rows and a row of an invalid sequence are answered as always, and
    without the forced underfill the outputs equal the default run's."""
    _need_gpu()
    d = synth.make_decode_inputs(6, 2, K // 3, 9000, K, seed=57 + K)
    d.seq_of_row[4] = d.seq_of_row.max() + 5                   # invalid sequence: code -1
    d.row_end[2] = d.row_start[2] + K // 2                      # a short row
    t = _dev(d)
    mqa.mqa_fp4_status()
    base = run_decode(t, K)
    st0 = mqa.mqa_fp4_status()
    assert st0 == mqa.STATUS_BAD_WINDOW
    got = run_decode(t, K, flags=mqa.FLAG_NO_FALLBACK)
    for a, b in zip(base, got):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert mqa.mqa_fp4_status() == st0
    raw, slot, cnt, score = run_decode(t, K, flags=mqa.FLAG_NO_FALLBACK | mqa.FLAG_FORCE_UNDERFILL)
    assert mqa.mqa_fp4_status() == st0 | mqa.STATUS_UNDERFILL
    n = d.row_end.astype(np.int64) - d.row_start.astype(np.int64)
    n_failed = 0
    for r in range(d.Q):
        if r == 4:
            assert cnt[r] == -1 and np.all(raw[r] == -1) and np.all(slot[r] == -1)
        elif n[r] <= K:
            assert cnt[r] == base[2][r] and np.array_equal(raw[r], base[0][r])
            assert np.array_equal(slot[r], base[1][r])
        else:
            assert cnt[r] == mqa.ROW_UNDERFILL, (r, cnt[r])
            assert np.all(raw[r] == -1) and np.all(slot[r] == -1) and np.all(np.isnan(score[r]))
            n_failed += 1
    assert n_failed >= 4
