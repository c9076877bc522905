"""Seeded randomized sweep over small shapes. Each case draws the number of
rows, the context, K, windows of every kind (empty, short, unaligned, whole
context), a page table with some entries out of range, rows with all-zero or
negated weights and rows with all-equal scores. Every entry point that returns
a TopK runs on it: the fused path with random flags and splits, the context-
tiled path with a random tile, and the decode form with one sequence. Every row
of each is checked against the oracle, and the three agree bit for bit on raw
indices, slots, counts and scores. A second set draws a few rows over long contexts
(65K-397K positions) and random context splits, so that the calibration runs
split and the merges see several splits' candidates. Failure messages name the
case's seed and shape."""
import numpy as np
import pytest

import fp4_mqa_scoring_amd as mqa
from fp4_mqa_scoring_amd import synth
import gpu_util as gu
from test_gpu_parity import check_rows

pytestmark = pytest.mark.gpu

N_CASES = 96
N_LONG_CASES = 40


def draw_case(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    K = int(rng.choice([512, 1024]))
    S = 64 * int(rng.integers(4, 80))                     # 256 .. 5,056 positions
    Q = int(rng.integers(1, 40))
    P_log = S // 64
    P_phys = P_log + int(rng.integers(0, 4))
    start = np.zeros(Q, np.int64)
    end = np.zeros(Q, np.int64)
    for r in range(Q):
        kind = int(rng.integers(0, 5))
        if kind == 0:                                     # empty window
            start[r] = end[r] = int(rng.integers(0, S + 1))
        elif kind == 1:                                   # short: at most K positions
            n = int(rng.integers(1, K + 1))
            start[r] = int(rng.integers(0, max(1, S - n + 1)))
            end[r] = min(S, start[r] + n)
        elif kind == 2:                                   # the whole context
            end[r] = S
        else:                                             # any window
            a, b = sorted(int(x) for x in rng.integers(0, S + 1, 2))
            start[r], end[r] = a, b
    inp = synth.make_inputs(Q, S, K, 50_000 + seed, row_start=start, row_end=end, P_phys=P_phys,
                            tie_rows=int(rng.integers(0, 2)) if Q > 1 else 0,
                            name=f"sweep seed {seed}: Q={Q} S={S} K={K}")
    for r in range(Q):
        u = rng.random()
        if u < 0.08:
            inp.weights[r] = 0.0                          # every score +0: the first K positions
        elif u < 0.2:
            inp.weights[r] = -inp.weights[r]
    if rng.random() < 0.3:                                # one page out of range
        inp.page_table[int(rng.integers(0, P_log))] = int(rng.choice([-1, P_phys, P_phys + 7]))
    flags = int(rng.choice([0, mqa.FLAG_NO_PREFILTER, mqa.FLAG_FORCE_UNDERFILL])) | int(rng.integers(0, 18))
    tile = 256 * int(rng.integers(1, 12))
    return inp, flags, tile


def draw_long_case(seed):
    """A few rows over a long context (65,536 .. 396,736 positions): the
    calibration runs split over the context when splits > 1."""
    rng = np.random.Generator(np.random.PCG64(10_000 + seed))
    K = int(rng.choice([512, 1024]))
    S = 64 * int(rng.integers(1024, 6200))
    Q = int(rng.integers(1, 20))
    start = np.zeros(Q, np.int64)
    end = np.zeros(Q, np.int64)
    for r in range(Q):
        kind = int(rng.integers(0, 5))
        if kind == 0:                                     # short
            n = int(rng.integers(1, K + 1))
            start[r] = int(rng.integers(0, S - n + 1))
            end[r] = start[r] + n
        elif kind == 1:                                   # causal-like: almost the whole context
            end[r] = S - int(rng.integers(0, 3000))
        elif kind == 2:                                   # a little longer than K
            n = int(rng.integers(K + 1, 4 * K))
            start[r] = int(rng.integers(0, S - n + 1))
            end[r] = start[r] + n
        else:                                             # any window
            a, b = sorted(int(x) for x in rng.integers(0, S + 1, 2))
            start[r], end[r] = a, b
    inp = synth.make_inputs(Q, S, K, 70_000 + seed, row_start=start, row_end=end, P_phys=S // 64 + 2,
                            tie_rows=int(rng.integers(0, 2)) if Q > 1 else 0,
                            name=f"long sweep seed {seed}: Q={Q} S={S} K={K}")
    return inp, int(rng.integers(2, 18))


def run_decode_one_sequence(dev, K):
    import torch
    Q = dev["q"].shape[0]
    outs = mqa.alloc_outputs(Q, K, dev["q"].device, with_score=True)
    for t in outs:
        t.fill_(-7)
    ws = torch.empty(mqa.mqa_fp4_decode_workspace_bytes(Q, K), dtype=torch.uint8, device=dev["q"].device)
    bt = dev["page_table"].reshape(1, -1).contiguous()
    seq = torch.zeros(Q, dtype=torch.int32, device=dev["q"].device)
    mqa.mqa_fp4_topk_decode(dev["q"], dev["q_scale"], dev["k_pages"], dev["k_scale"], dev["weights"], bt, seq,
                            dev["row_start"], dev["row_end"], K, outs[0], outs[1], outs[2], ws, out_score=outs[3])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in outs]


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    if not gu.has_gpu():
        pytest.skip("no GPU")
    inp, flags, tile = draw_case(seed)
    dev = gu.to_device(inp)
    tag = f"{inp.name} flags={flags:#x} tile={tile}"
    print(tag, flush=True)
    fused = gu.run_fused(dev, inp.K, flags=flags)
    check_rows(inp, range(inp.Q), *fused, where=f"{tag} fused")
    tiled = gu.run_tiled(dev, inp.K, tile=tile)
    check_rows(inp, range(inp.Q), *tiled, where=f"{tag} tiled")
    dec = run_decode_one_sequence(dev, inp.K)
    check_rows(inp, range(inp.Q), *dec, where=f"{tag} decode")
    for name, other in (("tiled", tiled), ("decode", dec)):
        for i, what in enumerate(("raw", "slot", "count", "score")):
            assert np.array_equal(np.asarray(fused[i]).view(np.uint32), np.asarray(other[i]).view(np.uint32)), \
                f"{tag}: fused and {name} differ in {what}"
    mqa.mqa_fp4_status()   # clear the sticky bits that fail-closed rows set


@pytest.mark.parametrize("seed", range(N_LONG_CASES))
def test_random_long_case(seed):
    """One context split against several (calibration split too) and against
    the automatic count, every row against the oracle, and the decode form
    bit-equal to them."""
    if not gu.has_gpu():
        pytest.skip("no GPU")
    inp, splits = draw_long_case(seed)
    dev = gu.to_device(inp)
    tag = f"{inp.name} splits={splits}"
    print(tag, flush=True)
    base = gu.run_fused(dev, inp.K, flags=1)
    check_rows(inp, range(inp.Q), *base, where=f"{tag} one split")
    for f in (splits, 0):   # the drawn count, then the automatic one
        got = gu.run_fused(dev, inp.K, flags=f)
        for a, b in zip(base, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{tag}: splits {f} change the outputs"
    dec = run_decode_one_sequence(dev, inp.K)
    for i, what in enumerate(("raw", "slot", "count", "score")):
        assert np.array_equal(np.asarray(base[i]).view(np.uint32), np.asarray(dec[i]).view(np.uint32)), \
            f"{tag}: fused and decode differ in {what}"
    mqa.mqa_fp4_status()
