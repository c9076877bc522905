#!/usr/bin/env python3
"""Benchmark of the fused FP4 paged-MQA indexer + exact TopK on one MI355X.

One step = one call of mqa_fp4_topk_prefill (row preparation, fused MXFP4
scoring + streaming TopK, exact split merge + page mapping) on the headline
workload of "[FlyDSL] Add FP4 LiteTopK prefill operator" (ROCm/aiter PR
5309), Validation table: V4-Pro shape, Q=8192 rows, H=64, D=128, K=1024,
C4 context 196,608 (786,432 raw tokens), ragged causal prefill windows,
shuffled pages, synthetic seeded FP4 data (fp4_mqa_scoring_amd/synth.py).

Prints ONE JSON line. Besides the timed fused steps it measures, outside the
timed region: the in-house dense comparator in alternating dense/fused pairs
(the pages' protocol: 5 warmup + 15 measured pairs), the library's scratch
bytes, and the CPU oracle on a bounded sample of rows (cpu_baseline).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FLOP_PER_PAIR = 2 * 64 * 128          # MXFP4 MFMA work per scored (row, position) pair
FLOP_PER_MFMA = 2 * 32 * 32 * 64      # one v_mfma_scale_f32_32x32x64_f8f6f4
VALU_PER_PAIR = 2 * 64                # integer ReLU + fp32 FMA per head
MXFP4_PEAK = 10.1e15                  # MI355X dense MXFP4 MFMA, FLOP/s
VALU_PEAK = 157.3e12 / 2              # fp32 vector: 157.3 TFLOP/s = 78.65e12 FMA lane-ops/s
# On gfx950 a SIMD runs MFMA and VALU work largely one after the other (the issue
# probe measures how little of it overlaps), so the scorer's ceiling at the
# published rates is the sum of both times per pair.
SERIAL_PAIR_S = FLOP_PER_PAIR / MXFP4_PEAK + VALU_PER_PAIR / VALU_PEAK
HBM_PEAK = 8.0e12
PAGES_LITETOPK_MS = {  # PR 5309 Validation table, MI355X, LiteTopK column
    (8192, 196608, 1024): 10.6433, (8192, 131072, 1024): 7.4099, (8192, 65536, 1024): 4.1911,
    (8192, 196608, 512): 10.4344, (8192, 131072, 512): 7.2235, (8192, 65536, 512): 3.9221,
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_kernel_traffic.json")


def code_hash(*files: str) -> str:
    """Hash of the code of the given csrc files (comments and whitespace removed):
    the byte counters in profiles/ stay valid while this hash is unchanged."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "fp4_mqa_scoring_amd", "csrc", f)) as fh:
            text = re.sub(r"//[^\n]*", "", fh.read())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return code_hash("mqa_device.h", "mqa_select.h", "mqa_launch.h", "mqa_kernels.hip")


def decode_source_hash() -> str:
    return code_hash("mqa_device.h", "mqa_select.h", "mqa_launch.h", "mqa_decode.hip")


class HipEvents:
    """hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n: int):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float(0.0)
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def cpu_baseline(inp, budget_s: float, seed: int):
    """The oracle as it stands on this host's cores: whole rows of the same
    workload (scores + full sort + page map) until the time budget is used."""
    import oracle
    rows = list(np.random.default_rng(seed).permutation(inp.Q))
    pairs, t0, done = 0, time.perf_counter(), []
    for r in rows:
        n = int(inp.row_end[r] - inp.row_start[r])
        oracle.topk_row(inp, int(r))
        pairs += n
        done.append(int(r))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": pairs / dt, "unit": "scored pairs/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": model, "os_cpu_count": os.cpu_count(),
            "extrapolated_full_call_s": inp.scored_pairs() / (pairs / dt),
            "extrapolation": "scored pairs of the whole call / the sample's pairs/s (not run)",
            "sample": f"{len(done)} full rows of the same workload ({pairs} scored pairs, "
                      f"{dt:.1f} s wall), float64 scores + full sort, OpenMP over positions"}


QUANT_BYTES = 128 * 4 + 64 + 4          # fp32 vector in, codes + scales out
CACHE_WRITE_BYTES = QUANT_BYTES + 4 + 4 # + logical position + page-table entry


def bench_quantize(args, torch, mqa, dev):
    """The producer of the operator's inputs at the headline shape: quantise the
    query tensor [8192, 64, 128] and write the C4 key cache of 196,608 positions
    through a shuffled page table. HBM-bound; one step = both launches."""
    Q, S = 8192, 196608
    g = torch.Generator(device=dev).manual_seed(20261202)
    xq = torch.randn((Q * 64, 128), generator=g, device=dev, dtype=torch.float32)
    xk = torch.randn((S, 128), generator=g, device=dev, dtype=torch.float32)
    P = S // 64
    page_table = torch.randperm(P, generator=g, device=dev).to(torch.int32)
    positions = torch.arange(S, dtype=torch.int32, device=dev)
    qc = torch.empty((Q * 64, 64), dtype=torch.uint8, device=dev)
    qs = torch.empty((Q * 64, 4), dtype=torch.uint8, device=dev)
    kp = torch.empty((P, 64, 64), dtype=torch.uint8, device=dev)
    ks = torch.empty((P, 64, 4), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        mqa.mqa_fp4_quantize(xq, qc, qs, stream=stream)
        if ev:
            ev[1].record(stream)
        mqa.mqa_fp4_cache_write(xk, positions, page_table, kp, ks, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    q_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    w_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    assert mqa.mqa_fp4_status(stream) == 0
    # practical ceiling for context: a plain device copy of the quantiser's input bytes
    y = torch.empty_like(xq)
    for _ in range(3):
        y.copy_(xq)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        y.copy_(xq)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * xq.numel() * 4 / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
    del y
    q_bytes = Q * 64 * QUANT_BYTES
    w_bytes = S * CACHE_WRITE_BYTES
    traffic = None
    tf = os.path.join(ROOT, "profiles", "mx_quantize_traffic.json")
    if os.path.exists(tf):
        with open(tf) as fh:
            tr = json.load(fh)
        if tr.get("kernel_source_hash") == code_hash("mqa_device.h", "mqa_quant.hip"):
            traffic = tr.get("bytes_per_launch")
    line = {
        "metric": "GB/s, MXFP4 quantisation of the query tensor + C4 cache write (headline shape)",
        "value": (q_bytes + w_bytes) / (wall_ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 -> mxfp4 (e2m1 + ue8m0)", "data": "synthetic",
        "config": {"workload": f"quantise q [{Q}, 64, 128] + write C4 cache of {S} positions",
                   "vectors_quantised": Q * 64, "cache_positions": S},
        "roofline": {"bound": "hbm", "achieved": q_bytes / (q_ms * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": q_bytes / (q_ms * 1e-3) / HBM_PEAK, "traffic": traffic,
                     "kernel": "mx_quantize_kernel (quantise)", "kernel_ms": q_ms,
                     "cache_write_ms": w_ms,
                     "cache_write_gbs": w_bytes / (w_ms * 1e-3) / 1e9,
                     "cache_write_frac": w_bytes / (w_ms * 1e-3) / HBM_PEAK,
                     "device_copy_gbs": copy_gbs},
        "cpu_baseline": None,
    }
    if args.cpu_budget > 0:
        import oracle
        xs = xq[: 1 << 16].cpu().numpy()
        t1, nvec = time.perf_counter(), 0
        while time.perf_counter() - t1 < min(args.cpu_budget, 10.0):
            oracle.mx_quantize(xs)
            nvec += xs.shape[0]
        dt = time.perf_counter() - t1
        line["cpu_baseline"] = {"value": nvec * QUANT_BYTES / dt / 1e9, "unit": "GB/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{nvec} vectors (65,536 per pass of the same query tensor), "
                                          f"{dt:.1f} s wall, single-threaded C"}
    print(json.dumps(line), flush=True)


DECODE_BYTES_PER_PAIR = 64 + 4         # key codes + scales read once per scored pair (no sharing between rows)


def bench_decode(args, torch, mqa, dev):
    """The multi-sequence form on a decode batch: 64 sequences, one query row
    each, C4 contexts uniform in [32768, 131072], K = 1024, pages of all
    sequences scattered over one shuffled pool. One step = one call, captured in
    a HIP graph and replayed (the eager call is timed beside it)."""
    from fp4_mqa_scoring_amd import synth
    K = 1024
    d = synth.make_decode_inputs(64, 1, 32768, 131072, K, seed=20261202)
    t = {n: torch.from_numpy(np.ascontiguousarray(getattr(d, n))).to(dev)
         for n in ("q", "q_scale", "k_pages", "k_scale", "weights", "block_table", "seq_of_row", "row_start",
                   "row_end")}
    Q = d.Q
    pairs = d.scored_pairs()
    outs = mqa.alloc_outputs(Q, K, dev)
    ws = torch.empty(mqa.mqa_fp4_decode_workspace_bytes(Q, K), dtype=torch.uint8, device=dev)

    def call(stream=None):
        mqa.mqa_fp4_topk_decode(t["q"], t["q_scale"], t["k_pages"], t["k_scale"], t["weights"], t["block_table"],
                                t["seq_of_row"], t["row_start"], t["row_end"], K, outs[0], outs[1], outs[2], ws,
                                stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(args.warmup, 1)):
            call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    graph_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    # eager calls with the library's stage events: the gated scan kernel alone
    hev = HipEvents()
    sev = [hev.create(5) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in sev:
        mqa.mqa_fp4_set_stage_events(e)
        call()
    mqa.mqa_fp4_set_stage_events(None)
    torch.cuda.synchronize()
    eager_ms = float(np.mean([hev.elapsed_ms(e[0], e[4]) for e in sev]))
    scan_ms = float(np.mean([hev.elapsed_ms(e[2], e[3]) for e in sev]))
    for e in sev:
        hev.destroy(e)
    assert mqa.mqa_fp4_status(stream) == 0
    counts = outs[2].cpu().numpy()
    n = d.lengths()
    ok = bool(np.all(counts == np.minimum(n, K)))
    key_bytes = pairs * DECODE_BYTES_PER_PAIR
    # scaled FETCH_SIZE + WRITE_SIZE bytes of one gated-scan launch, if counted on these sources
    traffic = None
    tf = os.path.join(ROOT, "profiles", "decode_gscan_traffic.json")
    if os.path.exists(tf):
        with open(tf) as fh:
            tr = json.load(fh)
        if tr.get("kernel_source_hash") == decode_source_hash():
            traffic = tr.get("bytes_per_launch")
    line = {
        "metric": "ms/call + scored pairs/s, decode batch (multi-sequence form, HIP graph replay)",
        "value": pairs / (wall_ms * 1e-3), "unit": "scored pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4 x mxfp4 -> f32", "data": "synthetic",
        "config": {"workload": "decode: 64 sequences x 1 row, C4 context 32768..131072, K=1024",
                   "Q": Q, "K": K, "scored_pairs": pairs, "workspace_bytes": ws.numel()},
        "roofline": {"bound": "hbm", "achieved": key_bytes / (scan_ms * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": key_bytes / (scan_ms * 1e-3) / HBM_PEAK, "traffic": traffic,
                     "kernel": "decode_gscan_kernel<1024>", "kernel_ms": scan_ms,
                     "graph_replay_ms": graph_ms, "eager_call_ms": eager_ms,
                     "call_key_gbs": key_bytes / (graph_ms * 1e-3) / 1e9,
                     "mfma_frac": pairs * FLOP_PER_PAIR / (scan_ms * 1e-3) / MXFP4_PEAK},
        "checks_ok": ok,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="H",
                    help="H (headline), 1..5, or another shape of the pages' Validation table: "
                         "F65, F131, F196 (V4-Flash, K=512), P65, P131 (V4-Pro, K=1024)")
    ap.add_argument("--pairs", type=int, default=15, help="alternating dense/fused pairs (0 = skip dense)")
    ap.add_argument("--tiled-pairs", type=int, default=5,
                    help="alternating context-tiled/fused pairs (0 = skip the tiled comparator)")
    ap.add_argument("--tile", type=int, default=0, help="positions per tile of the tiled comparator (0 = 4096)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (for counter scaling)")
    ap.add_argument("--splits", type=int, default=0, help="override context splits (0 = automatic)")
    ap.add_argument("--op", default="topk", choices=("topk", "quantize", "decode", "probe"),
                    help="topk: the fused operator (default); quantize: the MXFP4 quantiser and the C4 cache "
                         "writer on the headline call's query tensor and cache; decode: the multi-sequence "
                         "form on a decode batch, timed as HIP graph replays; probe: the issue and LDS probes "
                         "alone (for counter runs)")
    ap.add_argument("--processes", type=int, default=3,
                    help="fresh processes for --op topk, median reported (the pages' protocol; 1 = this one)")
    ap.add_argument("--extras", type=int, default=1,
                    help="also run the probes, the tiled comparator and the CPU baseline (1) or not (0)")
    argv = sys.argv[1:]
    args = ap.parse_args(argv)
    args.passthrough = child_args(argv)

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the operator shards by rows "
              "with no exchange between GPUs, so N GPUs would run N independent row slices", file=sys.stderr)
        sys.exit(2)
    if args.op == "topk" and args.processes > 1:
        run_processes(args)
        return

    import torch
    import fp4_mqa_scoring_amd as mqa
    from fp4_mqa_scoring_amd import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    mqa.lib()                          # fail loudly if the HIP library is not built
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    # one plain device copy of known size first, to scale the byte counters
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.op == "quantize":
        bench_quantize(args, torch, mqa, dev)
        return
    if args.op == "decode":
        bench_decode(args, torch, mqa, dev)
        return
    if args.op == "probe":
        from fp4_mqa_scoring_amd import probe
        out = {"issue_rates": probe.issue_rates(),
               "lds_read_probe_ms": {p: probe.lds_ms(i) for i, p in enumerate(("scan_image", "linear", "unswizzled"))}}
        print(json.dumps(out), flush=True)
        return
    cfg = int(args.workload) if args.workload.isdigit() else args.workload
    if cfg not in synth.CONFIGS:
        sys.exit(f"bench.py: unknown workload {args.workload!r} (H, 1..5, F65, F131, F196, P65, P131)")
    inp = synth.make_config(cfg)
    Q, S, K = inp.Q, inp.S, inp.K
    pairs = inp.scored_pairs()
    t = {n: torch.from_numpy(np.ascontiguousarray(getattr(inp, n))).to(dev)
         for n in ("q", "q_scale", "k_pages", "k_scale", "weights", "page_table", "row_start", "row_end")}
    out_raw, out_slot, out_count = mqa.alloc_outputs(Q, K, dev)
    stream = torch.cuda.current_stream(dev)


    def fused():
        mqa.mqa_fp4_topk_prefill_ex(t["q"], t["q_scale"], t["k_pages"], t["k_scale"], t["weights"],
                                    t["page_table"], t["row_start"], t["row_end"], K, out_raw, out_slot,
                                    out_count, None, args.splits, stream=stream)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()

    ev = HipEvents()
    evs = [ev.create(5) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        mqa.mqa_fp4_set_stage_events(evs[i])
        fused()
    mqa.mqa_fp4_set_stage_events(None)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    call_ms = [ev.elapsed_ms(e[0], e[4]) for e in evs]
    prep_ms = [ev.elapsed_ms(e[0], e[1]) for e in evs]
    calib_ms = [ev.elapsed_ms(e[1], e[2]) for e in evs]
    kern_ms = [ev.elapsed_ms(e[2], e[3]) for e in evs]      # the scan kernel alone
    merge_ms = [ev.elapsed_ms(e[3], e[4]) for e in evs]
    for e in evs:
        ev.destroy(e)
    status = mqa.mqa_fp4_status(stream)
    counts = out_count.cpu().numpy()
    n = inp.lengths()
    ok = bool(np.all(counts[n > K] == K) and np.all(counts[n <= K] == n[n <= K]) and status == 0)

    ms_step = wall_ms                   # synchronized wall clock of the timed steps
    kern = float(np.mean(kern_ms))
    value = pairs / (ms_step * 1e-3)
    kern_flops = pairs * FLOP_PER_PAIR / (kern * 1e-3)
    kern_valu = pairs * VALU_PER_PAIR / (kern * 1e-3)

    # issue rates of this device's SIMDs, in shader cycles (bench-only probe library),
    # and the LDS read pattern of the score-block image; outside the timed region
    rates, lds = None, None
    if args.extras:
        from fp4_mqa_scoring_amd import probe
        rates = probe.issue_rates(stream=stream)
        lds = {"scan_image": probe.lds_ms(0, stream=stream), "linear": probe.lds_ms(1, stream=stream),
               "unswizzled": probe.lds_ms(2, stream=stream)}

    # alternating dense / fused pairs, outside the timed region
    dense = None
    if args.pairs > 0:
        logits = torch.empty((Q, S), dtype=torch.float32, device=dev)
        d_out = mqa.alloc_outputs(Q, K, dev)

        def dense_call():
            mqa.mqa_fp4_dense_topk_prefill(t["q"], t["q_scale"], t["k_pages"], t["k_scale"], t["weights"],
                                           t["page_table"], t["row_start"], t["row_end"], K, logits, *d_out,
                                           stream=stream)
        dms, fms = [], []
        for i in range(5 + args.pairs):
            torch.cuda.synchronize()
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s2 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            dense_call()
            s1.record(stream)
            fused()
            s2.record(stream)
            torch.cuda.synchronize()
            if i >= 5:
                dms.append(s0.elapsed_time(s1))
                fms.append(s1.elapsed_time(s2))
        same = bool(torch.equal(d_out[0], out_raw) and torch.equal(d_out[2], out_count))
        dense = {"dense_ms_median": float(np.median(dms)), "fused_ms_median": float(np.median(fms)),
                 "pairs": args.pairs, "dense_equals_fused": same,
                 "dense_logits_bytes": Q * S * 4}
        del logits

    # alternating context-tiled / fused pairs, outside the timed region
    tiled = None
    if args.tiled_pairs > 0 and args.extras:
        t_out = mqa.alloc_outputs(Q, K, dev)

        def tiled_call():
            mqa.mqa_fp4_tiled_topk_prefill(t["q"], t["q_scale"], t["k_pages"], t["k_scale"], t["weights"],
                                           t["page_table"], t["row_start"], t["row_end"], K, *t_out,
                                           tile_positions=args.tile, stream=stream)
        tms, fms = [], []
        for i in range(2 + args.tiled_pairs):
            torch.cuda.synchronize()
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s2 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            tiled_call()
            s1.record(stream)
            fused()
            s2.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                tms.append(s0.elapsed_time(s1))
                fms.append(s1.elapsed_time(s2))
        same = bool(torch.equal(t_out[0], out_raw) and torch.equal(t_out[2], out_count))
        tiled = {"tiled_ms_median": float(np.median(tms)), "fused_ms_median": float(np.median(fms)),
                 "pairs": args.tiled_pairs, "tile_positions": args.tile or 4096,
                 "tiled_scratch_bytes": mqa.mqa_fp4_tiled_scratch_bytes(Q, K, args.tile),
                 "tiled_equals_fused": same}
        del t_out

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("workload") == str(args.workload):
            traffic = tr.get("bytes_per_launch")

    line = {
        "metric": "ms/call + scored pairs/s (% MXFP4 MFMA peak), Q=8192 C4=196608 K=1024",
        "value": value,
        "unit": "scored pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 x mxfp4 -> f32",
        "data": "synthetic",
        "config": {"workload": inp.name, "Q": Q, "c4_context": S, "K": K, "heads": 64, "head_dim": 128,
                   "page_size": 64, "windows": "ragged causal, end_i = S - floor((Q-1-i)/4)",
                   "scored_pairs": pairs, "splits": args.splits or "auto"},
        "roofline": {"bound": "mfma", "achieved": kern_flops / 1e12, "peak": MXFP4_PEAK / 1e12,
                     "unit": "TFLOP/s", "frac": kern_flops / MXFP4_PEAK, "traffic": traffic,
                     "kernel": f"scan_kernel<{K}>", "kernel_ms": kern,
                     "valu_frac": kern_valu / VALU_PEAK,
                     "mfma_plus_valu_frac": pairs * SERIAL_PAIR_S / (kern * 1e-3),
                     "measured_peak_tflops": rates["mxfp4_tflops_measured"] if rates else None,
                     "frac_of_measured_peak": kern_flops / 1e12 / rates["mxfp4_tflops_measured"] if rates else None,
                     # shader cycles per SIMD: MFMA and fp32 FMA issue, and how much of the
                     # shorter of the two hides when one SIMD runs both (0 = none)
                     "issue_rates": rates,
                     # LDS reads of the score-block image: the scan's pattern vs a linear
                     # (conflict-free) one and the unswizzled image
                     "lds_read_probe_ms": lds},
        "mxfp4_tflops_per_call": pairs * FLOP_PER_PAIR / (ms_step * 1e-3) / 1e12,
        "mxfp4_peak_frac_per_call": pairs * FLOP_PER_PAIR / (ms_step * 1e-3) / MXFP4_PEAK,
        "stage_ms": {"row_prep": float(np.mean(prep_ms)), "calibration": float(np.mean(calib_ms)),
                     "scan": kern, "merge_fallback": float(np.mean(merge_ms)),
                     "call_events": float(np.mean(call_ms))},
        "scratch_bytes": mqa.mqa_fp4_topk_scratch_bytes(Q, K, 0),
        "dense_comparator": dense,
        "tiled_comparator": tiled,
        "checks_ok": ok,
    }
    key = (Q, S, K)
    if key in PAGES_LITETOPK_MS:   # the pages' LiteTopK at this exact shape
        line["vs_baseline"] = PAGES_LITETOPK_MS[key] / ms_step
    if args.cpu_budget > 0 and args.extras:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, seed=1)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def child_args(argv):
    """The arguments a child process inherits: all but the process options."""
    out, skip = [], False
    for a in argv:
        if skip:
            skip = False
            continue
        if a in ("--processes", "--extras"):
            skip = True
            continue
        if a.startswith("--processes=") or a.startswith("--extras="):
            continue
        out.append(a)
    return out


def merge_lines(lines, args):
    """One line from the children's lines: the first child's, with its time
    figures replaced by the median over the children and every rate scaled to
    match; each child's figures listed under "processes"."""
    line = dict(lines[0])
    med = lambda xs: float(np.median(xs))
    ms = med([ln["ms_per_step"] for ln in lines])
    scale = lines[0]["ms_per_step"] / ms
    line["value"] = lines[0]["value"] * scale
    line["ms_per_step"] = ms
    if line.get("vs_baseline") is not None:
        line["vs_baseline"] *= scale
    for k in ("mxfp4_tflops_per_call", "mxfp4_peak_frac_per_call"):
        if k in line:
            line[k] *= scale
    roof = dict(line["roofline"])
    kms = med([ln["roofline"]["kernel_ms"] for ln in lines])
    ks = roof["kernel_ms"] / kms
    for k in ("achieved", "frac", "valu_frac", "mfma_plus_valu_frac", "frac_of_measured_peak"):
        if roof.get(k) is not None:
            roof[k] *= ks
    roof["kernel_ms"] = kms
    line["roofline"] = roof
    line["stage_ms"] = {k: med([ln["stage_ms"][k] for ln in lines]) for k in line["stage_ms"]}
    if line.get("dense_comparator"):
        line["dense_comparator"] = dict(line["dense_comparator"])
        for k in ("dense_ms_median", "fused_ms_median"):
            line["dense_comparator"][k] = med([ln["dense_comparator"][k] for ln in lines])
        line["dense_comparator"]["dense_equals_fused"] = all(ln["dense_comparator"]["dense_equals_fused"]
                                                             for ln in lines)
    line["checks_ok"] = all(ln["checks_ok"] for ln in lines)
    line["processes"] = [{"ms_per_step": ln["ms_per_step"], "kernel_ms": ln["roofline"]["kernel_ms"],
                          "dense_ms_median": (ln.get("dense_comparator") or {}).get("dense_ms_median")}
                         for ln in lines]
    line["protocol"] = (f"median of {len(lines)} fresh processes; each: {args.warmup} warmup + {args.steps} "
                        f"timed calls, then 5 warmup + {args.pairs} alternating dense/fused pairs")
    return line


def run_processes(args) -> None:
    """The pages' protocol ("[FlyDSL] Add FP4 LiteTopK prefill operator",
    Validation: median of three fresh processes): the same measurement in fresh
    child processes, started before this process touches the GPU; the first
    also runs the probes, the tiled comparator and the CPU baseline."""
    import subprocess
    lines = []
    for i in range(args.processes):
        cmd = [sys.executable, os.path.abspath(__file__), "--processes", "1",
               "--extras", "1" if i == 0 else "0"] + args.passthrough
        print(f"bench.py: process {i + 1} of {args.processes}", file=sys.stderr, flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        if r.returncode != 0:
            sys.exit(r.returncode)
        lines.append(json.loads(r.stdout.strip().splitlines()[-1]))
    print(json.dumps(merge_lines(lines, args)), flush=True)


if __name__ == "__main__":
    main()
