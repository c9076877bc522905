"""Host-side contract of bench.py (no GPU): a run asked for more than one GPU
stops with a message before touching a device, and the source hash that ties
the byte counters in profiles/ to the kernel sources ignores comments and
layout but not code."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")          # no result line


def test_code_hash_ignores_comments_and_layout_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "fp4_mqa_scoring_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("int f(int x) { return x + 1; }  // one\n")
    h0 = bench.code_hash("k.hip")
    (csrc / "k.hip").write_text("// a comment\nint f(int x) {\n  return x + 1;   // two\n}\n")
    assert bench.code_hash("k.hip") == h0
    (csrc / "k.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.code_hash("k.hip") != h0


def test_traffic_profiles_name_their_kernel_and_sources():
    """Each committed traffic profile carries the source hash that bench.py
    compares before reporting its bytes (a stale profile is reported as null)."""
    for name in ("scan_kernel_traffic.json", "decode_gscan_traffic.json", "mx_quantize_traffic.json"):
        with open(os.path.join(ROOT, "profiles", name)) as fh:
            t = json.load(fh)
        assert len(t["kernel_source_hash"]) == 16 and t["bytes_per_launch"] > 0, name


def test_children_inherit_every_argument_but_the_process_options():
    argv = ["--steps", "20", "--processes", "3", "--warmup", "5", "--extras=0", "--workload", "4"]
    assert bench.child_args(argv) == ["--steps", "20", "--warmup", "5", "--workload", "4"]


def test_merged_line_takes_the_median_process():
    """Three children's lines merge into one: ms_per_step is the median child's,
    every rate scales with it, the checks hold only if every child's hold."""
    class A:
        steps, warmup, pairs = 20, 5, 15

    def child(ms, kms, ok=True):
        return {"value": 1e12 / ms, "ms_per_step": ms, "vs_baseline": 10.0 / ms, "checks_ok": ok,
                "mxfp4_tflops_per_call": 100.0 / ms, "mxfp4_peak_frac_per_call": 0.01 / ms,
                "roofline": {"achieved": 50.0 / kms, "frac": 0.005 / kms, "kernel_ms": kms, "valu_frac": 0.1 / kms,
                             "mfma_plus_valu_frac": 0.2 / kms, "frac_of_measured_peak": None, "traffic": None},
                "stage_ms": {"scan": kms, "call_events": ms},
                "dense_comparator": {"dense_ms_median": 2 * ms, "fused_ms_median": ms, "dense_equals_fused": True}}
    lines = [child(8.0, 7.5), child(8.4, 7.9), child(8.2, 7.6)]
    m = bench.merge_lines(lines, A)
    assert m["ms_per_step"] == 8.2 and abs(m["value"] - 1e12 / 8.2) < 1
    assert abs(m["vs_baseline"] - 10.0 / 8.2) < 1e-12
    assert m["roofline"]["kernel_ms"] == 7.6 and abs(m["roofline"]["achieved"] - 50.0 / 7.6) < 1e-12
    assert abs(m["roofline"]["frac"] - 0.005 / 7.6) < 1e-15
    assert m["dense_comparator"]["dense_ms_median"] == 16.4 and m["checks_ok"]
    assert len(m["processes"]) == 3 and "median of 3" in m["protocol"]
    lines[1]["checks_ok"] = False
    assert not bench.merge_lines(lines, A)["checks_ok"]
