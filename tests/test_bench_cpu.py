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
