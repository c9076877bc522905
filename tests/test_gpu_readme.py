"""The Python example in README.md runs as written and its outputs match the
oracle (rows sampled across the batch) and the dense comparator (every row)."""
import re
import os

import numpy as np
import pytest

import fp4_mqa_scoring_amd as mqa
from fp4_mqa_scoring_amd import synth
import gpu_util as gu
from test_gpu_parity import check_rows

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example():
    if not gu.has_gpu():
        pytest.skip("no GPU")
    import torch
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    torch.cuda.synchronize()
    cpu = lambda n: ns[n].cpu().numpy()
    inp = synth.Inputs(cpu("q"), cpu("q_scale"), cpu("k_pages"), cpu("k_scale"), cpu("weights"), cpu("page_table"),
                       cpu("row_start"), cpu("row_end"), ns["K"], name="README example")
    raw, slot, count = cpu("raw"), cpu("slot"), cpu("count")
    assert np.all(count == ns["K"])
    check_rows(inp, [0, 1, 77, 128, 200, ns["Q"] - 1], raw, slot, count, where="README example")
    d_raw, d_slot, d_cnt = mqa.alloc_outputs(ns["Q"], ns["K"], "cuda")
    logits = torch.empty(ns["Q"], ns["S"], dtype=torch.float32, device="cuda")
    mqa.mqa_fp4_dense_topk_prefill(ns["q"], ns["q_scale"], ns["k_pages"], ns["k_scale"], ns["weights"],
                                   ns["page_table"], ns["row_start"], ns["row_end"], ns["K"], logits, d_raw, d_slot,
                                   d_cnt)
    torch.cuda.synchronize()
    assert np.array_equal(d_raw.cpu().numpy(), raw) and np.array_equal(d_slot.cpu().numpy(), slot)


def test_readme_decode_example():
    """The README's decode example runs as written; the graph replay's outputs
    equal an eager call's, and every row matches the oracle through its
    sequence's block table."""
    if not gu.has_gpu():
        pytest.skip("no GPU")
    import torch
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.findall(r"```python\n(.*?)```", text, re.S)[1]
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    torch.cuda.synchronize()
    cpu = lambda n: ns[n].cpu().numpy()
    replayed = [cpu(n) for n in ("raw", "slot", "count")]
    ns["step"]()
    torch.cuda.synchronize()
    for a, n in zip(replayed, ("raw", "slot", "count")):
        assert np.array_equal(a, cpu(n)), n
    K = ns["K"]
    d = synth.DecodeInputs(cpu("q"), cpu("q_scale"), cpu("k_pages"), cpu("k_scale"), cpu("weights"),
                           cpu("block_table"), cpu("seq_of_row"), cpu("row_start"), cpu("row_end"),
                           ns["lens"].numpy().astype(np.int64), K, name="README decode example")
    raw, slot, count = replayed
    assert np.all(count == K)
    for r in range(d.Q):
        check_rows(d.view(int(d.seq_of_row[r])), [r], raw, slot, count, where=f"README decode row {r}")
