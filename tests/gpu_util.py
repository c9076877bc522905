"""Helpers of the GPU tests: move seeded inputs to the device and run the
library's entry points through the Python binding (itself a thin C-ABI call)."""
import numpy as np

import fp4_mqa_scoring_amd as mqa


def has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(inp, device="cuda:0"):
    import torch
    d = {}
    for name in ("q", "q_scale", "k_pages", "k_scale", "weights", "page_table", "row_start", "row_end"):
        d[name] = torch.from_numpy(np.ascontiguousarray(getattr(inp, name))).to(device)
    return d


def run_fused(dev, K, flags=0, with_score=True, stream=None):
    import torch
    Q = dev["q"].shape[0]
    outs = mqa.alloc_outputs(Q, K, dev["q"].device, with_score=with_score)
    for t in outs:
        t.fill_(-7)
    score = outs[3] if with_score else None
    mqa.mqa_fp4_topk_prefill_ex(dev["q"], dev["q_scale"], dev["k_pages"], dev["k_scale"], dev["weights"],
                                dev["page_table"], dev["row_start"], dev["row_end"], K,
                                outs[0], outs[1], outs[2], score, flags, stream=stream)
    torch.cuda.synchronize()
    res = [t.cpu().numpy() for t in outs]
    return res[0], res[1], res[2], (res[3] if with_score else None)


def run_dense(dev, K, with_score=True):
    import torch
    Q = dev["q"].shape[0]
    S = 64 * dev["page_table"].shape[0]
    logits = torch.full((Q, S), float("nan"), dtype=torch.float32, device=dev["q"].device)
    outs = mqa.alloc_outputs(Q, K, dev["q"].device, with_score=with_score)
    for t in outs:
        t.fill_(-7)
    score = outs[3] if with_score else None
    mqa.mqa_fp4_dense_topk_prefill(dev["q"], dev["q_scale"], dev["k_pages"], dev["k_scale"], dev["weights"],
                                   dev["page_table"], dev["row_start"], dev["row_end"], K, logits,
                                   outs[0], outs[1], outs[2], score)
    torch.cuda.synchronize()
    res = [t.cpu().numpy() for t in outs]
    return res[0], res[1], res[2], (res[3] if with_score else None), logits


def dense_logits(dev):
    import torch
    Q = dev["q"].shape[0]
    S = 64 * dev["page_table"].shape[0]
    logits = torch.full((Q, S), float("nan"), dtype=torch.float32, device=dev["q"].device)
    mqa.mqa_fp4_dense_logits(dev["q"], dev["q_scale"], dev["k_pages"], dev["k_scale"], dev["weights"],
                             dev["page_table"], dev["row_start"], dev["row_end"], logits)
    torch.cuda.synchronize()
    return logits.cpu().numpy()


def run_tiled(dev, K, tile=0, with_score=True):
    import torch
    Q = dev["q"].shape[0]
    outs = mqa.alloc_outputs(Q, K, dev["q"].device, with_score=with_score)
    for t in outs:
        t.fill_(-7)
    score = outs[3] if with_score else None
    mqa.mqa_fp4_tiled_topk_prefill(dev["q"], dev["q_scale"], dev["k_pages"], dev["k_scale"], dev["weights"],
                                   dev["page_table"], dev["row_start"], dev["row_end"], K,
                                   outs[0], outs[1], outs[2], score, tile_positions=tile)
    torch.cuda.synchronize()
    res = [t.cpu().numpy() for t in outs]
    return res[0], res[1], res[2], (res[3] if with_score else None)
