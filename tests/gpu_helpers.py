"""Shared helpers of the GPU parity tests (inputs to the device, oracle
problems, printing the case before each GPU step)."""
import sys

import numpy as np
import torch

import fp8_mqa_logits_amd as mqa
import oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(wl, dev="cuda"):
    d = {
        "q": torch.from_numpy(wl.q).to(dev),
        "k": torch.from_numpy(wl.k).to(dev),
        "weights": torch.from_numpy(wl.weights).to(dev),
        "starts": torch.from_numpy(wl.starts).to(dev),
        "ends": torch.from_numpy(wl.ends).to(dev),
    }
    sb = torch.from_numpy(np.ascontiguousarray(wl.scale_bytes)).to(dev)
    d["scales"] = mqa.mqa_key_scales(sb)
    return d


def oracle_problem(wl):
    return oracle.Problem(wl.q, wl.k, oracle.key_scales(wl.scale_bytes), wl.weights, wl.starts,
                          wl.ends)


def fused(d, topk, flags=0, workspace=None):
    out = mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"],
                               d["ends"], topk, workspace=workspace, flags=flags)
    torch.cuda.synchronize()
    return out
