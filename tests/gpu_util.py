"""Shared helpers for the GPU tests: upload the generator's exact bits, fetch results as float64."""
import sys

import numpy as np


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits, dtype):
    import torch
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
    elif dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16)
    else:
        raise ValueError(dtype)
    return t.cuda()


def from_dev(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def upload(inp):
    q = to_dev(inp.bits["q"], inp.dtype)
    k = to_dev(inp.bits["k"], inp.dtype)
    v = to_dev(inp.bits["v"], inp.dtype)
    do = to_dev(inp.bits["do"], inp.dtype) if "do" in inp.bits else None
    return q, k, v, do


def sample_heads(B, H, n=3):
    """A few (b, h) pairs spread over the batch and head range (first, middle, last)."""
    pairs = [(0, 0), (B // 2, H // 2), (B - 1, H - 1)]
    out = []
    for p in pairs:
        if p not in out:
            out.append(p)
    return out[:n]
