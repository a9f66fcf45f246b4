"""Shared helpers for the GPU tests: upload the generator's exact bits, fetch results as float64."""
import math
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


def spread_heads(B, H, n=8):
    """n (b, h) pairs, one from each of n evenly spaced ranges of the B*H heads, at a different
    offset inside each range. With n = 8 that is one head from every XCD's contiguous head range
    (the kernels deal heads to the 8 XCDs in contiguous ranges)."""
    bh_total = B * H
    n = min(n, bh_total)
    per = bh_total // n
    out = []
    for x in range(n):
        bh = x * per + (x % per if per else 0)
        out.append((bh // H, bh % H))
    return out


def every_head(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


_SENTINEL = {1: 0x5A, 2: 0x7E5A, 4: 0x7FC0DEAD}  # bit patterns no kernel output here can take


class Guarded:
    """A contiguous device tensor of ``shape`` placed inside a larger buffer, with ``guard``
    elements before and after it. The guards and the tensor itself start out holding a fixed bit
    pattern; ``check()`` asserts that the guards are unchanged (nothing was written past either
    end) and, with ``written``, that no element of the tensor still holds the pattern (every
    element was written)."""

    def __init__(self, shape, dtype, guard=4096, device="cuda"):
        import torch
        self.shape, self.guard = tuple(shape), guard
        n = math.prod(self.shape)
        self.buf = torch.empty(n + 2 * guard, dtype=dtype, device=device)
        size = self.buf.element_size()
        self.ints = self.buf.view({1: torch.int8, 2: torch.int16, 4: torch.int32}[size])
        pat = _SENTINEL[size]
        self.pat = pat - (1 << (8 * size)) if pat >= 1 << (8 * size - 1) else pat
        self.ints.fill_(self.pat)
        self.t = self.buf[guard: guard + n].view(self.shape)

    def check(self, written=True, name="tensor"):
        g = self.guard
        before = self.ints[:g]
        after = self.ints[g + self.t.numel():]
        assert bool((before == self.pat).all()), f"{name}: written before its start"
        assert bool((after == self.pat).all()), f"{name}: written past its end"
        if written and self.t.numel():
            inner = self.ints[g: g + self.t.numel()]
            assert not bool((inner == self.pat).any()), f"{name}: elements left unwritten"
