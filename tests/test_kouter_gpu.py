"""K-outer (FA-1 order) forward ablation: parity with the float64 oracle through the C ABI.

The ablation computes the same attention as fattn_fwd with the loop order swapped, so it is held
to the same tolerances (fp16/bf16: O max-abs 1e-2, per-slice max-rel 2e-2, LSE max-abs 1e-3).
"""
import functools
import math

import numpy as np
import pytest

import fattn_inputs as fi
from oracle import attention as att
from oracle import metrics as M
from tests.gpu_util import from_dev, log, spread_heads, upload

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_tiled_fattn_amd as fa
    return fa


def _check(o, lse, o_ref, lse_ref, dtype):
    tol = M.TOL[dtype]
    ea, er, el = M.max_abs(o, o_ref), M.max_rel(o, o_ref), M.max_abs(lse, lse_ref)
    log(f"    O max-abs {ea:.3e} max-rel {er:.3e}  LSE max-abs {el:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert ea <= tol["o_abs"] and er <= tol["o_rel"] and el <= tol["lse_abs"], (ea, er, el)


def _run(inp, causal, scale=None):
    import torch
    q, k, v, _ = upload(inp)
    o, lse = _fa().forward_kouter(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return from_dev(o), from_dev(lse)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 3, 65, 129, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_kouter_small_shapes(dtype, d, N, causal):
    log(f"kouter dtype={dtype} d={d} N={N} causal={causal}")
    inp = fi.make_inputs((1, 2, N, d), dtype, 800 + N)
    o, lse = _run(inp, causal)
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, 1 / math.sqrt(d), causal)
    _check(o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_kouter_unusual_scales(scale):
    inp = fi.make_inputs((1, 2, 300, 64), "bf16", 810)
    for causal in (False, True):
        log(f"kouter scale={scale} causal={causal}")
        o, lse = _run(inp, causal, scale=scale)
        o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, scale, causal)
        _check(o, lse, o_ref, lse_ref, "bf16")


@functools.lru_cache(maxsize=1)
def _workload3():
    return fi.workload_inputs(3)


def test_kouter_workload3_sampled_heads_and_agrees_with_fattn_fwd():
    import torch
    fa = _fa()
    w = fi.WORKLOADS[3]
    inp = _workload3()
    log("kouter workload 3 (B=4 H=16 N=4096 d=128 causal)")
    q, k, v, _ = upload(inp)
    o, lse = fa.forward_kouter(q, k, v, causal=True)
    o2, lse2 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    o, lse, o2, lse2 = (from_dev(x) for x in (o, lse, o2, lse2))
    heads = spread_heads(w.B, w.H, 8)
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, w.scale, True, heads=heads)
    for b, h in heads:
        _check(o[b, h], lse[b, h], o_ref[b, h], lse_ref[b, h], "bf16")
    # every head: the two loop orders agree to within the rounding of the 16-bit output
    assert M.max_abs(o, o2) <= 1e-2 and M.max_abs(lse, lse2) <= 1e-3


def test_kouter_deterministic():
    import torch
    fa = _fa()
    inp = fi.make_inputs((2, 2, 700, 128), "bf16", 811)
    q, k, v, _ = upload(inp)
    a = fa.forward_kouter(q, k, v, causal=True)
    b = fa.forward_kouter(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
