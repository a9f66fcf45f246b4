"""Block-sparse forward against the float64 block-sparse oracle (same fp16/bf16 tolerances as the
dense forward), plus its reduction to the dense kernel on the same tile shape for an all-ones mask (bit for bit)."""
import math

import numpy as np
import pytest

import fattn_inputs as fi
from oracle import blocksparse as obs
from oracle import metrics as M
from tests.gpu_util import from_dev, log, sample_heads, upload

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_tiled_fattn_amd as fa
    return fa


def _check(o, lse, o_ref, lse_ref, dtype):
    tol = M.TOL[dtype]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), "rows without an allowed key differ"
    assert np.all(o[~fin] == 0)
    ea, er = M.max_abs(o, o_ref), M.max_rel(o, o_ref)
    el = M.max_abs(lse[fin], lse_ref[fin])
    log(f"    O max-abs {ea:.3e} max-rel {er:.3e}  LSE max-abs {el:.3e}  ({(~fin).sum()} empty rows)")
    assert np.all(np.isfinite(o))
    assert ea <= tol["o_abs"] and er <= tol["o_rel"] and el <= tol["lse_abs"], (ea, er, el)


def _run(inp, mask, causal):
    import torch
    q, k, v, _ = upload(inp)
    m = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    o, lse = _fa().forward_blocksparse(q, k, v, m, causal=causal)
    torch.cuda.synchronize()
    return from_dev(o), from_dev(lse)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [100, 300, 700])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density,diag", [(0.3, True), (0.6, False)])
def test_blocksparse_small_shapes(dtype, d, N, causal, density, diag):
    B, H = 1, 3
    nb = (N + 127) // 128
    log(f"blocksparse dtype={dtype} d={d} N={N} causal={causal} density={density} diag={diag}")
    inp = fi.make_inputs((B, H, N, d), dtype, 1000 + N)
    mask = fi.block_mask(B, H, nb, density, 1000 + N + d, diagonal=diag)
    o, lse = _run(inp, mask, causal)
    o_ref, lse_ref = obs.forward(inp.q, inp.k, inp.v, 1 / math.sqrt(d), mask, causal)
    _check(o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_all_ones_is_the_dense_kernel(d, causal):
    import torch
    fa = _fa()
    N = 777
    inp = fi.make_inputs((2, 2, N, d), "bf16", 1100 + d)
    q, k, v, _ = upload(inp)
    nb = (N + 127) // 128
    m = torch.ones((2, 2, nb, nb), dtype=torch.uint8, device="cuda")
    o1, l1 = fa.forward_blocksparse(q, k, v, m, causal=causal)
    o2, l2 = fa.forward(q, k, v, causal=causal, Br=128, Bc=64)  # the block-sparse path's tiles
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_blocksparse_empty_mask_and_single_block():
    import torch
    fa = _fa()
    N, d = 300, 128
    inp = fi.make_inputs((1, 1, N, d), "bf16", 1200)
    q, k, v, _ = upload(inp)
    m = torch.zeros((1, 1, 3, 3), dtype=torch.uint8, device="cuda")
    o, lse = fa.forward_blocksparse(q, k, v, m)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    m[0, 0, 2, 1] = 1  # only queries 256.. see keys 128..255
    o, lse = fa.forward_blocksparse(q, k, v, m)
    torch.cuda.synchronize()
    mask = m.cpu().numpy()
    o_ref, lse_ref = obs.forward(inp.q, inp.k, inp.v, 1 / math.sqrt(d), mask, False)
    _check(from_dev(o), from_dev(lse), o_ref, lse_ref, "bf16")


def test_blocksparse_workload5_shape_sampled_heads():
    w = fi.WORKLOADS[5]
    inp = fi.workload_inputs(5, with_do=False)
    nb = w.N // 128
    mask = fi.block_mask(w.B, w.H, nb, 0.25, 5)
    log("blocksparse B=2 H=16 N=4096 d=128 causal, density 0.25 + diagonal")
    o, lse = _run(inp, mask, True)
    heads = sample_heads(w.B, w.H)
    o_ref, lse_ref = obs.forward(inp.q, inp.k, inp.v, w.scale, mask, True, heads=heads)
    for b, h in heads:
        _check(o[b, h], lse[b, h], o_ref[b, h], lse_ref[b, h], "bf16")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
