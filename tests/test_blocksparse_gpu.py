"""Block-sparse forward and backward against the float64 block-sparse oracle (the dense path's
fp16/bf16 tolerances: O max-abs 1e-2 and max-rel 2e-2, LSE 1e-3, gradients max-rel 5e-2), plus
their reductions to the dense kernels for an all-ones mask (bit for bit)."""
import math

import numpy as np
import pytest

import fattn_inputs as fi
from oracle import blocksparse as obs
from oracle import metrics as M
from tests.gpu_util import from_dev, log, spread_heads, upload

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


def _tilted(N, d, seed, kind):
    """bf16 inputs whose logits get a large per-key offset through Q[..., 0] = 1 and K[..., 0]:
    'rising' adds 0.04 per key, 'alternate' adds 30 to the keys of every other 64-key tile. Either
    way the running maximum outgrows the forward's slack on many of the tiles a row visits, so the
    rescale path runs between skipped and visited tiles."""
    inp = fi.make_inputs((1, 2, N, d), "bf16", seed)
    scale = 1 / math.sqrt(d)
    q, k = inp.q.copy(), inp.k.copy()
    q[..., 0] = 1.0
    j = np.arange(N, dtype=np.float32)
    off = 0.04 * j if kind == "rising" else 30.0 * ((np.arange(N) // 64) % 2).astype(np.float32)
    k[..., 0] = off / np.float32(scale)
    q, qb = fi.round_bits(q, "bf16")
    k, kb = fi.round_bits(k, "bf16")
    bits = dict(inp.bits)
    bits["q"], bits["k"] = qb, kb
    return fi.Inputs("bf16", q, k, inp.v, None, bits), scale


@pytest.mark.parametrize("kind", ["rising", "alternate"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [1.0, 0.5])
def test_blocksparse_tilted_logits(kind, causal, density):
    N, d = 1000, 128
    log(f"blocksparse tilted logits kind={kind} causal={causal} density={density}")
    inp, scale = _tilted(N, d, 1300, kind)
    nb = (N + 127) // 128
    mask = fi.block_mask(1, 2, nb, density, 1301, diagonal=True)
    o, lse = _run(inp, mask, causal)
    o_ref, lse_ref = obs.forward(inp.q, inp.k, inp.v, scale, mask, causal)
    _check(o, lse, o_ref, lse_ref, "bf16")


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


def test_blocksparse_workload5_shape_spread_heads():
    w = fi.WORKLOADS[5]
    inp = fi.workload_inputs(5, with_do=False)
    nb = w.N // 128
    mask = fi.block_mask(w.B, w.H, nb, 0.25, 5)
    log("blocksparse B=2 H=16 N=4096 d=128 causal, density 0.25 + diagonal")
    o, lse = _run(inp, mask, True)
    heads = spread_heads(w.B, w.H, 8)
    o_ref, lse_ref = obs.forward(inp.q, inp.k, inp.v, w.scale, mask, True, heads=heads)
    for b, h in heads:
        _check(o[b, h], lse[b, h], o_ref[b, h], lse_ref[b, h], "bf16")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ---------------------------------------------------------------------------------------------
# Backward


def _check_grads(got, ref, dtype, empty_rows=None):
    tol = M.TOL[dtype]["grad_rel"]
    floor = 1e-3 * max(float(np.max(np.abs(r))) for r in ref)
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        er = M.max_rel(x, r, floor=floor)
        log(f"    {name} max-rel {er:.3e} max-abs {M.max_abs(x, r):.3e}")
        assert np.all(np.isfinite(x)), name
        assert er <= tol, (name, er)
    if empty_rows is not None:
        assert np.all(got[0][empty_rows] == 0), "dQ of rows without an allowed key"


def _run_bwd(inp, mask, causal):
    import torch
    fa = _fa()
    q, k, v, do = upload(inp)
    m = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    o, lse = fa.forward_blocksparse(q, k, v, m, causal=causal)
    dq, dk, dv = fa.backward_blocksparse(q, k, v, o, do, lse, m, causal=causal)
    torch.cuda.synchronize()
    return from_dev(dq), from_dev(dk), from_dev(dv), from_dev(lse)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [100, 300, 700])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density,diag", [(0.3, True), (0.6, False)])
def test_blocksparse_backward_small_shapes(dtype, d, N, causal, density, diag):
    B, H = 1, 3
    nb = (N + 127) // 128
    log(f"blocksparse bwd dtype={dtype} d={d} N={N} causal={causal} density={density} diag={diag}")
    inp = fi.make_inputs((B, H, N, d), dtype, 1300 + N, with_do=True)
    mask = fi.block_mask(B, H, nb, density, 1300 + N + d, diagonal=diag)
    dq, dk, dv, lse = _run_bwd(inp, mask, causal)
    ref = obs.backward(inp.q, inp.k, inp.v, inp.do, 1 / math.sqrt(d), mask, causal)
    _check_grads((dq, dk, dv), ref, dtype, empty_rows=~np.isfinite(lse))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_backward_all_ones_is_the_dense_backward(d, causal):
    import torch
    fa = _fa()
    N = 777
    inp = fi.make_inputs((2, 2, N, d), "bf16", 1400 + d, with_do=True)
    q, k, v, do = upload(inp)
    nb = (N + 127) // 128
    m = torch.ones((2, 2, nb, nb), dtype=torch.uint8, device="cuda")
    o, lse = fa.forward(q, k, v, causal=causal)
    g1 = fa.backward_blocksparse(q, k, v, o, do, lse, m, causal=causal)
    g2 = fa.backward(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_blocksparse_backward_empty_mask_and_single_block():
    import torch
    fa = _fa()
    N, d = 300, 128
    inp = fi.make_inputs((1, 1, N, d), "bf16", 1500, with_do=True)
    q, k, v, do = upload(inp)
    m = torch.zeros((1, 1, 3, 3), dtype=torch.uint8, device="cuda")
    o, lse = fa.forward_blocksparse(q, k, v, m)
    g = fa.backward_blocksparse(q, k, v, o, do, lse, m)
    torch.cuda.synchronize()
    assert all(torch.all(x == 0) for x in g)
    m[0, 0, 2, 1] = 1  # only queries 256.. see keys 128..255
    mask = m.cpu().numpy()
    dq, dk, dv, lse = _run_bwd(inp, mask, False)
    ref = obs.backward(inp.q, inp.k, inp.v, inp.do, 1 / math.sqrt(d), mask, False)
    _check_grads((dq, dk, dv), ref, "bf16", empty_rows=~np.isfinite(lse))
    assert np.all(dk[0, 0, :128] == 0) and np.all(dk[0, 0, 256:] == 0)


def test_blocksparse_backward_workload5_shape_spread_heads():
    w = fi.WORKLOADS[5]
    inp = fi.workload_inputs(5)
    nb = w.N // 128
    mask = fi.block_mask(w.B, w.H, nb, 0.25, 5)
    log("blocksparse bwd B=2 H=16 N=4096 d=128 causal, density 0.25 + diagonal")
    dq, dk, dv, _ = _run_bwd(inp, mask, True)
    heads = spread_heads(w.B, w.H, 8)
    ref = obs.backward(inp.q, inp.k, inp.v, inp.do, w.scale, mask, True, heads=heads)
    for b, h in heads:
        _check_grads((dq[b, h], dk[b, h], dv[b, h]), tuple(r[b, h] for r in ref), "bf16")
