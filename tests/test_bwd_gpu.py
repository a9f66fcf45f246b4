"""Backward parity of the HIP path (fattn_fwd then fattn_bwd through the C ABI) against the
float64 oracle's analytic backward on the same rounded Q, K, V, dO.

The device backward consumes the device forward's O (rounded to the storage type) and LSE, as a
training step would; the oracle recomputes everything in float64 from Q, K, V, dO alone. The
bar is the per-(b, h)-slice max-rel of dQ, dK, dV <= 5e-2 (oracle.metrics.TOL).
"""
import functools
import math

import numpy as np
import pytest

import fattn_inputs as fi
from oracle import attention as att
from oracle import metrics as M
from tests.gpu_util import Guarded, every_head, from_dev, log, upload
from tests.periodic import block_problem as _block_problem

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_tiled_fattn_amd as fa
    return fa


def _run(inp, causal, scale=None):
    import torch
    fa = _fa()
    q, k, v, do = upload(inp)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return from_dev(dq), from_dev(dk), from_dev(dv)


def _check(got, ref, dtype):
    tol = M.TOL[dtype]["grad_rel"]
    # A gradient that is identically zero in exact arithmetic (dQ, dK when a row has one key)
    # comes back as rounding noise; measure it against 1e-3 of the problem's largest gradient.
    floor = 1e-3 * max(float(np.max(np.abs(r))) for r in ref)
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        er = M.max_rel(x, r, floor=floor)
        log(f"    {name} max-rel {er:.3e} max-abs {M.max_abs(x, r):.3e} rel-l2 {M.rel_l2(x, r):.3e}")
        assert np.all(np.isfinite(x)), name
        assert er <= tol, (name, er)


@pytest.mark.parametrize("B,H", [(3, 16), (5, 8)])
def test_backward_causal_order_with_a_partial_head_group(B, H):
    # causal work-groups of an XCD run four heads at a time; 6 and 5 heads per XCD leave a last
    # group of 2 and 1: every head must still get each of its tiles exactly once
    log(f"bwd partial head group B={B} H={H}")
    inp = fi.make_inputs((B, H, 300, 128), "bf16", 231, with_do=True)
    scale = 1 / math.sqrt(128)
    got = _run(inp, True)
    ref = att.backward(inp.q, inp.k, inp.v, inp.do, scale, True)
    _check(got, ref, "bf16")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 3, 65, 100, 129, 257, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small_shapes(dtype, d, N, causal):
    log(f"bwd small dtype={dtype} d={d} N={N} causal={causal}")
    inp = fi.make_inputs((1, 2, N, d), dtype, 200 + N, with_do=True)
    scale = 1 / math.sqrt(d)
    got = _run(inp, causal)
    ref = att.backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
    _check(got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [0.0, -0.15])
def test_backward_unusual_scales(dtype, scale):
    inp = fi.make_inputs((2, 2, 190, 64), dtype, 21, with_do=True)
    for causal in (False, True):
        got = _run(inp, causal, scale=scale)
        ref = att.backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
        if scale == 0.0:
            # dQ = dK = 0 exactly in math (scale multiplies both); compare dV only and check
            # the others vanish
            assert np.all(got[0] == 0) and np.all(got[1] == 0)
            assert M.max_rel(got[2], ref[2]) <= M.TOL[dtype]["grad_rel"]
        else:
            _check(got, ref, dtype)


@functools.lru_cache(maxsize=1)
def _workload5():
    return fi.workload_inputs(5)


def test_workload5_backward_every_head():
    # every (b, h) slice of dQ, dK and dV compared element by element with the oracle
    w = fi.WORKLOADS[5]
    inp = _workload5()
    got = _run(inp, True)
    heads = every_head(w.B, w.H)
    ref = att.backward(inp.q, inp.k, inp.v, inp.do, w.scale, True, heads=heads)
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        log(f"    {name}: max-rel over {len(heads)} heads {M.max_rel(x, r):.3e}, rel-l2 {M.rel_l2(x, r):.3e}")
    _check(got, ref, "bf16")


def test_workload5_gradient_identities_every_head():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i hold for every head (exact in math)."""
    w = fi.WORKLOADS[5]
    inp = _workload5()
    dq, dk, dv = _run(inp, True)
    do = inp.do.astype(np.float64)
    sdk = np.abs(dk.sum(axis=2))
    sdv = np.abs(dv.sum(axis=2) - do.sum(axis=2))
    # The device rounds P, dS and O to bf16 (2^-9 relative) before they enter sums over N terms;
    # bound the identity residual by 2^-6 of the sum of the magnitudes it cancels.
    bk = 2.0 ** -6 * np.abs(dk).sum(axis=2) + 1e-3
    bv = 2.0 ** -6 * (np.abs(dv).sum(axis=2) + np.abs(do).sum(axis=2)) + 1e-3
    log(f"    max |sum dK| {sdk.max():.3e} (bound {bk.min():.3e}); max |sum dV - sum dO| {sdv.max():.3e}")
    assert np.all(sdk <= bk)
    assert np.all(sdv <= bv)


def test_backward_deterministic():
    import torch
    fa = _fa()
    inp = fi.make_inputs((2, 4, 1000, 128), "bf16", 22, with_do=True)
    q, k, v, do = upload(inp)
    o, lse = fa.forward(q, k, v, causal=True)
    a = fa.backward(q, k, v, o, do, lse, causal=True)
    b = fa.backward(q, k, v, o, do, lse, causal=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_causal_prefix_invariance():
    """Gradients w.r.t. Q[0..i] do not depend on K, V rows after i (causal)."""
    import torch
    fa = _fa()
    inp = fi.make_inputs((1, 2, 600, 64), "bf16", 23, with_do=True)
    other = fi.make_inputs((1, 2, 600, 64), "bf16", 24)
    q, k, v, do = upload(inp)
    _, ko, vo, _ = upload(other)
    cut = 250
    o, lse = fa.forward(q, k, v, causal=True)
    dq1, _, _ = fa.backward(q, k, v, o, do, lse, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, cut + 1:] = ko[:, :, cut + 1:]
    v2[:, :, cut + 1:] = vo[:, :, cut + 1:]
    o2, lse2 = fa.forward(q, k2, v2, causal=True)
    dq2, _, _ = fa.backward(q, k2, v2, o2, do, lse2, causal=True)
    assert torch.equal(dq1[:, :, : cut + 1], dq2[:, :, : cut + 1])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [100, 300])
def test_backward_stage_entry_points_match_fattn_bwd(causal, N):
    """preprocess, dK/dV and dQ called one by one give fattn_bwd's results bit for bit."""
    import torch
    fa = _fa()
    inp = fi.make_inputs((1, 3, N, 128), "bf16", 31 + N, with_do=True)
    q, k, v, do = upload(inp)
    o, lse = fa.forward(q, k, v, causal=causal)
    ref = fa.backward(q, k, v, o, do, lse, causal=causal)
    dvec = torch.empty(1 * 3 * N, dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.backward_stages(q, k, v, o, do, lse, dq, dk, dv, dvec, causal=causal, stages=(0, 1, 2))
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x, y)


# --------------------------------------------------------------------------------------------
# A head of 2 GiB or more: the backward's 64-bit address path


@pytest.mark.timeout(900)
def test_backward_huge_head_uses_64bit_addressing():
    # One causal bf16 head of N = 64 R + 37 rows (Q, K, V, dO repeat one 64-row block), so that
    # N d 2 >= 2^31 bytes: the dK/dV and dQ kernels take 64-bit addresses, with a ragged last
    # tile. Exact gradients follow from small oracle problems (_block_problem): dQ for every row
    # of blocks 0, 1, R/2, R-1 and the tail, dK and dV for every key of the last two blocks (keys
    # of block c are seen by query blocks c .. R, so only blocks R-1 and R contribute there).
    import torch
    fa = _fa()
    d, t = 128, 37
    R = (1 << 23) // 64 + 1
    N = 64 * R + t
    assert N * d * 2 >= 1 << 31
    scale = 1 / math.sqrt(d)
    blk = fi.make_inputs((1, 1, 64, d), "bf16", 678, with_do=True)
    qb, kb, vb, dob = upload(blk)
    reps = lambda x: torch.cat([x[0, 0].repeat(R, 1), x[0, 0, :t]]).reshape(1, 1, N, d)
    q, k, v, do = reps(qb), reps(kb), reps(vb), reps(dob)
    log(f"backward huge head N={N}: forward")
    o, lse = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    log("  backward")
    gq, gk, gv = (Guarded((1, 1, N, d), torch.bfloat16) for _ in range(3))
    fa.backward(q, k, v, o, do, lse, causal=True, dq=gq.t, dk=gk.t, dv=gv.t)
    torch.cuda.synchronize()
    log("  checks")
    for g, name in ((gq, "dQ"), (gk, "dK"), (gv, "dV")):
        g.check(name=name)
    # exact identities over the whole head: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i
    dk_sum = gk.t[0, 0].double().sum(0)
    dv_sum = gv.t[0, 0].double().sum(0) - do[0, 0].double().sum(0)
    bk = 2.0 ** -6 * gk.t[0, 0].double().abs().sum(0) + 1e-3
    bv = 2.0 ** -6 * (gv.t[0, 0].double().abs().sum(0) + do[0, 0].double().abs().sum(0)) + 1e-3
    assert bool((dk_sum.abs() <= bk).all()) and bool((dv_sum.abs() <= bv).all())
    q64, k64, v64, do64 = (x[0, 0].astype(np.float64) for x in (blk.q, blk.k, blk.v, blk.do))
    rows = lambda g, c, n: from_dev(g.t[0, 0, 64 * c: 64 * c + n])
    ref_q, got_q = [], []
    for c in (0, 1, R // 2, R - 1, R):
        nr = 64 if c < R else t
        ref_q.append(_block_problem(q64, k64, v64, do64, scale, c, nr)[0])
        got_q.append(rows(gq, c, nr))
    # keys of block R - 1: its own query block (diagonal part) and the tail block (folded keys)
    _, _, _, dk_own, dv_own = _block_problem(q64, k64, v64, do64, scale, R - 1, 64)
    _, dk_fold, dv_fold, dk_tail, dv_tail = _block_problem(q64, k64, v64, do64, scale, R, t)
    ref_k = np.concatenate([dk_own + dk_fold, dk_tail])
    ref_v = np.concatenate([dv_own + dv_fold, dv_tail])
    got_k = np.concatenate([rows(gk, R - 1, 64), rows(gk, R, t)])
    got_v = np.concatenate([rows(gv, R - 1, 64), rows(gv, R, t)])
    got = (np.concatenate(got_q)[None], got_k[None], got_v[None])
    ref = (np.concatenate(ref_q)[None], ref_k[None], ref_v[None])
    _check(got, ref, "bf16")
