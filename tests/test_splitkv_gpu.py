"""Split-KV forward parity (partials, merge, and the whole path) against the float64 oracle.

The HIP path is called through the C ABI (the thin binding); expected values come only from
``oracle.attention`` / ``oracle.splitkv`` on the generator's rounded inputs. Tolerances are the
fp16/bf16 ones of oracle.metrics (O max-abs 1e-2, per-slice max-rel 2e-2, LSE max-abs 1e-3);
the float32 merge of float32 partials is held to 1e-5.
"""
import math

import numpy as np
import pytest

import fattn_inputs as fi
from oracle import attention as att
from oracle import metrics as M
from oracle import splitkv as osk
from tests.gpu_util import from_dev, log, spread_heads, to_dev

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_tiled_fattn_amd as fa
    return fa


def _torch():
    import torch
    return torch


def _up(inp):
    return tuple(to_dev(inp.bits[n], inp.dtype) for n in ("q", "k", "v"))


def _check(o, lse, o_ref, lse_ref, dtype, o_abs=None, lse_abs=None):
    tol = M.TOL[dtype]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), "rows with no visible key differ"
    assert np.all(lse[~fin] == -np.inf)
    ea = M.max_abs(o, o_ref)
    er = M.max_rel(o, o_ref)
    el = M.max_abs(lse[fin], lse_ref[fin])
    log(f"    O max-abs {ea:.3e} max-rel {er:.3e}  LSE max-abs {el:.3e}")
    assert np.all(np.isfinite(o))
    assert ea <= (o_abs if o_abs is not None else tol["o_abs"]), ea
    if o_abs is None and tol["o_rel"] is not None:
        assert er <= tol["o_rel"], er
    assert el <= (lse_abs if lse_abs is not None else tol["lse_abs"]), el


def _splitkv(inp, causal, S, scale=None):
    fa = _fa()
    q, k, v = _up(inp)
    o, lse = fa.forward_splitkv(q, k, v, causal=causal, scale=scale, num_splits=S)
    _torch().cuda.synchronize()
    return from_dev(o), from_dev(lse)


# --------------------------------------------------------------------------------------------
# Whole path (partials + merge) on small shapes: one and several query tiles, ragged key ends,
# splits shorter than a tile, empty splits, Nq == Nk.


SHAPES = [(1, 1), (1, 63), (1, 300), (3, 129), (16, 1000), (33, 700), (40, 40), (5, 2000), (70, 70)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_small_shapes(dtype, d, nq, nk, causal):
    B, H = 1, 2
    inp = fi.make_decode_inputs(B, H, nq, nk, d, dtype, 600 + nq * 7 + nk)
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, scale, causal, causal_offset=nk - nq)
    for S in (1, 3, 8, 0):
        log(f"splitkv dtype={dtype} d={d} Nq={nq} Nk={nk} causal={causal} S={S}")
        o, lse = _splitkv(inp, causal, S)
        _check(o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nq,nk,S,causal", [(1, 300, 5, False), (16, 1000, 7, True), (33, 200, 16, True),
                                            (3, 129, 3, True), (40, 40, 2, True), (2, 64, 64, False)])
def test_partials_match_oracle_elementwise(dtype, nq, nk, S, causal):
    fa = _fa()
    d, B, H = 128, 2, 2
    log(f"partials dtype={dtype} Nq={nq} Nk={nk} S={S} causal={causal}")
    inp = fi.make_decode_inputs(B, H, nq, nk, d, dtype, 650 + S)
    scale = 1 / math.sqrt(d)
    q, k, v = _up(inp)
    op, lp = fa.forward_partial(q, k, v, S, causal=causal)
    _torch().cuda.synchronize()
    op, lp = from_dev(op), from_dev(lp)
    _, _, op_ref, lp_ref = osk.forward(inp.q, inp.k, inp.v, scale, S, causal)
    empty = ~np.isfinite(lp_ref)
    assert np.array_equal(~np.isfinite(lp), empty)
    assert np.all(op[empty] == 0.0)
    _check(op.reshape(-1, nq, d), lp.reshape(-1, nq), op_ref.reshape(-1, nq, d), lp_ref.reshape(-1, nq), dtype)


def test_combine_f32_matches_oracle_with_empty_partials():
    fa = _fa()
    torch = _torch()
    r = np.random.default_rng(np.random.SeedSequence([66, 1]))
    S, B, H, nq, d = 9, 2, 3, 5, 128
    op = r.standard_normal((S, B, H, nq, d)).astype(np.float32)
    lp = (r.standard_normal((S, B, H, nq)) * 20).astype(np.float32)
    drop = r.random((S, B, H, nq)) < 0.3
    lp[drop] = -np.inf
    op[drop] = np.nan  # never read: an empty partial's O is skipped
    lp[:, 0, 0, 0] = -np.inf  # a row with no key at all
    op_ok = np.where(drop[..., None], 0.0, op)
    o_ref, lse_ref = osk.combine(op_ok.astype(np.float64), lp.astype(np.float64))
    for dt, tol in ((torch.float32, 1e-5), (torch.bfloat16, 1e-2), (torch.float16, 1e-2)):
        log(f"combine out={dt}")
        o, lse = fa.combine(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(), dtype=dt)
        torch.cuda.synchronize()
        o, lse = from_dev(o), from_dev(lse)
        assert np.all(o[0, 0, 0] == 0) and lse[0, 0, 0] == -np.inf
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin)
        assert M.max_abs(o, o_ref) <= tol
        assert M.max_abs(lse[fin], lse_ref[fin]) <= 1e-5


# --------------------------------------------------------------------------------------------
# Page 3's worked example through the device merge, and numerically awkward inputs


def test_combine_worked_example_fifty_thirds():
    fa = _fa()
    torch = _torch()
    d = 64
    # two one-key partials of page 3: (O, LSE) = (10, 0) and (20, ln 2), every column alike
    op = np.zeros((2, 1, 1, 1, d), np.float32)
    op[0] = 10.0
    op[1] = 20.0
    lp = np.array([0.0, math.log(2.0)], np.float32).reshape(2, 1, 1, 1)
    o, lse = fa.combine(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda())
    torch.cuda.synchronize()
    o, lse = from_dev(o), from_dev(lse)
    assert np.max(np.abs(o - 50.0 / 3.0)) <= 1e-5
    assert abs(lse[0, 0, 0] - math.log(3.0)) <= 1e-6


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [0.0, -0.0883883, 0.5])
def test_splitkv_unusual_scales(dtype, scale):
    nq, nk, d = 4, 500, 128
    log(f"splitkv scale={scale} dtype={dtype}")
    inp = fi.make_decode_inputs(1, 2, nq, nk, d, dtype, 670)
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, scale, True, causal_offset=nk - nq)
    o, lse = _splitkv(inp, True, 5, scale=scale)
    # A sharp softmax makes rows of O close to single values (|O| up to ~4); rounding P and O to
    # 8 significant bits then costs about 2^-8 |O|, so the absolute bound is max(1e-2, 2^-7 max|O|),
    # as for the whole-row forward (max-rel unchanged).
    o_abs = max(M.TOL[dtype]["o_abs"], 2.0 ** -7 * float(np.max(np.abs(o_ref))))
    _check(o, lse, o_ref, lse_ref, dtype, o_abs=o_abs)
    assert M.max_rel(o, o_ref) <= M.TOL[dtype]["o_rel"]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_splitkv_plus_500_shift_stays_finite(dtype):
    # every logit raised by exactly 500 (Q[...,0] = 1, K[...,0] += 500 / scale): O unchanged,
    # LSE + 500 (page 1's stability example)
    nq, nk, d = 3, 400, 64
    scale = 1 / math.sqrt(d)
    base = fi.make_decode_inputs(1, 1, nq, nk, d, dtype, 671)
    q = base.q.copy()
    q[..., 0] = 1.0
    k = base.k.copy()
    k[..., 0] += np.float32(500.0 / scale)
    q, qb = fi.round_bits(q, dtype)
    k, kb = fi.round_bits(k, dtype)
    inp = fi.Inputs(dtype, q, k, base.v, None, {"q": qb, "k": kb, "v": base.bits["v"]})
    o_ref, lse_ref = att.forward(q, k, base.v, scale, False)
    log(f"splitkv +500 dtype={dtype}: oracle LSE around {lse_ref.mean():.1f}")
    o, lse = _splitkv(inp, False, 4)
    _check(o, lse, o_ref, lse_ref, dtype)


# --------------------------------------------------------------------------------------------
# Full-size decode workloads: one head from every XCD's head range against the oracle


@pytest.mark.parametrize("ident", sorted(fi.DECODE_WORKLOADS))
@pytest.mark.parametrize("causal", [False, True])
def test_decode_workloads_spread_heads(ident, causal):
    fa = _fa()
    w = fi.DECODE_WORKLOADS[ident]
    log(f"decode workload {ident} ({w.name}) causal={causal}")
    inp = fi.decode_workload_inputs(ident)
    q, k, v = _up(inp)
    o, lse = fa.forward_splitkv(q, k, v, causal=causal)
    _torch().cuda.synchronize()
    o, lse = from_dev(o), from_dev(lse)
    heads = spread_heads(w.B, w.H, 8) + [(1, 7)]
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, w.scale, causal, heads=heads,
                                 causal_offset=w.Nk - w.Nq)
    for b, h in heads:
        _check(o[b, h], lse[b, h], o_ref[b, h], lse_ref[b, h], w.dtype)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_splitkv_square_causal_matches_oracle():
    # Nq == Nk: the ordinary causal problem, computed with splits
    B, H, N, d = 1, 4, 1000, 128
    log("splitkv square causal N=1000")
    inp = fi.make_decode_inputs(B, H, N, N, d, "bf16", 672)
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, 1 / math.sqrt(d), True)
    o, lse = _splitkv(inp, True, 6)
    _check(o, lse, o_ref, lse_ref, "bf16")


def test_splitkv_huge_head_uses_64bit_addressing():
    # one head whose K and V are 2 GiB each (Nk * d * 2 >= 2^31): the 64-bit address path. K/V
    # repeat one 64-row block R times plus a 37-row tail, so the exact result is the merge of the
    # block's result taken R times (LSE + ln R, same O) with the tail's result.
    fa = _fa()
    torch = _torch()
    d, R, t = 128, (1 << 23) // 64, 37
    nk = 64 * R + t
    log(f"splitkv huge head Nk={nk}")
    blk = fi.make_decode_inputs(1, 1, 2, 64, d, "bf16", 673)
    scale = 1 / math.sqrt(d)
    qd, kb, vb = _up(blk)
    k = torch.cat([kb[0, 0].repeat(R, 1), kb[0, 0, :t]]).reshape(1, 1, nk, d)
    v = torch.cat([vb[0, 0].repeat(R, 1), vb[0, 0, :t]]).reshape(1, 1, nk, d)
    o, lse = fa.forward_splitkv(qd, k, v, causal=False, num_splits=64)
    torch.cuda.synchronize()
    o, lse = from_dev(o), from_dev(lse)
    del k, v
    q64, k64, v64 = (x[0, 0].astype(np.float64) for x in (blk.q, blk.k, blk.v))
    ob, lb = att.forward_slice(q64, k64, v64, scale)
    ot, lt = att.forward_slice(q64, k64[:t], v64[:t], scale)
    o_ref, lse_ref = osk.combine(np.stack([ob, ot]), np.stack([lb + math.log(R), lt]))
    _check(o[0, 0], lse[0, 0], o_ref, lse_ref, "bf16")


# --------------------------------------------------------------------------------------------
# Run-to-run determinism and streams


def test_splitkv_deterministic_and_on_side_stream():
    fa = _fa()
    torch = _torch()
    inp = fi.make_decode_inputs(2, 4, 16, 3000, 128, "bf16", 674)
    q, k, v = _up(inp)
    o1, l1 = fa.forward_splitkv(q, k, v, causal=True, num_splits=7)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = fa.forward_splitkv(q, k, v, causal=True, num_splits=7, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
