"""Dropout on P: device forward and backward against the float64 dropout oracle.

Both sides draw the keep mask from the same counter-based generator (16-bit field j % 8 of
Philox4x32-10 at counter (j / 8, i, b*H + h, 0) under the seed), so the comparison is element by
element with the usual fp16/bf16 tolerances (O max-abs 1e-2, per-slice max-rel 2e-2, LSE 1e-3,
gradients max-rel 5e-2), and the mask itself is checked exactly in the forward (through O), the
dK/dV kernel (through dV) and the dQ kernel (through dQ).
"""
import functools
import math

import numpy as np
import pytest

import fattn_inputs as fi
from oracle import dropout as odr
from oracle import metrics as M
from tests.gpu_util import from_dev, log, spread_heads, to_dev, upload

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_tiled_fattn_amd as fa
    return fa


def _check_fwd(o, lse, o_ref, lse_ref, dtype, o_abs=None):
    # Dropout scales the kept probabilities by 1 / (1 - p), so |O| can pass the range where the
    # 1e-2 bound covers rounding O and P to 16 bits; the derived bound for |O| >> 1 applies:
    # max(1e-2, 2^-7 max|O|), the cost of 8 significant bits.
    tol = M.TOL[dtype]
    if o_abs is None:
        o_abs = max(tol["o_abs"], 2.0 ** -7 * float(np.max(np.abs(o_ref))))
    ea, er, el = M.max_abs(o, o_ref), M.max_rel(o, o_ref), M.max_abs(lse, lse_ref)
    log(f"    O max-abs {ea:.3e} (bound {o_abs:.3e}) max-rel {er:.3e}  LSE max-abs {el:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert ea <= o_abs and er <= tol["o_rel"] and el <= tol["lse_abs"], (ea, er, el)


def _check_bwd(got, ref, dtype):
    errs = [M.max_rel(g, r) for g, r in zip(got, ref)]
    log(f"    dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e} (max-rel)")
    assert max(errs) <= M.TOL[dtype]["grad_rel"], errs


def _run(inp, causal, p, seed, backward=True):
    import torch
    fa = _fa()
    q, k, v, do = upload(inp)
    o, lse = fa.forward(q, k, v, causal=causal, p_drop=p, seed=seed)
    out = [o, lse]
    if backward:
        out += list(fa.backward(q, k, v, o, do, lse, causal=causal, p_drop=p, seed=seed))
    torch.cuda.synchronize()
    return [from_dev(x) for x in out]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [3, 65, 200, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_small_shapes(dtype, d, N, causal):
    p, seed = 0.2, 0x5EED0000 + N
    log(f"dropout dtype={dtype} d={d} N={N} causal={causal} p={p}")
    inp = fi.make_inputs((1, 2, N, d), dtype, 900 + N, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse, dq, dk, dv = _run(inp, causal, p, seed)
    o_ref, lse_ref = odr.forward(inp.q, inp.k, inp.v, scale, causal, p, seed)
    _check_fwd(o, lse, o_ref, lse_ref, dtype)
    ref = odr.backward(inp.q, inp.k, inp.v, inp.do, scale, causal, p, seed)
    _check_bwd((dq, dk, dv), ref, dtype)


@pytest.mark.parametrize("p", [0.05, 0.5, 0.9])
def test_dropout_mask_is_exact(p):
    # Q = 0 makes P uniform (1/N) and V = I makes O[i, j] = M[i, j] / (N (1 - p)): the device's
    # keep mask shows up exactly, compared with the oracle's mask bit for bit
    import torch
    fa = _fa()
    N = d = 128
    B, H = 2, 3
    seed = 2**40 + 12345
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    v = torch.eye(N, dtype=torch.bfloat16, device="cuda").expand(B, H, N, N).contiguous()
    log(f"dropout mask p={p}")
    o, _ = fa.forward(q, k, v, causal=False, p_drop=p, seed=seed)
    torch.cuda.synchronize()
    got = from_dev(o) > 0
    for b in range(B):
        for h in range(H):
            want = odr.keep_mask(seed, p, b * H + h, np.arange(N), np.arange(N))
            assert np.array_equal(got[b, h], want), (b, h)
    rate = got.mean()
    log(f"    keep rate {rate:.4f} (1 - p = {1 - p:.4f})")
    assert abs(rate - (1 - p)) < 5 * math.sqrt(p * (1 - p) / got.size)


@pytest.mark.parametrize("p", [0.05, 0.5, 0.9])
def test_dropout_backward_mask_is_exact_in_dv(p):
    # Q = 0 makes P uniform (1/N) and dO = I makes dV = Pd^T dO = Pd^T: dV[j, i] =
    # M[i, j] / (N (1 - p)), so the dK/dV kernel's keep mask shows up exactly
    import torch
    fa = _fa()
    N = d = 128
    B, H = 2, 3
    seed = 2**41 + 777
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    v = torch.randn(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    do = torch.eye(N, dtype=torch.bfloat16, device="cuda").expand(B, H, N, N).contiguous()
    log(f"dropout backward mask (dV) p={p}")
    o, lse = fa.forward(q, k, v, causal=False, p_drop=p, seed=seed)
    _, _, dv = fa.backward(q, k, v, o, do, lse, causal=False, p_drop=p, seed=seed)
    torch.cuda.synchronize()
    got = np.swapaxes(from_dev(dv), -1, -2) > 0
    for b in range(B):
        for h in range(H):
            want = odr.keep_mask(seed, p, b * H + h, np.arange(N), np.arange(N))
            assert np.array_equal(got[b, h], want), (b, h)


@pytest.mark.parametrize("p", [0.3, 0.5, 0.9])
def test_dropout_backward_mask_is_exact_in_dq(p):
    # Q = 0 (P = 1/N), K = V = I and dO = 1: dP = M / (1 - p), D_i = kept_i / (N (1 - p)) and
    # dQ = scale dS K = (scale / N) (M / (1 - p) - D): kept entries are >= (scale / N) p / (1 - p)
    # up to rounding, dropped ones about -(scale / N), so the sign of dQ is the dQ kernel's mask
    import torch
    fa = _fa()
    N = d = 128
    B, H = 2, 3
    seed = 2**42 + 31337
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    eye = torch.eye(N, dtype=torch.bfloat16, device="cuda").expand(B, H, N, N).contiguous()
    do = torch.ones(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    log(f"dropout backward mask (dQ) p={p}")
    o, lse = fa.forward(q, eye, eye, causal=False, p_drop=p, seed=seed)
    dq, _, _ = fa.backward(q, eye, eye, o, do, lse, causal=False, p_drop=p, seed=seed)
    torch.cuda.synchronize()
    got = from_dev(dq) > 0
    for b in range(B):
        for h in range(H):
            want = odr.keep_mask(seed, p, b * H + h, np.arange(N), np.arange(N))
            assert np.array_equal(got[b, h], want), (b, h)


def test_dropout_p_zero_is_the_plain_path_and_seeds_matter():
    import torch
    fa = _fa()
    inp = fi.make_inputs((1, 2, 300, 128), "bf16", 950, with_do=True)
    q, k, v, do = upload(inp)
    o0, l0 = fa.forward(q, k, v, causal=True)
    o1, l1 = fa.forward(q, k, v, causal=True, p_drop=0.0, seed=99)
    a = fa.forward(q, k, v, causal=True, p_drop=0.3, seed=7)
    b = fa.forward(q, k, v, causal=True, p_drop=0.3, seed=7)
    c = fa.forward(q, k, v, causal=True, p_drop=0.3, seed=8)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0])
    assert torch.equal(a[1], l0)  # LSE is the undropped statistic


@functools.lru_cache(maxsize=1)
def _workload5():
    return fi.workload_inputs(5)


def test_dropout_workload5_spread_heads():
    w = fi.WORKLOADS[5]
    inp = _workload5()
    p, seed = 0.1, 20261202
    log("dropout workload 5 (B=2 H=16 N=4096 d=128 causal, p=0.1)")
    o, lse, dq, dk, dv = _run(inp, True, p, seed)
    heads = spread_heads(w.B, w.H, 8)
    o_ref, lse_ref = odr.forward(inp.q, inp.k, inp.v, w.scale, True, p, seed, heads=heads)
    ref = odr.backward(inp.q, inp.k, inp.v, inp.do, w.scale, True, p, seed, heads=heads)
    for b, h in heads:
        _check_fwd(o[b, h], lse[b, h], o_ref[b, h], lse_ref[b, h], "bf16")
        _check_bwd((dq[b, h], dk[b, h], dv[b, h]), tuple(r[b, h] for r in ref), "bf16")
