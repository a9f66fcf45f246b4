"""Every output is written exactly within its bounds (GPU).

O, LSE, dQ, dK, dV and the backward's D workspace are placed inside larger buffers whose guard
bands hold a fixed bit pattern; after the call the guards must be untouched and every element of
the output must have been written. The shapes end in ragged tiles (N = 1, 65, 129, 1000) at both
head dimensions, where an off-by-one in a tail tile would show (page "从零实现 FlashAttention-2",
tips: edge tiles are handled explicitly). The values are checked against the oracle as well.
"""
import math

import numpy as np
import pytest

import fattn_inputs as fi
from oracle import attention as att
from oracle import metrics as M
from tests.gpu_util import Guarded, from_dev, log, upload

pytestmark = pytest.mark.gpu

NS = [1, 65, 129, 1000]


def _fa():
    import io_aware_tiled_fattn_amd as fa
    fa.lib()
    return fa


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("causal", [False, True])
def test_forward_writes_exactly_o_and_lse(dtype, d, N, causal):
    import torch
    fa = _fa()
    log(f"guard fwd dtype={dtype} d={d} N={N} causal={causal}")
    B, H = 2, 3
    inp = fi.make_inputs((B, H, N, d), dtype, 900 + N + d, with_do=False)
    q, k, v, _ = upload(inp)
    go = Guarded((B, H, N, d), q.dtype)
    gl = Guarded((B, H, N), torch.float32)
    fa.forward(q, k, v, causal=causal, out=go.t, lse=gl.t)
    torch.cuda.synchronize()
    go.check(name="O")
    gl.check(name="LSE")
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, 1 / math.sqrt(d), causal)
    tol = M.TOL[dtype]
    assert M.max_abs(from_dev(go.t), o_ref) <= tol["o_abs"]
    assert M.max_abs(from_dev(gl.t), lse_ref) <= tol["lse_abs"]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", NS)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_writes_exactly_dq_dk_dv_and_d(dtype, d, N, causal):
    import torch
    fa = _fa()
    log(f"guard bwd dtype={dtype} d={d} N={N} causal={causal}")
    B, H = 2, 3
    scale = 1 / math.sqrt(d)
    inp = fi.make_inputs((B, H, N, d), dtype, 950 + N + d, with_do=True)
    q, k, v, do = upload(inp)
    o, lse = fa.forward(q, k, v, causal=causal)
    grads = [Guarded((B, H, N, d), q.dtype) for _ in range(3)]
    need = fa.fattn_bwd_workspace_size(B, H, N, d, fa.dtype_code(q))
    assert need >= 4 * B * H * N
    gw = Guarded((need,), torch.uint8)
    fa.backward(q, k, v, o, do, lse, causal=causal, workspace=gw.t, dq=grads[0].t, dk=grads[1].t, dv=grads[2].t)
    torch.cuda.synchronize()
    for g, name in zip(grads, ("dQ", "dK", "dV")):
        g.check(name=name)
    # the D vector occupies the first 4 B H N bytes of the workspace; the rest is padding
    gw.check(written=False, name="workspace")
    dvec = gw.t[: 4 * B * H * N].view(torch.float32)
    assert bool(torch.isfinite(dvec).all())
    ref = att.backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
    floor = 1e-3 * max(float(np.max(np.abs(r))) for r in ref)
    for g, r, name in zip(grads, ref, ("dQ", "dK", "dV")):
        assert M.max_rel(from_dev(g.t), r, floor=floor) <= M.TOL[dtype]["grad_rel"], name


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 1000), (16, 129), (37, 65)])
def test_splitkv_writes_exactly_o_and_lse(Nq, Nk):
    import torch
    fa = _fa()
    log(f"guard split-KV Nq={Nq} Nk={Nk}")
    B, H, d = 2, 3, 128
    inp = fi.make_decode_inputs(B, H, Nq, Nk, d, "bf16", 980 + Nq + Nk)
    q, k, v, _ = upload(inp)
    go = Guarded((B, H, Nq, d), q.dtype)
    gl = Guarded((B, H, Nq), torch.float32)
    S = 3
    gw = Guarded((fa.fattn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, S),), torch.uint8)
    fa.forward_splitkv(q, k, v, causal=True, num_splits=S, out=go.t, lse=gl.t, workspace=gw.t)
    torch.cuda.synchronize()
    go.check(name="O")
    gl.check(name="LSE")
    gw.check(written=False, name="workspace")
    o_ref, lse_ref = att.forward(inp.q, inp.k, inp.v, 1 / math.sqrt(d), True, causal_offset=Nk - Nq)
    assert M.max_abs(from_dev(go.t), o_ref) <= 1e-2
    assert M.max_abs(from_dev(gl.t), lse_ref) <= 1e-3
