"""The library's entry points under HIP graph capture (torch.cuda.CUDAGraph), against eager calls.

Every entry point only checks its arguments on the host and launches kernels on the given stream
(no allocation, memset or synchronisation), so a caller can capture it. Each test captures one
call sequence on static buffers, then three times: writes new seeded inputs into those buffers,
runs the same sequence eagerly into separate outputs, synchronises, replays the graph, and
requires every replayed output to equal the eager one bit for bit (the kernels are
deterministic). A graph keeps the arguments it was captured with: the dropout seed included.
"""
import numpy as np
import pytest

import fattn_inputs as fi
from tests.gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_tiled_fattn_amd as fa
    fa.lib()
    return fa


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # one eager run on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _refill(static, shape, dtype, seed):
    """Write a fresh seeded problem (the generator's bits) into the static input tensors."""
    inp = fi.make_inputs(shape, dtype, seed, with_do=True)
    for name, t in static.items():
        t.copy_(to_dev(inp.bits[name], dtype))


def _same(name, replayed, eager):
    import torch
    assert torch.equal(replayed, eager), f"{name}: replay differs from the eager call"


@pytest.mark.parametrize("causal", [True, False])
def test_training_step_graph_replays_match_eager(causal):
    import torch
    fa = _fa()
    shape, dtype = (2, 4, 1000, 128), "bf16"
    B, H, N, d = shape
    log(f"graph: training step B={B} H={H} N={N} d={d} {dtype} causal={causal}")
    z = lambda: torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    st = {"q": z(), "k": z(), "v": z(), "do": z()}
    o, dq, dk, dv = z(), z(), z(), z()
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fattn_bwd_workspace_size(B, H, N, d, fa.FATTN_BF16), dtype=torch.uint8, device="cuda")

    def step():
        fa.forward(st["q"], st["k"], st["v"], causal=causal, out=o, lse=lse)
        fa.backward(st["q"], st["k"], st["v"], o, st["do"], lse, causal=causal, workspace=ws, dq=dq, dk=dk, dv=dv)

    _refill(st, shape, dtype, 7100)
    g = _capture(step)
    for r in range(3):
        _refill(st, shape, dtype, 7101 + r)
        eo, el = fa.forward(st["q"], st["k"], st["v"], causal=causal)
        edq, edk, edv = fa.backward(st["q"], st["k"], st["v"], eo, st["do"], el, causal=causal)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in (("O", o, eo), ("LSE", lse, el), ("dQ", dq, edq), ("dK", dk, edk), ("dV", dv, edv)):
            _same(f"replay {r} {name}", x, y)


def test_noalloc_backward_graph_replays_match_eager():
    import torch
    fa = _fa()
    shape, dtype, causal = (1, 4, 777, 64), "f16", True
    B, H, N, d = shape
    log(f"graph: fattn_bwd_noalloc B={B} H={H} N={N} d={d} {dtype} causal")
    z = lambda: torch.zeros(shape, dtype=torch.float16, device="cuda")
    st = {"q": z(), "k": z(), "v": z(), "do": z()}
    o, dq, dk, dv = z(), z(), z(), z()
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    code, scale = fa.dtype_code(o), d ** -0.5

    def step():
        s = torch.cuda.current_stream().cuda_stream
        assert fa.fattn_fwd(st["q"].data_ptr(), st["k"].data_ptr(), st["v"].data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, H, N, d, scale, 1, code, s) == 0
        assert fa.fattn_bwd_noalloc(st["q"].data_ptr(), st["k"].data_ptr(), st["v"].data_ptr(), o.data_ptr(),
                                    st["do"].data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), B, H, N, d, scale, 1, code, s) == 0

    _refill(st, shape, dtype, 7200)
    g = _capture(step)
    for r in range(3):
        _refill(st, shape, dtype, 7201 + r)
        eo, el = fa.forward(st["q"], st["k"], st["v"], causal=causal)
        edq, edk, edv = fa.backward(st["q"], st["k"], st["v"], eo, st["do"], el, causal=causal)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in (("O", o, eo), ("LSE", lse, el), ("dQ", dq, edq), ("dK", dk, edk), ("dV", dv, edv)):
            _same(f"replay {r} {name}", x, y)


def test_dropout_step_graph_replays_match_eager():
    import torch
    fa = _fa()
    shape, dtype, causal, p, seed = (1, 4, 640, 128), "bf16", True, 0.2, 99
    B, H, N, d = shape
    log(f"graph: dropout step B={B} H={H} N={N} d={d} {dtype} p={p}")
    z = lambda: torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    st = {"q": z(), "k": z(), "v": z(), "do": z()}
    o, dq, dk, dv = z(), z(), z(), z()
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fattn_bwd_workspace_size(B, H, N, d, fa.FATTN_BF16), dtype=torch.uint8, device="cuda")

    def step():
        fa.forward(st["q"], st["k"], st["v"], causal=causal, out=o, lse=lse, p_drop=p, seed=seed)
        fa.backward(st["q"], st["k"], st["v"], o, st["do"], lse, causal=causal, workspace=ws, p_drop=p, seed=seed,
                    dq=dq, dk=dk, dv=dv)

    _refill(st, shape, dtype, 7300)
    g = _capture(step)
    for r in range(3):
        _refill(st, shape, dtype, 7301 + r)
        eo, el = fa.forward(st["q"], st["k"], st["v"], causal=causal, p_drop=p, seed=seed)
        edq, edk, edv = fa.backward(st["q"], st["k"], st["v"], eo, st["do"], el, causal=causal, p_drop=p, seed=seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in (("O", o, eo), ("LSE", lse, el), ("dQ", dq, edq), ("dK", dk, edk), ("dV", dv, edv)):
            _same(f"replay {r} {name}", x, y)


def test_blocksparse_step_graph_replays_match_eager():
    import torch
    fa = _fa()
    shape, dtype, causal = (2, 2, 700, 128), "bf16", True
    B, H, N, d = shape
    nb = (N + 127) // 128
    log(f"graph: block-sparse step B={B} H={H} N={N} d={d} {dtype}")
    z = lambda: torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    st = {"q": z(), "k": z(), "v": z(), "do": z()}
    o, dq, dk, dv = z(), z(), z(), z()
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fattn_bwd_workspace_size(B, H, N, d, fa.FATTN_BF16), dtype=torch.uint8, device="cuda")
    bmask = torch.from_numpy(fi.block_mask(B, H, nb, 0.5, 31)).cuda()

    def step():
        fa.forward_blocksparse(st["q"], st["k"], st["v"], bmask, causal=causal, out=o, lse=lse)
        fa.backward_blocksparse(st["q"], st["k"], st["v"], o, st["do"], lse, bmask, causal=causal, workspace=ws,
                                dq=dq, dk=dk, dv=dv)

    _refill(st, shape, dtype, 7400)
    g = _capture(step)
    for r in range(3):
        _refill(st, shape, dtype, 7401 + r)
        eo, el = fa.forward_blocksparse(st["q"], st["k"], st["v"], bmask, causal=causal)
        edq, edk, edv = fa.backward_blocksparse(st["q"], st["k"], st["v"], eo, st["do"], el, bmask, causal=causal)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in (("O", o, eo), ("LSE", lse, el), ("dQ", dq, edq), ("dK", dk, edk), ("dV", dv, edv)):
            _same(f"replay {r} {name}", x, y)


def test_splitkv_decode_graph_replays_match_eager():
    import torch
    fa = _fa()
    B, H, Nq, Nk, d = 2, 4, 3, 5000, 128
    log(f"graph: split-KV decode B={B} H={H} Nq={Nq} Nk={Nk} d={d} bf16 causal")
    rng = np.random.default_rng(7500)
    qs = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    ks = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    vs = torch.zeros_like(ks)
    S = fa.fattn_splitkv_num_splits(B, H, Nq, Nk, d)
    ws = torch.empty(fa.fattn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, S), dtype=torch.uint8, device="cuda")
    o = torch.zeros_like(qs)
    lse = torch.zeros((B, H, Nq), dtype=torch.float32, device="cuda")

    def refill():
        for t in (qs, ks, vs):
            t.copy_(torch.from_numpy(rng.standard_normal(t.shape, dtype=np.float32)).to(torch.bfloat16))

    def step():
        fa.forward_splitkv(qs, ks, vs, causal=True, num_splits=S, out=o, lse=lse, workspace=ws)

    refill()
    g = _capture(step)
    for r in range(3):
        refill()
        eo, el = fa.forward_splitkv(qs, ks, vs, causal=True, num_splits=S)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(f"replay {r} O", o, eo)
        _same(f"replay {r} LSE", lse, el)
