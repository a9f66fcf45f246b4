"""fattn_bwd_noalloc (the backward that allocates nothing) against fattn_bwd, through the C ABI.

Two calls in a row on one GPU, the second on a smaller problem of another head dim and mask, so
the static buffer is reused with stale contents from the first; each must give fattn_bwd's
results bit for bit (the same kernels run on the same D values). Sizes past the buffer are
rejected before any HIP call.
"""
import math

import pytest

import fattn_inputs as fi
from tests.gpu_util import log, upload

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_tiled_fattn_amd as fa
    fa.lib()
    return fa


def _both(fa, shape, dtype, causal, seed):
    import torch
    B, H, N, d = shape
    inp = fi.make_inputs(shape, dtype, seed, with_do=True)
    q, k, v, do = upload(inp)
    o, lse = fa.forward(q, k, v, causal=causal)
    scale = 1 / math.sqrt(d)
    code = fa.dtype_code(q)
    ref = fa.backward(q, k, v, o, do, lse, causal=causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    stream = torch.cuda.current_stream().cuda_stream
    st = fa.fattn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(),
                              B, H, N, d, scale, int(causal), code, stream)
    assert st == 0, fa.fattn_strerror(st)
    torch.cuda.synchronize()
    for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(x, y), name


def test_noalloc_backward_matches_fattn_bwd_on_two_calls():
    fa = _fa()
    log("noalloc bwd call 1: B=2 H=4 N=1000 d=128 bf16 causal")
    _both(fa, (2, 4, 1000, 128), "bf16", True, 1201)
    log("noalloc bwd call 2: B=1 H=2 N=300 d=64 f16 non-causal")
    _both(fa, (1, 2, 300, 64), "f16", False, 1202)


def test_noalloc_backward_rejects_sizes_past_its_buffer():
    import torch
    fa = _fa()
    cap = fa.fattn_bwd_noalloc_max_bytes()
    assert cap == 16 << 20
    rows = cap // 4  # D holds one float32 per row
    # distinct, aligned device addresses (never read: the calls are rejected before any launch)
    t = torch.empty(8192, dtype=torch.bfloat16, device="cuda")
    p = t.data_ptr()
    args = tuple(p + 1024 * i for i in range(9))
    st = fa.fattn_bwd_noalloc(*args, 1, 1, rows + 1, 64, 0.125, 0, fa.FATTN_BF16, None)
    assert st == -14 and "static scratch" in fa.fattn_strerror(st)
    st = fa.fattn_bwd_noalloc(*args, 4, 1, rows // 4 + 1, 128, 0.125, 1, fa.FATTN_BF16, None)
    assert st == -14
