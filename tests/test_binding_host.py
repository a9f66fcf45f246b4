"""The Python binding checks every tensor before it reaches the library (CPU, no GPU needed).

Stand-in tensors that claim to live on a device carry the shape, dtype, device and layout the
wrappers inspect; the raw C-ABI mirrors are replaced by recorders, so a test can tell whether a
call would have reached the library. A host tensor, a wrong dtype, a wrong shape or a short
workspace must raise ValueError before any launch; correct arguments must get through.
"""
import math

import pytest
import torch

import io_aware_tiled_fattn_amd as fa

DEV = torch.device("cuda:0")


class Dev:
    """A device-tensor stand-in: only the attributes the wrappers read."""

    def __init__(self, shape, dtype=torch.bfloat16, device=DEV, contiguous=True, is_cuda=True):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = device
        self.is_cuda = is_cuda
        self._contig = contiguous

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return 0x100000

    def numel(self):
        return math.prod(self.shape)

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()

    def dim(self):
        return len(self.shape)


class Stream:
    cuda_stream = 0


B, H, N, d = 1, 2, 64, 64
SHAPE = (B, H, N, d)


@pytest.fixture
def calls(monkeypatch):
    rec = []

    def recorder(name):
        def f(*args):
            rec.append(name)
            return 0
        return f

    for name in ("fattn_fwd_tiled", "fattn_fwd_dropout", "fattn_bwd", "fattn_bwd_dropout",
                 "fattn_bwd_preprocess", "fattn_bwd_dkdv", "fattn_bwd_dq", "fattn_fwd_kouter",
                 "fattn_fwd_blocksparse", "fattn_bwd_blocksparse", "fattn_fwd_splitkv",
                 "fattn_fwd_partial", "fattn_combine"):
        monkeypatch.setattr(fa, name, recorder(name))
    monkeypatch.setattr(fa, "fattn_bwd_workspace_size", lambda *a: 4 * B * H * N)
    monkeypatch.setattr(fa, "fattn_fwd_kouter_workspace_size", lambda *a: 4 * B * H * N * (d + 2))
    monkeypatch.setattr(fa, "fattn_fwd_splitkv_workspace_size", lambda *a: 1024)
    return rec


def _t(shape=SHAPE, **kw):
    return Dev(shape, **kw)


def _lse(**kw):
    kw.setdefault("dtype", torch.float32)
    return Dev((B, H, N), **kw)


BAD_LSE = {
    "host": lambda: Dev((B, H, N), torch.float32, device=torch.device("cpu"), is_cuda=False),
    "bf16": lambda: Dev((B, H, N), torch.bfloat16),
    "short": lambda: Dev((B, H, N - 1), torch.float32),
    "strided": lambda: Dev((B, H, N), torch.float32, contiguous=False),
    "other device": lambda: Dev((B, H, N), torch.float32, device=torch.device("cuda:1")),
}


def _fwd(lse, **kw):
    return fa.forward(_t(), _t(), _t(), out=_t(), lse=lse, stream=Stream(), **kw)


def _bwd(lse, **kw):
    kw.setdefault("workspace", Dev((4 * B * H * N,), torch.uint8))
    return fa.backward(_t(), _t(), _t(), _t(), _t(), lse, stream=Stream(), dq=_t(), dk=_t(), dv=_t(), **kw)


def test_good_arguments_reach_the_library(calls):
    _fwd(_lse())
    _fwd(_lse(), p_drop=0.1, seed=3)
    _bwd(_lse())
    _bwd(_lse(), p_drop=0.1, seed=3)
    fa.backward_stages(_t(), _t(), _t(), _t(), _t(), _lse(), _t(), _t(), _t(), _lse(), stream=Stream())
    assert calls == ["fattn_fwd_tiled", "fattn_fwd_dropout", "fattn_bwd", "fattn_bwd_dropout",
                     "fattn_bwd_preprocess", "fattn_bwd_dkdv", "fattn_bwd_dq"]


@pytest.mark.parametrize("bad", sorted(BAD_LSE))
def test_forward_rejects_a_bad_lse(calls, bad):
    with pytest.raises(ValueError, match="lse"):
        _fwd(BAD_LSE[bad]())
    with pytest.raises(ValueError, match="lse"):
        _fwd(BAD_LSE[bad](), p_drop=0.1)
    assert calls == []


@pytest.mark.parametrize("bad", sorted(BAD_LSE))
def test_backward_rejects_a_bad_lse(calls, bad):
    with pytest.raises(ValueError, match="lse"):
        _bwd(BAD_LSE[bad]())
    with pytest.raises(ValueError, match="lse"):
        fa.backward_blocksparse(_t(), _t(), _t(), _t(), _t(), BAD_LSE[bad](), Dev((B, H, 1, 1), torch.uint8),
                                stream=Stream(), workspace=Dev((4 * B * H * N,), torch.uint8),
                                dq=_t(), dk=_t(), dv=_t())
    assert calls == []


@pytest.mark.parametrize("which", ["lse", "dq", "dk", "dv", "dvec", "o", "do"])
@pytest.mark.parametrize("bad", ["host", "dtype", "shape"])
def test_backward_stages_rejects_bad_buffers(calls, which, bad):
    args = dict(q=_t(), k=_t(), v=_t(), o=_t(), do=_t(), lse=_lse(), dq=_t(), dk=_t(), dv=_t(), dvec=_lse())
    good = args[which]
    if bad == "host":
        args[which] = Dev(good.shape, good.dtype, device=torch.device("cpu"), is_cuda=False)
    elif bad == "dtype":
        args[which] = Dev(good.shape, torch.float16 if good.dtype != torch.float16 else torch.float32)
    else:
        args[which] = Dev(tuple(good.shape[:-1]) + (good.shape[-1] + 1,), good.dtype)
    with pytest.raises(ValueError, match=which):
        fa.backward_stages(**args, stream=Stream())
    assert calls == []


def test_backward_rejects_bad_workspace_and_outputs(calls):
    with pytest.raises(ValueError, match="workspace"):
        _bwd(_lse(), workspace=Dev((4 * B * H * N - 1,), torch.uint8))
    with pytest.raises(ValueError, match="workspace"):
        _bwd(_lse(), workspace=Dev((4 * B * H * N,), torch.uint8, device=torch.device("cpu"), is_cuda=False))
    with pytest.raises(ValueError, match="dk"):
        fa.backward(_t(), _t(), _t(), _t(), _t(), _lse(), stream=Stream(), dq=_t(), dk=_t(dtype=torch.float16),
                    dv=_t(), workspace=Dev((4 * B * H * N,), torch.uint8))
    with pytest.raises(ValueError, match="do"):
        fa.backward(_t(), _t(), _t(), _t(), _t((B, H, N, 128)), _lse(), stream=Stream(), dq=_t(), dk=_t(),
                    dv=_t(), workspace=Dev((4 * B * H * N,), torch.uint8))
    assert calls == []


def test_other_wrappers_check_their_outputs(calls):
    with pytest.raises(ValueError, match="lse"):
        fa.forward_kouter(_t(), _t(), _t(), out=_t(), lse=BAD_LSE["short"](), stream=Stream(),
                          workspace=Dev((10**6,), torch.uint8))
    with pytest.raises(ValueError, match="out"):
        fa.forward_kouter(_t(), _t(), _t(), out=_t(dtype=torch.float16), lse=_lse(), stream=Stream(),
                          workspace=Dev((10**6,), torch.uint8))
    with pytest.raises(ValueError, match="workspace"):
        fa.forward_kouter(_t(), _t(), _t(), out=_t(), lse=_lse(), stream=Stream(), workspace=Dev((8,), torch.uint8))
    with pytest.raises(ValueError, match="lse"):
        fa.forward_blocksparse(_t(), _t(), _t(), Dev((B, H, 1, 1), torch.uint8), out=_t(),
                               lse=BAD_LSE["bf16"](), stream=Stream())
    with pytest.raises(ValueError, match="block_mask"):
        fa.forward_blocksparse(_t(), _t(), _t(), Dev((B, H, 2, 2), torch.uint8), out=_t(), lse=_lse(),
                               stream=Stream())
    with pytest.raises(ValueError, match="workspace"):
        fa.forward_splitkv(_t((B, H, 4, d)), _t(), _t(), out=_t((B, H, 4, d)), lse=Dev((B, H, 4), torch.float32),
                           workspace=Dev((1023,), torch.uint8), stream=Stream())
    with pytest.raises(ValueError, match="k"):
        fa.forward_splitkv(_t((B, H, 4, d)), _t((B, H, N, d), dtype=torch.float16), _t(), stream=Stream())
    assert calls == []
    fa.forward_kouter(_t(), _t(), _t(), out=_t(), lse=_lse(), stream=Stream(), workspace=Dev((10**6,), torch.uint8))
    fa.forward_blocksparse(_t(), _t(), _t(), Dev((B, H, 1, 1), torch.uint8), out=_t(), lse=_lse(), stream=Stream())
    fa.forward_splitkv(_t((B, H, 4, d)), _t(), _t(), out=_t((B, H, 4, d)), lse=Dev((B, H, 4), torch.float32),
                       workspace=Dev((1024,), torch.uint8), stream=Stream())
    assert calls == ["fattn_fwd_kouter", "fattn_fwd_blocksparse", "fattn_fwd_splitkv"]


def test_backward_stages_accepts_a_flat_dvec(calls):
    fa.backward_stages(_t(), _t(), _t(), _t(), _t(), _lse(), _t(), _t(), _t(), Dev((B * H * N,), torch.float32),
                       stream=Stream(), stages=(0,))
    with pytest.raises(ValueError, match="dvec"):
        fa.backward_stages(_t(), _t(), _t(), _t(), _t(), _lse(), _t(), _t(), _t(),
                           Dev((B * H * N - 1,), torch.float32), stream=Stream())
    assert calls == ["fattn_bwd_preprocess"]
