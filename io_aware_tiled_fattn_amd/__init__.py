"""Python binding of libfattn (exact FlashAttention-style attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the
C ABI declared in include/fattn.h. PyTorch is used to allocate device memory and to name the
stream; there is no CPU or PyTorch fallback, and a missing library raises.

Low-level names mirror the C entry points (``fattn_fwd``, ``fattn_fwd_tiled``, ``fattn_bwd``,
``fattn_bwd_workspace_size``, ``fattn_bwd_preprocess``, ``fattn_bwd_dkdv``, ``fattn_bwd_dq``,
``fattn_fwd_splitkv``, ``fattn_fwd_splitkv_workspace_size``,
``fattn_splitkv_num_splits``, ``fattn_fwd_partial``, ``fattn_combine``, ``fattn_fwd_kouter``,
``fattn_fwd_kouter_workspace_size``, ``fattn_fwd_dropout``, ``fattn_bwd_dropout``,
``fattn_fwd_blocksparse``, ``fattn_bwd_blocksparse``, ``fattn_bwd_noalloc``,
``fattn_bwd_noalloc_max_bytes``, ``fattn_strerror``, ``fattn_version``) and take raw device addresses. ``forward``, ``backward``,
``backward_stages``, ``forward_splitkv``, ``forward_partial``, ``combine`` and ``forward_kouter`` wrap them for
contiguous torch tensors.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FATTN_F32", "FATTN_F16", "FATTN_BF16", "FattnError", "lib", "library_path",
    "fattn_fwd", "fattn_fwd_tiled", "fattn_bwd", "fattn_bwd_workspace_size", "fattn_strerror",
    "fattn_bwd_preprocess", "fattn_bwd_dkdv", "fattn_bwd_dq",
    "fattn_version", "forward", "backward", "backward_stages", "dtype_code",
    "fattn_fwd_splitkv", "fattn_fwd_splitkv_workspace_size", "fattn_splitkv_num_splits",
    "fattn_fwd_partial", "fattn_combine", "forward_splitkv", "forward_partial", "combine",
    "fattn_fwd_kouter", "fattn_fwd_kouter_workspace_size", "forward_kouter",
    "fattn_fwd_dropout", "fattn_bwd_dropout", "fattn_fwd_blocksparse", "forward_blocksparse",
    "fattn_bwd_blocksparse", "backward_blocksparse", "fattn_bwd_noalloc", "fattn_bwd_noalloc_max_bytes",
]

FATTN_F32, FATTN_F16, FATTN_BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libfattn.so")


class FattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fattn_strerror(status)} (status {status})")


def lib():
    """Load libfattn.so (built in-tree by io_aware_tiled_fattn_amd.build); raise if missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libfattn.so not found at {path}; build it with "
                           "`python -m io_aware_tiled_fattn_amd.build` (no fallback exists)")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fattn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    L.fattn_fwd.restype = i
    L.fattn_fwd_tiled.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, i, vp]
    L.fattn_fwd_tiled.restype = i
    L.fattn_bwd_workspace_size.argtypes = [i, i, i, i, i]
    L.fattn_bwd_workspace_size.restype = sz
    L.fattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]
    L.fattn_bwd.restype = i
    L.fattn_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    L.fattn_bwd_preprocess.restype = i
    L.fattn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    L.fattn_bwd_dkdv.restype = i
    L.fattn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    L.fattn_bwd_dq.restype = i
    L.fattn_splitkv_num_splits.argtypes = [i, i, i, i, i]
    L.fattn_splitkv_num_splits.restype = i
    L.fattn_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i, i]
    L.fattn_fwd_splitkv_workspace_size.restype = sz
    L.fattn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    L.fattn_fwd_splitkv.restype = i
    L.fattn_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    L.fattn_fwd_partial.restype = i
    L.fattn_combine.argtypes = [vp, vp, i, vp, vp, i, i, i, i, i, vp]
    L.fattn_combine.restype = i
    L.fattn_fwd_kouter_workspace_size.argtypes = [i, i, i, i, i]
    L.fattn_fwd_kouter_workspace_size.restype = sz
    L.fattn_fwd_kouter.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]
    L.fattn_fwd_kouter.restype = i
    u64 = ctypes.c_ulonglong
    L.fattn_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, f, u64, vp]
    L.fattn_fwd_dropout.restype = i
    L.fattn_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, f, u64, vp, sz, vp]
    L.fattn_bwd_dropout.restype = i
    L.fattn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, vp]
    L.fattn_fwd_blocksparse.restype = i
    L.fattn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, vp, sz, vp]
    L.fattn_bwd_blocksparse.restype = i
    L.fattn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    L.fattn_bwd_noalloc.restype = i
    L.fattn_bwd_noalloc_max_bytes.argtypes = []
    L.fattn_bwd_noalloc_max_bytes.restype = sz
    L.fattn_strerror.argtypes = [i]
    L.fattn_strerror.restype = ctypes.c_char_p
    L.fattn_version.argtypes = []
    L.fattn_version.restype = i
    _LIB = L
    return L


# --- raw C-ABI mirrors (pointers are ints: device addresses; stream is an int or None) -------


def fattn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream=None) -> int:
    return lib().fattn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream)


def fattn_fwd_tiled(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, Br, Bc, stream=None) -> int:
    return lib().fattn_fwd_tiled(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, Br, Bc, stream)


def fattn_bwd_workspace_size(B, H, N, d, dtype) -> int:
    return lib().fattn_bwd_workspace_size(B, H, N, d, dtype)


def fattn_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype,
              workspace, workspace_bytes, stream=None) -> int:
    return lib().fattn_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype,
                           workspace, workspace_bytes, stream)


def fattn_bwd_preprocess(o, dO, dvec, B, H, N, d, dtype, stream=None) -> int:
    return lib().fattn_bwd_preprocess(o, dO, dvec, B, H, N, d, dtype, stream)


def fattn_bwd_dkdv(q, k, v, dO, lse, dvec, dk, dv, B, H, N, d, scale, causal, dtype, stream=None) -> int:
    return lib().fattn_bwd_dkdv(q, k, v, dO, lse, dvec, dk, dv, B, H, N, d, scale, causal, dtype, stream)


def fattn_bwd_dq(q, k, v, dO, lse, dvec, dq, B, H, N, d, scale, causal, dtype, stream=None) -> int:
    return lib().fattn_bwd_dq(q, k, v, dO, lse, dvec, dq, B, H, N, d, scale, causal, dtype, stream)


def fattn_splitkv_num_splits(B, H, Nq, Nk, d) -> int:
    return lib().fattn_splitkv_num_splits(B, H, Nq, Nk, d)


def fattn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, num_splits) -> int:
    return lib().fattn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, num_splits)


def fattn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits,
                      workspace, workspace_bytes, stream=None) -> int:
    return lib().fattn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits,
                                   workspace, workspace_bytes, stream)


def fattn_fwd_partial(q, k, v, o_parts, lse_parts, B, H, Nq, Nk, d, scale, causal, dtype, num_splits,
                      stream=None) -> int:
    return lib().fattn_fwd_partial(q, k, v, o_parts, lse_parts, B, H, Nq, Nk, d, scale, causal, dtype,
                                   num_splits, stream)


def fattn_combine(o_parts, lse_parts, num_splits, o, lse, B, H, Nq, d, dtype, stream=None) -> int:
    return lib().fattn_combine(o_parts, lse_parts, num_splits, o, lse, B, H, Nq, d, dtype, stream)


def fattn_fwd_kouter_workspace_size(B, H, N, d, dtype) -> int:
    return lib().fattn_fwd_kouter_workspace_size(B, H, N, d, dtype)


def fattn_fwd_kouter(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, workspace, workspace_bytes,
                     stream=None) -> int:
    return lib().fattn_fwd_kouter(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, workspace,
                                  workspace_bytes, stream)


def fattn_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, p_drop, seed, stream=None) -> int:
    return lib().fattn_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, p_drop, seed, stream)


def fattn_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, p_drop, seed,
                      workspace, workspace_bytes, stream=None) -> int:
    return lib().fattn_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype,
                                   p_drop, seed, workspace, workspace_bytes, stream)


def fattn_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, block_mask, stream=None) -> int:
    return lib().fattn_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, block_mask, stream)


def fattn_bwd_blocksparse(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, block_mask,
                          workspace, workspace_bytes, stream=None) -> int:
    return lib().fattn_bwd_blocksparse(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype,
                                       block_mask, workspace, workspace_bytes, stream)


def fattn_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, stream=None) -> int:
    return lib().fattn_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, stream)


def fattn_bwd_noalloc_max_bytes() -> int:
    return lib().fattn_bwd_noalloc_max_bytes()


def fattn_strerror(status: int) -> str:
    return lib().fattn_strerror(status).decode()


def fattn_version() -> int:
    return lib().fattn_version()


# --- torch-tensor wrappers ---------------------------------------------------------------------
#
# Every tensor handed to the library is checked here before any launch: it must be a contiguous
# device tensor on q's device, of the shape and dtype the entry point reads or writes. A host
# tensor, a wrong dtype or a short buffer would otherwise reach a kernel as a bad address or an
# out-of-range access.


def dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FATTN_F32, torch.float16: FATTN_F16, torch.bfloat16: FATTN_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_dev(t, name, shape=None, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")


def _check(t, name, like=None):
    """A [B, H, N, d] tensor; with ``like``, of like's shape, dtype and device."""
    if like is None:
        _check_dev(t, name)
        if len(t.shape) != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
    else:
        _check_dev(t, name, like.shape, like.dtype, like.device)


def _check_rows(t, name, q, flat_ok=False):
    """A float32 [B, H, N] per-row tensor (LSE, D) for q [B, H, N, d]; with ``flat_ok`` a
    contiguous [B * H * N] vector is accepted as well."""
    import torch
    B, H, N, _ = q.shape
    if flat_ok and t is not None and len(t.shape) == 1:
        _check_dev(t, name, (B * H * N,), torch.float32, q.device)
    else:
        _check_dev(t, name, (B, H, N), torch.float32, q.device)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _workspace(workspace, need, device):
    """The caller's workspace (checked: a device tensor on ``device`` of at least ``need`` bytes)
    or a new one."""
    import torch
    if workspace is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    _check_dev(workspace, "workspace", device=device)
    if _nbytes(workspace) < need:
        raise ValueError(f"workspace holds {_nbytes(workspace)} bytes, {need} needed")
    return workspace


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def forward(q, k, v, causal=False, scale=None, Br=0, Bc=0, out=None, lse=None, stream=None,
            p_drop=0.0, seed=0):
    """O, LSE for contiguous [B, H, N, d] device tensors (float32, float16 or bfloat16).

    ``out`` and ``lse`` may be given to write into existing tensors (no allocation then).
    ``p_drop`` > 0 applies dropout to P with the keep mask of ``seed`` (fattn_fwd_dropout;
    16-bit types, default tile shape).
    """
    import torch
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(out, "out", q)
    _check_rows(lse, "lse", q)
    if p_drop:
        if Br or Bc:
            raise ValueError("dropout runs with the default tile shape")
        st = fattn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, N, d, float(scale), int(bool(causal)), dtype_code(q), float(p_drop),
                               int(seed), _stream(stream))
        if st != 0:
            raise FattnError(st, "fattn_fwd_dropout")
        return out, lse
    st = fattn_fwd_tiled(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, H, N, d, float(scale), int(bool(causal)), dtype_code(q), int(Br), int(Bc),
                         _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_fwd")
    return out, lse


def _check_bwd_inputs(q, k, v, o, do, lse):
    _check(q, "q")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, q)
    _check_rows(lse, "lse", q)


def _grad_outputs(q, dq, dk, dv):
    import torch
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, q)
    return dq, dk, dv


def backward(q, k, v, o, do, lse, causal=False, scale=None, workspace=None, stream=None, p_drop=0.0,
             seed=0, dq=None, dk=None, dv=None):
    """dQ, dK, dV for contiguous [B, H, N, d] float16/bfloat16 device tensors (with dropout of
    ``p_drop`` and ``seed`` when p_drop > 0: the same mask as the forward). ``dq``, ``dk``,
    ``dv`` may be given to write into existing tensors."""
    _check_bwd_inputs(q, k, v, o, do, lse)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = dtype_code(q)
    workspace = _workspace(workspace, fattn_bwd_workspace_size(B, H, N, d, code), q.device)
    dq, dk, dv = _grad_outputs(q, dq, dk, dv)
    if p_drop:
        st = fattn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                               B, H, N, d, float(scale), int(bool(causal)), code, float(p_drop), int(seed),
                               workspace.data_ptr(), _nbytes(workspace), _stream(stream))
        if st != 0:
            raise FattnError(st, "fattn_bwd_dropout")
        return dq, dk, dv
    st = fattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                   lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                   B, H, N, d, float(scale), int(bool(causal)), code,
                   workspace.data_ptr(), _nbytes(workspace), _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_bwd")
    return dq, dk, dv


def backward_stages(q, k, v, o, do, lse, dq, dk, dv, dvec, causal=False, scale=None, stream=None,
                    stages=(0, 1, 2)):
    """Run the chosen stages of the backward (0: D = rowsum(dO*O), 1: dK/dV, 2: dQ) into
    preallocated outputs; ``dvec`` is a float32 [B, H, N] (or flat [B * H * N]) device tensor."""
    _check_bwd_inputs(q, k, v, o, do, lse)
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, q)
    _check_rows(dvec, "dvec", q, flat_ok=True)
    for stage in stages:
        if stage not in (0, 1, 2):
            raise ValueError(f"unknown backward stage {stage}")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = dtype_code(q)
    s = _stream(stream)
    for stage in stages:
        if stage == 0:
            st = fattn_bwd_preprocess(o.data_ptr(), do.data_ptr(), dvec.data_ptr(), B, H, N, d, code, s)
        elif stage == 1:
            st = fattn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                                dvec.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale),
                                int(bool(causal)), code, s)
        else:
            st = fattn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                              dvec.data_ptr(), dq.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                              code, s)
        if st != 0:
            raise FattnError(st, f"backward stage {stage}")


def _decode_shapes(q, k, v):
    _check_dev(q, "q")
    _check_dev(k, "k")
    if len(q.shape) != 4 or len(k.shape) != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check_dev(k, "k", (B, H, Nk, d), q.dtype, q.device)
    _check_dev(v, "v", (B, H, Nk, d), q.dtype, q.device)
    return B, H, Nq, Nk, d


def forward_splitkv(q, k, v, causal=False, scale=None, num_splits=0, out=None, lse=None,
                    workspace=None, stream=None):
    """O [B, H, Nq, d], LSE [B, H, Nq] of q [B, H, Nq, d] against k, v [B, H, Nk, d] by split-KV
    partials and their merge (float16/bfloat16). ``num_splits`` 0 lets the library choose."""
    import torch
    B, H, Nq, Nk, d = _decode_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fattn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, int(num_splits))
    workspace = _workspace(workspace, need, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_dev(out, "out", q.shape, q.dtype, q.device)
    _check_dev(lse, "lse", (B, H, Nq), torch.float32, q.device)
    st = fattn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           B, H, Nq, Nk, d, float(scale), int(bool(causal)), dtype_code(q), int(num_splits),
                           workspace.data_ptr(), _nbytes(workspace), _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_fwd_splitkv")
    return out, lse


def forward_partial(q, k, v, num_splits, causal=False, scale=None, o_parts=None, lse_parts=None,
                    stream=None):
    """Per-split partials O_s [S, B, H, Nq, d] and LSE_s [S, B, H, Nq] (float32)."""
    import torch
    B, H, Nq, Nk, d = _decode_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = int(num_splits)
    if o_parts is None:
        o_parts = torch.empty((S, B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_parts is None:
        lse_parts = torch.empty((S, B, H, Nq), dtype=torch.float32, device=q.device)
    _check_dev(o_parts, "o_parts", (S, B, H, Nq, d), torch.float32, q.device)
    _check_dev(lse_parts, "lse_parts", (S, B, H, Nq), torch.float32, q.device)
    st = fattn_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_parts.data_ptr(),
                           lse_parts.data_ptr(), B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                           dtype_code(q), S, _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_fwd_partial")
    return o_parts, lse_parts


def combine(o_parts, lse_parts, dtype=None, out=None, lse=None, stream=None):
    """Merge float32 partials O_s [S, B, H, Nq, d], LSE_s [S, B, H, Nq] into O (``dtype``, default
    float32) and LSE [B, H, Nq]."""
    import torch
    _check_dev(o_parts, "o_parts", None, torch.float32)
    if len(o_parts.shape) != 5:
        raise ValueError("o_parts must be [S, B, H, Nq, d]")
    S, B, H, Nq, d = o_parts.shape
    dev = o_parts.device
    _check_dev(lse_parts, "lse_parts", (S, B, H, Nq), torch.float32, dev)
    dtype = torch.float32 if dtype is None else dtype
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    _check_dev(out, "out", (B, H, Nq, d), None, dev)
    _check_dev(lse, "lse", (B, H, Nq), torch.float32, dev)
    st = fattn_combine(o_parts.data_ptr(), lse_parts.data_ptr(), S, out.data_ptr(), lse.data_ptr(),
                       B, H, Nq, d, dtype_code(out), _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_combine")
    return out, lse


def forward_kouter(q, k, v, causal=False, scale=None, out=None, lse=None, workspace=None, stream=None):
    """O, LSE by the K-outer loop order (the ablation); same contract as ``forward``."""
    import torch
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = dtype_code(q)
    workspace = _workspace(workspace, fattn_fwd_kouter_workspace_size(B, H, N, d, code), q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(out, "out", q)
    _check_rows(lse, "lse", q)
    st = fattn_fwd_kouter(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, N, d, float(scale), int(bool(causal)), code, workspace.data_ptr(),
                          _nbytes(workspace), _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_fwd_kouter")
    return out, lse


def forward_blocksparse(q, k, v, block_mask, causal=False, scale=None, out=None, lse=None, stream=None):
    """O, LSE of block-sparse attention; ``block_mask`` is a uint8 device tensor [B, H, nb, nb]
    over 128 x 128 (query, key) blocks, nb = ceil(N / 128)."""
    import torch
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    B, H, N, d = q.shape
    nb = (N + 127) // 128
    _check_dev(block_mask, "block_mask", (B, H, nb, nb), torch.uint8, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(out, "out", q)
    _check_rows(lse, "lse", q)
    st = fattn_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, N, d, float(scale), int(bool(causal)), dtype_code(q),
                               block_mask.data_ptr(), _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_fwd_blocksparse")
    return out, lse


def backward_blocksparse(q, k, v, o, do, lse, block_mask, causal=False, scale=None, workspace=None,
                         stream=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV of block-sparse attention (the same ``block_mask`` as forward_blocksparse)."""
    import torch
    _check_bwd_inputs(q, k, v, o, do, lse)
    B, H, N, d = q.shape
    nb = (N + 127) // 128
    _check_dev(block_mask, "block_mask", (B, H, nb, nb), torch.uint8, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = dtype_code(q)
    workspace = _workspace(workspace, fattn_bwd_workspace_size(B, H, N, d, code), q.device)
    dq, dk, dv = _grad_outputs(q, dq, dk, dv)
    st = fattn_bwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                               B, H, N, d, float(scale), int(bool(causal)), code, block_mask.data_ptr(),
                               workspace.data_ptr(), _nbytes(workspace), _stream(stream))
    if st != 0:
        raise FattnError(st, "fattn_bwd_blocksparse")
    return dq, dk, dv
