"""The C-ABI library loads without a GPU, exports every declared symbol, and rejects every bad
argument on the host before any HIP call (so these calls are safe with fake device pointers)."""
import ctypes
import math
import os
import re

import pytest

import io_aware_tiled_fattn_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fattn.h")

# Fake, 16-byte-aligned device addresses: only ever passed to calls that must fail validation.
P = [0x10000 * (i + 1) for i in range(12)]
MIS = 0x10008  # 8-byte aligned only


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fattn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.library_path()):
        pytest.fail("libfattn.so is not built (run python -m io_aware_tiled_fattn_amd.build)")
    return fa.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"fattn_fwd", "fattn_fwd_tiled", "fattn_bwd", "fattn_bwd_workspace_size",
            "fattn_strerror", "fattn_version", "fattn_bwd_preprocess", "fattn_bwd_dkdv",
            "fattn_bwd_dq", "fattn_fwd_splitkv",
            "fattn_fwd_splitkv_workspace_size", "fattn_splitkv_num_splits", "fattn_fwd_partial",
            "fattn_combine", "fattn_fwd_kouter", "fattn_fwd_kouter_workspace_size",
            "fattn_fwd_dropout", "fattn_bwd_dropout", "fattn_fwd_blocksparse",
            "fattn_bwd_blocksparse", "fattn_bwd_noalloc", "fattn_bwd_noalloc_max_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
        assert getattr(fa, n) is not None


def test_version_and_strerror(L):
    assert fa.fattn_version() >= 100
    for code in range(0, -15, -1):
        s = fa.fattn_strerror(code)
        assert s and s != "unknown status", code
    assert fa.fattn_strerror(12345) == "unknown status"


def fwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=16, d=64, scale=0.125,
             causal=0, dtype=fa.FATTN_BF16, Br=0, Bc=0, stream=None)
    a.update(kw)
    return fa.fattn_fwd_tiled(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                              a["d"], a["scale"], a["causal"], a["dtype"], a["Br"], a["Bc"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(N=0), -2), (dict(N=-5), -2), (dict(B=-1), -2),
    (dict(N=16777217), -2), (dict(B=65536, H=65536), -2),
    (dict(d=96), -3), (dict(d=32), -3), (dict(d=256), -3), (dict(d=0), -3),
    (dict(dtype=3), -4), (dict(dtype=-1), -4),
    (dict(Br=96, Bc=64), -5), (dict(Br=128, Bc=32), -5), (dict(Br=64, Bc=0), -5),
    (dict(Br=512, Bc=64), -5), (dict(Br=256, Bc=32), -5), (dict(Br=256, Bc=256), -5),
    (dict(dtype=fa.FATTN_F32, Br=128, Bc=64), -5),
    (dict(q=MIS), -6), (dict(o=MIS), -6), (dict(lse=MIS), -6),
    (dict(scale=float("nan")), -7), (dict(scale=float("inf")), -7), (dict(scale=-math.inf), -7),
    (dict(o=P[0]), -11), (dict(lse=P[1]), -11), (dict(lse=P[3]), -11),
    (dict(causal=2), -12), (dict(causal=-1), -12),
])
def test_forward_rejects_bad_arguments(L, kw, status):
    assert fwd(**kw) == status


def bwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], dO=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8],
             B=2, H=3, N=100, d=128, scale=0.088, causal=1, dtype=fa.FATTN_BF16, ws=P[9],
             wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = fa.fattn_bwd_workspace_size(a["B"], a["H"], a["N"], a["d"], a["dtype"]) if a["dtype"] in (1, 2) and a["d"] in (64, 128) and min(a["B"], a["H"], a["N"]) > 0 else 0
    return fa.fattn_bwd(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"], a["dq"], a["dk"], a["dv"],
                        a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], a["ws"],
                        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(dO=None), -1), (dict(lse=None), -1), (dict(dv=None), -1),
    (dict(N=0), -2), (dict(H=0), -2),
    (dict(d=80), -3),
    (dict(dtype=fa.FATTN_F32), -4), (dict(dtype=9), -4),
    (dict(dq=MIS), -6), (dict(k=MIS), -6),
    (dict(scale=float("nan")), -7),
    (dict(ws=None), -8), (dict(wsb=16), -8),
    (dict(dq=P[0]), -11), (dict(dk=P[4]), -11), (dict(dv=P[6]), -11), (dict(ws=P[6]), -11), (dict(ws=P[1]), -11),
    (dict(causal=3), -12),
])
def test_backward_rejects_bad_arguments(L, kw, status):
    assert bwd(**kw) == status


def test_workspace_size(L):
    n = fa.fattn_bwd_workspace_size(2, 16, 4096, 128, fa.FATTN_BF16)
    assert n >= 4 * 2 * 16 * 4096 and n % 256 == 0
    assert fa.fattn_bwd_workspace_size(2, 16, 4096, 96, fa.FATTN_BF16) == 0
    assert fa.fattn_bwd_workspace_size(0, 16, 4096, 128, fa.FATTN_BF16) == 0
    assert fa.fattn_bwd_workspace_size(1, 1, 16, 64, fa.FATTN_F32) == 0


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


@pytest.mark.parametrize("call,status", [
    (lambda: fa.fattn_bwd_preprocess(None, P[1], P[2], 1, 1, 8, 64, 2), -1),
    (lambda: fa.fattn_bwd_preprocess(P[0], P[1], P[2], 1, 1, 8, 64, 0), -4),
    (lambda: fa.fattn_bwd_preprocess(P[0], P[1], P[0], 1, 1, 8, 64, 2), -11),
    (lambda: fa.fattn_bwd_preprocess(P[0], P[1], MIS, 1, 1, 8, 64, 2), -6),
    (lambda: fa.fattn_bwd_preprocess(P[0], P[1], P[2], 1, 1, 8, 96, 2), -3),
    (lambda: fa.fattn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], None, 1, 1, 8, 64, 0.1, 0, 2), -1),
    (lambda: fa.fattn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[6], 1, 1, 8, 64, 0.1, 0, 2), -11),
    (lambda: fa.fattn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[0], 1, 1, 8, 64, 0.1, 0, 2), -11),
    (lambda: fa.fattn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 1, 1, 8, 64, float("nan"), 0, 2), -7),
    (lambda: fa.fattn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 1, 1, 8, 64, 0.1, 5, 2), -12),
    (lambda: fa.fattn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 1, 1, 8, 64, 0.1, 0, 0), -4),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], None, P[6], 1, 1, 8, 64, 0.1, 0, 2), -1),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[5], 1, 1, 8, 64, 0.1, 0, 2), -11),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], MIS, 1, 1, 8, 64, 0.1, 0, 2), -6),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 0, 1, 8, 64, 0.1, 0, 2), -2),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], None, 1, 1, 8, 64, 0.1, 0, 2), -1),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[3], 1, 1, 8, 64, 0.1, 0, 2), -11),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 1, 1, 8, 96, 0.1, 0, 2), -3),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 1, 1, 8, 64, 0.1, 2, 2), -12),
    (lambda: fa.fattn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 1, 1, 8, 64, 0.1, 0, 0), -4),
])
def test_backward_stages_reject_bad_arguments(L, call, status):
    assert call() == status


# --------------------------------------------------------------------------------------------
# Split-KV entry points


def _r256(x):
    return (x + 255) // 256 * 256


def test_splitkv_sizes(L):
    S = fa.fattn_splitkv_num_splits(8, 32, 1, 16384, 128)
    assert 1 <= S <= 1024
    # a head-rich shape needs no splitting beyond what fills the chip; tiny Nk cannot be split
    assert fa.fattn_splitkv_num_splits(64, 64, 1, 16384, 128) >= 1
    assert fa.fattn_splitkv_num_splits(1, 1, 1, 100, 128) == 1
    assert fa.fattn_splitkv_num_splits(1, 1, 1, 100, 96) == 0
    for B, H, nq, nk, d, s in [(8, 32, 1, 16384, 128, 8), (2, 3, 40, 1000, 64, 5), (1, 1, 1, 1, 64, 1)]:
        n = fa.fattn_fwd_splitkv_workspace_size(B, H, nq, nk, d, s)
        assert n == _r256(s * B * H * nq * d * 4) + _r256(s * B * H * nq * 4)
    auto = fa.fattn_splitkv_num_splits(8, 32, 16, 16384, 128)
    assert fa.fattn_fwd_splitkv_workspace_size(8, 32, 16, 16384, 128, 0) == \
        fa.fattn_fwd_splitkv_workspace_size(8, 32, 16, 16384, 128, auto)
    assert fa.fattn_fwd_splitkv_workspace_size(8, 32, 16, 16384, 128, 1025) == 0
    assert fa.fattn_fwd_splitkv_workspace_size(8, 32, 0, 16384, 128, 4) == 0


def split(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, Nq=4, Nk=100, d=64, scale=0.125,
             causal=0, dtype=fa.FATTN_BF16, S=2, ws=P[5], wsb=1 << 20, stream=None)
    a.update(kw)
    return fa.fattn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["S"], a["ws"],
                                a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(dtype=fa.FATTN_F32), -4), (dict(dtype=7), -4), (dict(d=96), -3),
    (dict(Nq=0), -2), (dict(Nk=0), -2), (dict(B=0), -2), (dict(S=1025), -2), (dict(S=-1), -2),
    (dict(causal=1, Nq=101), -2), (dict(causal=3), -12), (dict(scale=float("inf")), -7),
    (dict(ws=None), -8), (dict(wsb=100), -8), (dict(q=MIS), -6), (dict(ws=MIS), -6),
    (dict(o=P[0]), -11), (dict(lse=P[1]), -11), (dict(ws=P[3]), -11), (dict(o=P[4]), -11),
    (dict(Nq=16777217), -2),
])
def test_splitkv_rejects_bad_arguments(L, kw, status):
    assert split(**kw) == status


@pytest.mark.parametrize("call,status", [
    (lambda: fa.fattn_fwd_partial(P[0], P[1], P[2], None, P[4], 1, 1, 4, 100, 64, 0.1, 0, 2, 2), -1),
    (lambda: fa.fattn_fwd_partial(P[0], P[1], P[2], P[3], P[4], 1, 1, 4, 100, 64, 0.1, 0, 2, 0), -2),
    (lambda: fa.fattn_fwd_partial(P[0], P[1], P[2], P[3], P[3], 1, 1, 4, 100, 64, 0.1, 0, 2, 2), -11),
    (lambda: fa.fattn_fwd_partial(P[0], P[1], P[2], P[0], P[4], 1, 1, 4, 100, 64, 0.1, 0, 2, 2), -11),
    (lambda: fa.fattn_fwd_partial(P[0], P[1], P[2], P[3], MIS, 1, 1, 4, 100, 64, 0.1, 0, 2, 2), -6),
    (lambda: fa.fattn_fwd_partial(P[0], P[1], P[2], P[3], P[4], 1, 1, 4, 100, 64, 0.1, 0, 0, 2), -4),
    (lambda: fa.fattn_fwd_partial(P[0], P[1], P[2], P[3], P[4], 1, 1, 200, 100, 64, 0.1, 1, 2, 2), -2),
    (lambda: fa.fattn_combine(None, P[1], 2, P[2], P[3], 1, 1, 4, 64, 2), -1),
    (lambda: fa.fattn_combine(P[0], P[1], 0, P[2], P[3], 1, 1, 4, 64, 2), -2),
    (lambda: fa.fattn_combine(P[0], P[1], 2, P[0], P[3], 1, 1, 4, 64, 2), -11),
    (lambda: fa.fattn_combine(P[0], P[1], 2, P[2], P[2], 1, 1, 4, 64, 2), -11),
    (lambda: fa.fattn_combine(P[0], P[1], 2, P[2], P[3], 1, 1, 4, 64, 9), -4),
    (lambda: fa.fattn_combine(P[0], P[1], 2, P[2], P[3], 1, 1, 4, 80, 0), -3),
    (lambda: fa.fattn_combine(P[0], MIS, 2, P[2], P[3], 1, 1, 4, 64, 0), -6),
])
def test_partial_and_combine_reject_bad_arguments(L, call, status):
    assert call() == status


# --------------------------------------------------------------------------------------------
# K-outer ablation


def test_kouter_workspace_size(L):
    n = fa.fattn_fwd_kouter_workspace_size(2, 16, 4096, 128, fa.FATTN_BF16)
    assert n == _r256(2 * 16 * 4096 * 130 * 4)
    assert fa.fattn_fwd_kouter_workspace_size(2, 16, 4096, 128, fa.FATTN_F32) == 0
    assert fa.fattn_fwd_kouter_workspace_size(2, 16, 4096, 96, fa.FATTN_BF16) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(dtype=fa.FATTN_F32), -4), (dict(d=96), -3),
    (dict(N=0), -2), (dict(causal=2), -12), (dict(scale=float("nan")), -7), (dict(ws=None), -8),
    (dict(wsb=16), -8), (dict(ws=MIS), -6), (dict(o=P[1]), -11), (dict(ws=P[0]), -11),
])
def test_kouter_rejects_bad_arguments(L, kw, status):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=16, d=64, scale=0.1, causal=0,
             dtype=fa.FATTN_BF16, ws=P[5], wsb=1 << 20)
    a.update(kw)
    assert fa.fattn_fwd_kouter(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                               a["scale"], a["causal"], a["dtype"], a["ws"], a["wsb"]) == status


# --------------------------------------------------------------------------------------------
# Dropout


@pytest.mark.parametrize("p,dtype,status", [
    (1.0, 2, -13), (-0.1, 2, -13), (float("nan"), 2, -13), (1.5, 1, -13), (0.1, 0, -4), (0.1, 7, -4),
])
def test_fwd_dropout_rejects_bad_arguments(L, p, dtype, status):
    assert fa.fattn_fwd_dropout(P[0], P[1], P[2], P[3], P[4], 1, 1, 16, 64, 0.1, 0, dtype, p, 1) == status


@pytest.mark.parametrize("kw,status", [
    (dict(p=1.0), -13), (dict(p=-1e-9), -13), (dict(dq=None), -1), (dict(ws=None), -8), (dict(dtype=0), -4),
    (dict(dk=P[0]), -11), (dict(d=96), -3), (dict(causal=4), -12),
])
def test_bwd_dropout_rejects_bad_arguments(L, kw, status):
    a = dict(p=0.2, dq=P[6], dk=P[7], ws=P[9], dtype=2, d=64, causal=0)
    a.update(kw)
    assert fa.fattn_bwd_dropout(P[0], P[1], P[2], P[3], P[4], P[5], a["dq"], a["dk"], P[8], 1, 1, 16, a["d"], 0.1,
                                a["causal"], a["dtype"], a["p"], 7, a["ws"], 1 << 20) == status


def test_dropout_seed_is_64_bit(L):
    # a seed above 2^32 passes the host checks (rejected here only for the fake NULL output)
    assert fa.fattn_fwd_dropout(P[0], P[1], P[2], None, P[4], 1, 1, 16, 64, 0.1, 0, 2, 0.3, 2**63 + 5) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(m=None), -1), (dict(q=None), -1), (dict(dtype=0), -4), (dict(d=96), -3), (dict(N=0), -2),
    (dict(causal=5), -12), (dict(scale=float("inf")), -7), (dict(o=MIS), -6), (dict(o=P[5]), -11),
    (dict(lse=P[0]), -11),
])
def test_blocksparse_rejects_bad_arguments(L, kw, status):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], m=P[5], N=300, d=64, causal=0, dtype=2, scale=0.1)
    a.update(kw)
    assert fa.fattn_fwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 2, a["N"], a["d"], a["scale"],
                                    a["causal"], a["dtype"], a["m"]) == status


@pytest.mark.parametrize("kw,status", [
    (dict(m=None), -1), (dict(dq=None), -1), (dict(dtype=0), -4), (dict(d=96), -3), (dict(N=0), -2),
    (dict(causal=5), -12), (dict(scale=float("nan")), -7), (dict(dq=MIS), -6), (dict(dq=P[3]), -11),
    (dict(dk=P[10]), -11), (dict(ws=P[10]), -11), (dict(ws=None), -8), (dict(wsb=16), -8),
])
def test_bwd_blocksparse_rejects_bad_arguments(L, kw, status):
    # P[10] plays the block mask: an output or the workspace equal to it is an alias
    a = dict(m=P[10], dq=P[6], dk=P[7], ws=P[9], wsb=1 << 20, N=300, d=64, causal=0, dtype=2, scale=0.1)
    a.update(kw)
    m = a["m"]
    assert fa.fattn_bwd_blocksparse(P[0], P[1], P[2], P[3], P[4], P[5], a["dq"], a["dk"], P[8], 1, 2, a["N"],
                                    a["d"], a["scale"], a["causal"], a["dtype"], m, a["ws"], a["wsb"]) == status


def bwd_noalloc(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], dO=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8],
             B=2, H=3, N=100, d=128, scale=0.088, causal=1, dtype=fa.FATTN_BF16, stream=None)
    a.update(kw)
    return fa.fattn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"], a["dq"], a["dk"],
                                a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                                a["dtype"], a["stream"])


def test_bwd_noalloc_buffer_size(L):
    assert fa.fattn_bwd_noalloc_max_bytes() == 16 << 20


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(dv=0), -1), (dict(d=96), -3), (dict(dtype=fa.FATTN_F32), -4),
    (dict(N=0), -2), (dict(causal=2), -12), (dict(scale=math.inf), -7), (dict(dk=MIS), -6),
    (dict(dq=P[0]), -11), (dict(dk=P[6]), -11),
    # the D vector of B * H * N rows must fit the 16 MiB static buffer (4,194,304 rows)
    (dict(B=1, H=1, N=4194305), -14), (dict(B=4, H=8, N=131073), -14),
    (dict(B=64, H=64, N=1025, d=64), -14),
])
def test_bwd_noalloc_rejects_bad_arguments(L, kw, status):
    assert bwd_noalloc(**kw) == status
