"""Seeded synthetic inputs for the attention workloads, shared by the tests and the benchmark.

This module only draws random numbers and rounds them to the storage dtype. It holds none of
the attention arithmetic, so the float64 oracle and the HIP path can both take their inputs
from here without sharing any of the method.

Every tensor is drawn iid N(0, 1) in float32 from its own counter-based stream
``SeedSequence([workload, variant, tensor_index])``, so drawing Q never depends on whether K
was drawn. Values are then rounded to the storage dtype with round-to-nearest-even; the
rounded values are returned as float32 arrays (exactly representable in the storage dtype)
together with their raw bits, so the device gets the identical bits and the oracle gets an
exact float64 upcast of them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Tensor stream indices.
_Q, _K, _V, _DO = 0, 1, 2, 3

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload: shape [B, H, N, d], storage dtype and mask set."""

    ident: int
    name: str
    dtype: str
    B: int
    H: int
    N: int
    d: int
    masks: tuple  # subset of ("noncausal", "causal")
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def shape(self) -> tuple:
        return (self.B, self.H, self.N, self.d)


# The five workloads, in the order the benchmark suite lists them.
WORKLOADS = {
    1: Workload(1, "single-head fp32 forward", "f32", 1, 1, 256, 64, ("noncausal", "causal")),
    2: Workload(2, "multi-head fp16 forward", "f16", 1, 8, 1024, 64, ("noncausal", "causal")),
    3: Workload(3, "prefill bf16 forward", "bf16", 4, 16, 4096, 128, ("causal",)),
    4: Workload(4, "long-context bf16 forward", "bf16", 1, 32, 16384, 128, ("noncausal", "causal")),
    5: Workload(5, "training bf16 forward+backward", "bf16", 2, 16, 4096, 128, ("causal",), True),
}


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """A decode-shaped workload: Nq new query rows per head against an Nk-long key/value cache."""

    ident: int
    name: str
    dtype: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    kv_seed: int  # seed of the key/value cache draw (shared by workloads over the same cache)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# Split-KV forward workloads: one query per head (token-by-token decode) and 16 (a block of
# draft tokens checked at once), both over the same 16384-key cache at d = 128.
DECODE_WORKLOADS = {
    6: DecodeWorkload(6, "decode bf16 split-KV forward", "bf16", 8, 32, 1, 16384, 128, 6),
    7: DecodeWorkload(7, "multi-token decode bf16 split-KV forward", "bf16", 8, 32, 16, 16384, 128, 6),
}

# Variants: 0 = base draw; 1 = every logit shifted by exactly +500 (Q[...,0] = 1 and
# K[...,0] += 500/scale, see ``shifted_pair``); 2 = the literal construction where only K[...,0]
# gets the +500/scale offset, so row i moves by 500*q[i,0].
VARIANT_BASE, VARIANT_SHIFT_EXACT, VARIANT_SHIFT_LITERAL = 0, 1, 2


def round_bits(x: np.ndarray, dtype: str):
    """Round float32 ``x`` to ``dtype`` with round-to-nearest-even.

    Returns ``(values, bits)``: ``values`` is float32 holding the rounded numbers exactly,
    ``bits`` is uint16 (f16/bf16) or uint32 (f32) holding the storage bits.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x, x.view(np.uint32)
    if dtype == "f16":
        h = x.astype(np.float16)  # numpy's float32->float16 cast is round-to-nearest-even
        return h.astype(np.float32), h.view(np.uint16)
    if dtype == "bf16":
        if not np.all(np.isfinite(x)):
            raise ValueError("bf16 rounding expects finite inputs")
        # finite floats have bits <= 0xFF7FFFFF, so adding at most 0x8000 stays within 32 bits
        u = x.view(np.uint32)
        r = (u + ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)) >> 16
        bits = r.astype(np.uint16)
        r <<= 16
        vals = r.view(np.float32)
        return vals, bits
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(shape, seed_words, dtype: str):
    """Draw one tensor iid N(0,1) in float32 from ``SeedSequence(seed_words)``, rounded to dtype."""
    rng = np.random.default_rng(np.random.SeedSequence(list(seed_words)))
    return round_bits(rng.standard_normal(shape, dtype=np.float32), dtype)


@dataclasses.dataclass
class Inputs:
    """Rounded inputs: float32 values (exact in ``dtype``) and their storage bits."""

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    bits: dict


def make_inputs(shape, dtype: str, seed: int, variant: int = VARIANT_BASE, with_do: bool = False,
                scale: float | None = None) -> Inputs:
    """Seeded Q, K, V (and dO) of ``shape`` = (B, H, N, d), rounded to ``dtype``.

    ``seed`` selects the stream family (the workload id for the five workloads). Variants 1 and
    2 add the +500 logit offset described at ``VARIANT_*``; they need ``scale``.
    """
    B, H, N, d = shape
    q, qb = draw(shape, (seed, variant, _Q), dtype)
    k, kb = draw(shape, (seed, variant, _K), dtype)
    v, vb = draw(shape, (seed, variant, _V), dtype)
    do = dob = None
    if with_do:
        do, dob = draw(shape, (seed, variant, _DO), dtype)
    if variant in (VARIANT_SHIFT_EXACT, VARIANT_SHIFT_LITERAL):
        if scale is None:
            raise ValueError("shifted variants need the softmax scale")
        q, k = q.copy(), k.copy()
        offset = np.float32(500.0 / scale)
        if variant == VARIANT_SHIFT_EXACT:
            q[..., 0] = 1.0
        k[..., 0] = k[..., 0] + offset
        q, qb = round_bits(q, dtype)
        k, kb = round_bits(k, dtype)
    bits = {"q": qb, "k": kb, "v": vb}
    if with_do:
        bits["do"] = dob
    return Inputs(dtype, q, k, v, do, bits)


def make_decode_inputs(B, H, nq, nk, d, dtype: str, seed: int, variant: int = VARIANT_BASE,
                       kv_seed: int | None = None, with_q: bool = True, with_kv: bool = True) -> Inputs:
    """Seeded Q [B, H, nq, d] and K, V [B, H, nk, d], rounded to ``dtype`` (no dO).

    K and V come from ``kv_seed`` (default ``seed``); ``with_q`` / ``with_kv`` = False skip a
    draw (the field is then None), so a shared cache is drawn once.
    """
    kv_seed = seed if kv_seed is None else kv_seed
    q = qb = k = kb = v = vb = None
    if with_q:
        q, qb = draw((B, H, nq, d), (seed, variant, _Q), dtype)
    if with_kv:
        k, kb = draw((B, H, nk, d), (kv_seed, variant, _K), dtype)
        v, vb = draw((B, H, nk, d), (kv_seed, variant, _V), dtype)
    return Inputs(dtype, q, k, v, None, {"q": qb, "k": kb, "v": vb})


def decode_workload_inputs(ident: int, with_q: bool = True, with_kv: bool = True) -> Inputs:
    """Inputs of decode workload ``ident`` (6, 7) at full size."""
    w = DECODE_WORKLOADS[ident]
    return make_decode_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, ident, kv_seed=w.kv_seed,
                              with_q=with_q, with_kv=with_kv)


def block_mask(B, H, nb, density, seed, diagonal=True):
    """Seeded 0/1 block mask [B, H, nb, nb] (uint8): each block kept with probability ``density``;
    with ``diagonal`` the diagonal blocks are always kept, so every query row has a key."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 77]))
    m = (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    if diagonal:
        m[..., np.arange(nb), np.arange(nb)] = 1
    return m


def unshifted_partner(inp: Inputs, scale: float) -> Inputs:
    """For variant 1, the tensors whose logits are exactly 500 lower than ``inp``'s.

    Q is unchanged (its column 0 is already 1); K's column 0 has the rounded offset
    (500/scale) taken back out, which is exact because the rounded column holds
    offset + an integer that the storage dtype represents.
    """
    k = inp.k.copy()
    k[..., 0] = k[..., 0] - np.float32(500.0 / scale)
    k2, kb = round_bits(k, inp.dtype)
    if not np.array_equal(k2, k):
        raise ValueError("offset removal is not exact for this dtype/scale")
    bits = dict(inp.bits)
    bits["k"] = kb
    return Inputs(inp.dtype, inp.q, k2, inp.v, inp.do, bits)


def workload_inputs(ident: int, variant: int = VARIANT_BASE, with_do: bool | None = None) -> Inputs:
    """Inputs of workload ``ident`` (1..5) at full size."""
    w = WORKLOADS[ident]
    if with_do is None:
        with_do = w.backward
    return make_inputs(w.shape, w.dtype, ident, variant, with_do, w.scale)
