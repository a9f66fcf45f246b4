"""Float64 block-sparse attention: exact attention restricted to allowed (query, key) blocks.

Test infrastructure only: the product path never imports it.

Page "FlashAttention为什么更快更省显存" (section on computing the table in blocks) notes that the
FlashAttention paper also discusses a block-sparse approximate variant and that it is a different
matter from exact attention; the pages give no definition. The reading taken here is the plainest
one consistent with tiled attention: a 0/1 mask over blocks of MB x MB (query, key) pairs decides
which blocks exist; scores in a zero block are -inf (the block is never computed), and within
the allowed blocks the result is exact softmax attention (also under the causal mask):

    S[i, j] = scale q_i . k_j  if  mask[i // MB, j // MB] = 1 (and j <= i when causal), else -inf
    O = softmax(S) V,  LSE = log sum_j exp S[i, j]

A row with no allowed key gets O = 0 and LSE = -inf (the empty state of the merge rule).
Approximation: against dense attention this drops every score in a zero block.

Backward: the chain rule through the same definition. Masked scores carry P = 0, so with
D_i = sum_t dO[i,t] O[i,t]:  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
dK = scale dS^T Q. A row with no allowed key has P = 0 everywhere: its dQ is 0 and it adds
nothing to dK or dV.
"""
from __future__ import annotations

import numpy as np

MB = 128


def dense_mask(block_mask, nq, nk, causal=False, mb=MB):
    """Element-level boolean mask [nq, nk] of a block mask [ceil(nq/mb), ceil(nk/mb)]."""
    bm = np.asarray(block_mask).astype(bool)
    m = bm[np.arange(nq)[:, None] // mb, np.arange(nk)[None, :] // mb]
    if causal:
        m = m & (np.arange(nk)[None, :] <= np.arange(nq)[:, None])
    return m


def forward_slice(q, k, v, scale, block_mask, causal=False, mb=MB):
    """O [N, d], LSE [N] of one (b, h) slice; ``block_mask`` [ceil(N/mb), ceil(N/mb)] of 0/1."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    n = q.shape[0]
    allowed = dense_mask(block_mask, n, k.shape[0], causal, mb)
    s = np.where(allowed, (q @ k.T) * scale, -np.inf)
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    rows = allowed.any(axis=1)
    if rows.any():
        sr = s[rows]
        m = sr.max(axis=1)
        e = np.exp(sr - m[:, None])
        l = e.sum(axis=1)
        o[rows] = (e @ v) / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


def forward(q, k, v, scale, block_mask, causal=False, heads=None, mb=MB):
    """O [B,H,N,d], LSE [B,H,N]; ``block_mask`` [B, H, nb, nb]; ``heads`` limits the (b, h) pairs."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    o = np.full((B, H, N, d), np.nan)
    lse = np.full((B, H, N), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        o[b, h], lse[b, h] = forward_slice(q[b, h], k[b, h], v[b, h], scale, block_mask[b, h], causal, mb)
    return o, lse


def backward_slice(q, k, v, do, scale, block_mask, causal=False, mb=MB):
    """dQ, dK, dV (float64) of one (b, h) slice, recomputing O and LSE from the definition."""
    q, k, v, do = (np.asarray(t, np.float64) for t in (q, k, v, do))
    n = q.shape[0]
    allowed = dense_mask(block_mask, n, k.shape[0], causal, mb)
    o, lse = forward_slice(q, k, v, scale, block_mask, causal, mb)
    rows = np.isfinite(lse)
    p = np.zeros((n, k.shape[0]))
    s = np.where(allowed, (q @ k.T) * scale, -np.inf)
    p[rows] = np.exp(s[rows] - lse[rows, None])
    dv = p.T @ do
    dp = do @ v.T
    dvec = np.sum(do * o, axis=1)
    ds = p * (dp - dvec[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


def backward(q, k, v, do, scale, block_mask, causal=False, heads=None, mb=MB):
    """dQ, dK, dV [B,H,N,d]; ``block_mask`` [B, H, nb, nb]; ``heads`` limits the (b, h) pairs."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    out = [np.full((B, H, N, d), np.nan) for _ in range(3)]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        g = backward_slice(q[b, h], k[b, h], v[b, h], do[b, h], scale, block_mask[b, h], causal, mb)
        for t in range(3):
            out[t][b, h] = g[t]
    return tuple(out)
