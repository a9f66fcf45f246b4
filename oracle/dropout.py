"""Float64 attention with dropout on the probabilities, and the counter-based keep mask.

Test infrastructure only: the product path never imports it.

Page "mianstack q-0277" (section on whether the result changes) names dropout as one source of
numeric difference between implementations; the pages fix no convention for it. The readings
taken here:

* Dropout acts on the softmax probabilities: with keep mask M (1 = kept) and drop probability p,
  O = ((P * M) / (1 - p)) V, where P = softmax(S) is the undropped softmax. LSE is the undropped
  statistic (the backward rebuilds P from it).
* The keep decision for (head bh = b*H + h, query row i, key j) comes from the counter-based
  generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
  1, 2, 3", SC 2011), which both this oracle and the kernels implement from its definition:
  counter (j // 8, i, bh, 0), key (seed mod 2^32, seed // 2^32). One call covers 8 keys with
  16 bits each: key j takes field f = j % 8, the low half (f < 4) or the high half (f >= 4) of
  output word f % 4, as x in [0, 2^16). The key is kept iff x >= floor(p * 2^16), so
  P(keep) = 1 - p up to 2^-16.
* Backward, by the chain rule through O = Pd V with Pd = P * M / (1 - p):
  dV = Pd^T dO;  dP = (dO V^T) * M / (1 - p);  D = rowsum(dO * O) (= rowsum(P * dP));
  dS = P * (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.

Philox4x32 round (one of ten; the key is bumped by the Weyl constants between rounds):
  (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 (32 x 32 -> 64-bit products)
  c' = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
with M0 = 0xD2511F53, M1 = 0xCD9E8D57, W0 = 0x9E3779B9, W1 = 0xBB67AE85.
"""
from __future__ import annotations

import numpy as np

from . import attention

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32-10 of one counter (4 words) and key (2 words), plain Python integers."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in ctr)
    k0, k1 = (int(x) & MASK32 for x in key)
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK32, p1 & MASK32, ((p0 >> 32) ^ c3 ^ k1) & MASK32, p0 & MASK32
    return c0, c1, c2, c3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """The same generator on numpy arrays of counters (broadcast); returns 4 uint64 arrays."""
    c = [np.asarray(x, np.uint64) & np.uint64(MASK32) for x in (c0, c1, c2, c3)]
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & MASK32)
    k1 = np.uint64(int(k1) & MASK32)
    m = np.uint64(MASK32)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + W0) & MASK32)
            k1 = np.uint64((int(k1) + W1) & MASK32)
        p0 = np.uint64(M0) * c0  # < 2^64: both factors < 2^32
        p1 = np.uint64(M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0) & m, p1 & m, ((p0 >> np.uint64(32)) ^ c3 ^ k1) & m, p0 & m
    return c0, c1, c2, c3


def threshold(p):
    """Integer threshold floor(p * 2^16) of drop probability p in [0, 1)."""
    p = float(np.float32(p))
    if not (0.0 <= p < 1.0):
        raise ValueError("drop probability must be in [0, 1)")
    return int(np.floor(p * 65536.0))


def keep_field(words, j):
    """The 16-bit field of key j (j % 8) in the 4 output words of its call."""
    f = int(j) % 8
    return (int(words[f % 4]) >> (16 * (f // 4))) & 0xFFFF


def keep_mask(seed, p, bh, rows, keys):
    """Boolean keep mask [len(rows), len(keys)] of head bh."""
    rows = np.asarray(rows, np.int64)[:, None]
    keys = np.asarray(keys, np.int64)[None, :]
    words = philox4x32_10_np(keys >> 3, rows, bh, 0, seed & MASK32, (seed >> 32) & MASK32)
    f = keys & 7
    w = np.where((f & 3) == 0, words[0], np.where((f & 3) == 1, words[1], np.where((f & 3) == 2, words[2], words[3])))
    x = (w >> (np.uint64(16) * (f >> 2).astype(np.uint64))) & np.uint64(0xFFFF)
    return x >= np.uint64(threshold(p))


def forward_slice(q, k, v, scale, causal, p, seed, bh):
    """O [N, d] and the undropped LSE [N] of one (b, h) slice with dropout on P."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    n = q.shape[0]
    s = (q @ k.T) * scale
    if causal:
        s[np.arange(k.shape[0])[None, :] > np.arange(n)[:, None]] = -np.inf
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    prob = e / l[:, None]
    keep = keep_mask(seed, p, bh, np.arange(n), np.arange(k.shape[0]))
    pd = np.where(keep, prob, 0.0) / (1.0 - float(np.float32(p)))
    return pd @ v, m + np.log(l)


def backward_slice(q, k, v, do, scale, causal, p, seed, bh):
    """dQ, dK, dV (float64) of one slice with dropout, by the chain rule above."""
    q, k, v, do = (np.asarray(t, np.float64) for t in (q, k, v, do))
    n = q.shape[0]
    o, lse = forward_slice(q, k, v, scale, causal, p, seed, bh)
    s = (q @ k.T) * scale
    if causal:
        s[np.arange(k.shape[0])[None, :] > np.arange(n)[:, None]] = -np.inf
    prob = np.exp(s - lse[:, None])
    keep = keep_mask(seed, p, bh, np.arange(n), np.arange(k.shape[0]))
    inv_keep = 1.0 / (1.0 - float(np.float32(p)))
    pd = np.where(keep, prob, 0.0) * inv_keep
    dv = pd.T @ do
    dp = np.where(keep, do @ v.T, 0.0) * inv_keep
    dvec = np.sum(do * o, axis=1)
    ds = prob * (dp - dvec[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


def forward(q, k, v, scale, causal, p, seed, heads=None):
    """O [B,H,N,d], LSE [B,H,N] with dropout; ``heads`` limits the evaluated (b, h) pairs."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    o = np.full((B, H, N, d), np.nan)
    lse = np.full((B, H, N), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        o[b, h], lse[b, h] = forward_slice(q[b, h], k[b, h], v[b, h], scale, causal, p, seed, b * H + h)
    return o, lse


def backward(q, k, v, do, scale, causal, p, seed, heads=None):
    """dQ, dK, dV [B,H,N,d] with dropout; ``heads`` limits the evaluated (b, h) pairs."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    out = [np.full((B, H, N, d), np.nan) for _ in range(3)]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        g = backward_slice(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, p, seed, b * H + h)
        for t in range(3):
            out[t][b, h] = g[t]
    return tuple(out)


# the undropped definition, for the p = 0 reduction
undropped_forward_slice = attention.forward_slice
