"""Plain float64 attention: the definition written out, forward and analytic backward.

Test infrastructure only: the product path never imports this module.

Forward (page "FlashAttention为什么更快更省显存", opening formula; page "从零实现 FlashAttention-2",
section on why softmax needs a whole row, and its stable reference ``naive_attention`` that
subtracts the row max before the exponential):

    S = scale * Q K^T,  S[i, j] = -inf where causal and j > i + causal_offset
    m_i = max_j S[i, j],  P[i, j] = exp(S[i, j] - m_i),  l_i = sum_j P[i, j]
    O_i = (sum_j P[i, j] V_j) / l_i,  LSE_i = m_i + ln l_i

The per-row statistic kept for the backward is the natural-log logsumexp of the scaled logits.
The pages keep "the per-row max and sum" (page 2, backward section); LSE carries the same
information, since P = exp(S - LSE).

Backward (page 2, backward section: rebuild P from Q, K, V and the per-row statistics instead of
storing it). The pages print no gradient formulas; these follow from the forward by the chain
rule, for a loss L with dO = dL/dO:

    P = exp(S - LSE)          (masked entries are exactly 0)
    dV = P^T dO,  dP = dO V^T,  D_i = sum_t dO[i, t] O[i, t]  (= sum_j P[i, j] dP[i, j])
    dS = P * (dP - D[:, None]),  dQ = scale * dS K,  dK = scale * dS^T Q

Everything is computed in float64 over whole rows of S, a chunk of rows at a time so that the
N = 16384 workload fits in host memory. No online merge happens here.

Queries and keys of different lengths (decode against a key/value cache, page "mianstack
q-0277", backward section, which names the cache): the pages fix no causal convention for that
case. The reading taken here is that the Nq queries are the LAST Nq positions of the Nk-long
sequence, so query i sits at position i + (Nk - Nq) and sees keys j <= i + causal_offset with
causal_offset = Nk - Nq. With Nq == Nk the offset is 0 and this is the ordinary causal mask.
"""
from __future__ import annotations

import numpy as np

_CHUNK = 1024


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _masked_scores(q_rows, k, scale, causal, row0, causal_offset=0):
    """Scaled logits for query rows row0.. (one (b, h) slice); with ``causal``, -inf where key
    j > row + causal_offset."""
    s = (q_rows @ k.T) * scale
    if causal:
        rows = np.arange(row0, row0 + q_rows.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s[cols > rows + causal_offset] = -np.inf
    return s


def forward_slice(q, k, v, scale, causal=False, rows=None, chunk=_CHUNK, causal_offset=0):
    """O and LSE for one (b, h) slice. q: [Nq, d], k, v: [Nk, d]; float64 results.

    ``rows`` optionally restricts the computation to those query indices (then q holds all
    rows and only the selected ones are evaluated, in the order given). With ``causal``, query i
    sees keys j <= i + causal_offset; every evaluated row must see at least one key.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((idx.size, v.shape[1]))
    lse = np.empty(idx.size)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        s = (q[sel] @ k.T) * scale
        if causal:
            s[np.arange(k.shape[0])[None, :] > sel[:, None] + causal_offset] = -np.inf
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        out[c0:c0 + sel.size] = (p @ v) / l[:, None]
        lse[c0:c0 + sel.size] = m + np.log(l)
    return out, lse


def forward(q, k, v, scale, causal=False, rows=None, heads=None, causal_offset=0):
    """O [B,H,n,d] and LSE [B,H,n] for q [B,H,Nq,d] and k, v [B,H,Nk,d].

    ``heads`` optionally lists (b, h) pairs to evaluate (others are left NaN); ``rows`` limits
    every evaluated head to those query rows (n = len(rows)).
    """
    q = np.asarray(q)
    B, H, N, d = q.shape
    n = N if rows is None else len(rows)
    o = np.full((B, H, n, d), np.nan)
    lse = np.full((B, H, n), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        o[b, h], lse[b, h] = forward_slice(q[b, h], k[b, h], v[b, h], scale, causal, rows,
                                           causal_offset=causal_offset)
    return o, lse


def backward_slice(q, k, v, do, scale, causal=False, chunk=_CHUNK, causal_offset=0):
    """dQ [Nq, d], dK, dV [Nk, d] (float64) for one (b, h) slice, recomputing O and LSE from the
    definition; with ``causal``, query i sees keys j <= i + causal_offset (as in forward_slice)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    o, lse = forward_slice(q, k, v, scale, causal, chunk=chunk, causal_offset=causal_offset)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.sum(do * o, axis=1)
    for r0 in range(0, q.shape[0], chunk):
        r1 = min(q.shape[0], r0 + chunk)
        s = _masked_scores(q[r0:r1], k, scale, causal, r0, causal_offset)
        p = np.exp(s - lse[r0:r1, None])
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        ds = p * (dp - dvec[r0:r1, None])
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def backward(q, k, v, do, scale, causal=False, heads=None):
    """dQ, dK, dV [B,H,N,d] (float64); ``heads`` limits the evaluated (b, h) pairs."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    dq = np.full((B, H, N, d), np.nan)
    dk = np.full((B, H, N, d), np.nan)
    dv = np.full((B, H, N, d), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        dq[b, h], dk[b, h], dv[b, h] = backward_slice(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv


def softmax_unshifted_f32(x):
    """Negative control: softmax without the max shift, in float32.

    Page 2's stability check says this overflows to NaN once logits sit a few hundred above
    zero (exp(500) is inf in float32, and inf/inf is NaN); the stable form above does not.
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        return e / e.sum(axis=-1, keepdims=True)


def forward_unshifted_f32(q, k, v, scale, causal=False):
    """Negative control: whole attention with the unshifted float32 softmax (one slice)."""
    s = (np.asarray(q, np.float32) @ np.asarray(k, np.float32).T) * np.float32(scale)
    if causal:
        n = s.shape[0]
        s[np.arange(s.shape[1])[None, :] > np.arange(n)[:, None]] = -np.inf
    p = softmax_unshifted_f32(s)
    with np.errstate(invalid="ignore"):
        return p @ np.asarray(v, np.float32)
