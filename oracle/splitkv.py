"""Float64 model of split-KV attention: per-range partial results and their merge.

Test infrastructure only: the product path never imports it.

What is computed. The keys of a row are cut into consecutive ranges ("splits"). For each split
the row's attention over that range alone is a partial result (O_s, LSE_s): O_s is the softmax-
weighted mean of the split's values and LSE_s the natural-log exp-sum of the split's logits,
both from the definition in ``oracle.attention``. Partials are then merged with the two-state
rule of page "mianstack q-0277" (section on keeping the blockwise softmax normalised):

    m_new = max(m, m_b),  l_new = exp(m - m_new) l + exp(m_b - m_new) l_b,
    u_new = exp(m - m_new) u + exp(m_b - m_new) u_b,  O = u / l.

A partial enters the merge as the state (m, l, u) = (LSE_s, 1, O_s). That is the split's own
state (m_s, l_s, u_s) with every term divided by l_s = exp(LSE_s - m_s): the ratio u / l and the
sum m + ln l are unchanged, and the merge rule commutes with such a rescaling, so the merged
state is the one the whole row would have had. After the last partial, O = u / l and
LSE = m + ln l. The merge runs over the splits in order with ``oracle.tiled.merge``.

Readings where the pages are silent:
  * Partition: with num_splits = S and alignment A, every split holds L = A * ceil(Nk / (A * S))
    consecutive keys, split s covering [s L, min(Nk, (s + 1) L)); splits that start at or past
    Nk are empty. Splits then begin on tile boundaries of any tile size dividing A.
  * A split in which a row sees no key (empty split, or every key masked) has O_s = 0 and
    LSE_s = -inf: the empty state, which the merge leaves without effect.
  * A row that sees no key at all (Nk = 0) gets O = 0 and LSE = -inf.
  * Causal with Nq != Nk uses the bottom-right reading of ``oracle.attention`` (query i sees
    keys j <= i + Nk - Nq).
"""
from __future__ import annotations

import numpy as np

from . import attention, tiled

ALIGN = 64


def split_ranges(nk, num_splits, align=ALIGN):
    """[(k0, k1)] for splits 0..num_splits-1 of nk keys (empty splits have k0 == k1)."""
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    per = -(-nk // (align * num_splits)) * align if nk > 0 else align
    out = []
    for s in range(num_splits):
        k0 = min(nk, s * per)
        out.append((k0, min(nk, k0 + per) if k0 < nk else k0))
    return out


def partials_slice(q, k, v, scale, ranges, causal=False, causal_offset=0):
    """Per-split (O_s [S, Nq, d], LSE_s [S, Nq]) of one (b, h) slice over the given key ranges."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    nq, d = q.shape
    o = np.zeros((len(ranges), nq, v.shape[1]))
    lse = np.full((len(ranges), nq), -np.inf)
    for s, (k0, k1) in enumerate(ranges):
        if k1 <= k0:
            continue
        # rows that see at least one key of [k0, k1): all of them, or (causal) i + off >= k0
        rows = np.arange(nq)
        if causal:
            rows = rows[rows + causal_offset >= k0]
        if rows.size == 0:
            continue
        o[s, rows], lse[s, rows] = attention.forward_slice(
            q, k[k0:k1], v[k0:k1], scale, causal, rows=rows, causal_offset=causal_offset - k0)
    return o, lse


def combine(o_parts, lse_parts):
    """Merge partials (O_s [S, ..., d], LSE_s [S, ...]) into (O [..., d], LSE [...])."""
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    shape = lse_parts.shape[1:]
    m = np.full(shape, -np.inf)
    l = np.zeros(shape)
    u = np.zeros(shape + o_parts.shape[-1:])
    for s in range(lse_parts.shape[0]):
        m, l, u = tiled.merge(m, l, u, lse_parts[s], np.ones(shape), o_parts[s])
    o = np.zeros_like(u)
    lse = np.full(shape, -np.inf)
    ok = l > 0
    o[ok] = u[ok] / l[ok][..., None]
    lse[ok] = m[ok] + np.log(l[ok])
    return o, lse


def forward(q, k, v, scale, num_splits, causal=False, align=ALIGN, heads=None):
    """Split-KV forward for q [B,H,Nq,d], k, v [B,H,Nk,d].

    Returns (O [B,H,Nq,d], LSE [B,H,Nq], O_parts [S,B,H,Nq,d], LSE_parts [S,B,H,Nq]); ``heads``
    optionally lists the (b, h) pairs to evaluate (the others stay NaN).
    """
    q = np.asarray(q)
    B, H, nq, d = q.shape
    nk = np.asarray(k).shape[2]
    ranges = split_ranges(nk, num_splits, align)
    off = nk - nq
    op = np.full((num_splits, B, H, nq, d), np.nan)
    lp = np.full((num_splits, B, H, nq), np.nan)
    o = np.full((B, H, nq, d), np.nan)
    lse = np.full((B, H, nq), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        op[:, b, h], lp[:, b, h] = partials_slice(q[b, h], k[b, h], v[b, h], scale, ranges, causal, off)
        o[b, h], lse[b, h] = combine(op[:, b, h], lp[:, b, h])
    return o, lse, op, lp
