"""Float64 model of the tiled forward with the online softmax merge.

Test infrastructure only: it is checked against the definition in ``oracle.attention`` and pins
the algorithm the pages describe; the product path never imports it and it is never the
ground truth for the device.

Algorithm, in the pages' order and notation:

* The query rows are cut into blocks of Br rows (outer loop) and the key/value rows into blocks
  of Bc rows (inner loop); a query block stays put while every key/value block streams past
  (page "从零实现 FlashAttention-2", FA-1 to FA-2 section: Q outer, K/V inner).
* For a key block, each row gets its block statistics: the block max m_b, the exp-sum relative
  to it l_b = sum exp(s - m_b) and the unnormalised weighted values u_b = sum exp(s - m_b) v
  (page "mianstack q-0277", section on how the blockwise softmax stays normalised).
* The running state (m, l, u) of the row absorbs the block by the merge rule of the same
  section: m_new = max(m, m_b), l_new = exp(m - m_new) l + exp(m_b - m_new) l_b and
  u_new = exp(m - m_new) u + exp(m_b - m_new) u_b.
* After the last block, O = u / l (page 2, rescale-identity section; page 3, same section).
* ``forward_slice_kouter`` runs the same blocks in the other loop order (key/value blocks outer,
  query blocks inner, page 2's FA-1 to FA-2 section), keeping every query block's state between
  visits; it exists to pin the ablation of that order.
* Causal masking happens inside the block: a key index above the query index is dropped, and a
  block lying wholly above the diagonal is not visited at all (page 2, backward section and
  tips). Blocks at the end of the sequence may be short (page 2, tips).

A row whose block holds only masked keys has m_b = -inf and contributes nothing; the merge
below treats exp(-inf - m_new) as 0 and never forms -inf - (-inf).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _factor(m_part, m_new):
    """exp(m_part - m_new), with the -inf cases taken as 0 (empty state or empty block)."""
    out = np.zeros_like(m_new)
    ok = np.isfinite(m_part)
    out[ok] = np.exp(m_part[ok] - m_new[ok])
    return out


def block_stats(s, v):
    """Per-row (m_b, l_b, u_b) of one block of logits s [r, c] against values v [c, d]."""
    m_b = s.max(axis=1)
    e = np.zeros_like(s)
    ok = np.isfinite(m_b)
    e[ok] = np.exp(s[ok] - m_b[ok, None])
    return m_b, e.sum(axis=1), e @ v


def merge(m, l, u, m_b, l_b, u_b):
    """Two-state merge of running (m, l, u) with a block's (m_b, l_b, u_b), row-wise."""
    m = np.asarray(m, np.float64)
    m_b = np.asarray(m_b, np.float64)
    m_new = np.maximum(m, m_b)
    a = _factor(m, m_new)
    b = _factor(m_b, m_new)
    l_new = a * l + b * l_b
    u_new = a[..., None] * u + b[..., None] * u_b
    return m_new, l_new, u_new


def forward_slice(q, k, v, scale, Br, Bc, causal=False, trace=None):
    """Tiled forward of one (b, h) slice. Returns (O, LSE, visited_blocks).

    ``trace``, if a list, receives (i_block, j_block, m, l, u) copies after every merge, which is
    what the pages' worked examples print.
    """
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    N, d = q.shape
    Nk = k.shape[0]
    o = np.empty((N, v.shape[1]))
    lse = np.empty(N)
    visited = 0
    for i0 in range(0, N, Br):
        i1 = min(N, i0 + Br)
        qi = q[i0:i1]
        m = np.full(i1 - i0, NEG_INF)
        l = np.zeros(i1 - i0)
        u = np.zeros((i1 - i0, v.shape[1]))
        for j0 in range(0, Nk, Bc):
            if causal and j0 > i1 - 1:
                break  # every key of this and later blocks lies above the diagonal
            j1 = min(Nk, j0 + Bc)
            s = (qi @ k[j0:j1].T) * scale
            if causal:
                rows = np.arange(i0, i1)[:, None]
                cols = np.arange(j0, j1)[None, :]
                s = np.where(cols > rows, NEG_INF, s)
            m, l, u = merge(m, l, u, *block_stats(s, v[j0:j1]))
            visited += 1
            if trace is not None:
                trace.append((i0 // Br, j0 // Bc, m.copy(), l.copy(), u.copy()))
        o[i0:i1] = u / l[:, None]
        lse[i0:i1] = m + np.log(l)
    return o, lse, visited


def forward_slice_kouter(q, k, v, scale, Br, Bc, causal=False, trace=None):
    """The same tiled forward in the K-outer order (page 2, FA-1 to FA-2 section).

    The key/value block j is the outer loop and the query blocks the inner one, so every visit
    (i, j) reloads query block i and its running state (m, l, u), which the Q-outer order keeps
    on chip. The state of every query block lives in ``states`` between visits (HBM, on a
    device). Each row still merges its key blocks in increasing j with the same rule, so the
    result equals ``forward_slice`` exactly. Returns (O, LSE, visits); ``trace`` receives
    (i_block, j_block, m, l, u) after every merge, in visiting order.
    """
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    N, d = q.shape
    Nk = k.shape[0]
    states = {}
    visits = 0
    for j0 in range(0, Nk, Bc):
        j1 = min(Nk, j0 + Bc)
        for i0 in range(0, N, Br):
            i1 = min(N, i0 + Br)
            if causal and j0 > i1 - 1:
                continue  # this key block lies wholly above the diagonal of query block i
            m, l, u = states.get(i0, (np.full(i1 - i0, NEG_INF), np.zeros(i1 - i0),
                                      np.zeros((i1 - i0, v.shape[1]))))
            s = (q[i0:i1] @ k[j0:j1].T) * scale
            if causal:
                rows = np.arange(i0, i1)[:, None]
                cols = np.arange(j0, j1)[None, :]
                s = np.where(cols > rows, NEG_INF, s)
            states[i0] = merge(m, l, u, *block_stats(s, v[j0:j1]))
            visits += 1
            if trace is not None:
                trace.append((i0 // Br, j0 // Bc) + tuple(x.copy() for x in states[i0]))
    o = np.empty((N, v.shape[1]))
    lse = np.empty(N)
    for i0, (m, l, u) in states.items():
        o[i0:i0 + len(l)] = u / l[:, None]
        lse[i0:i0 + len(l)] = m + np.log(l)
    return o, lse, visits


def forward(q, k, v, scale, Br, Bc, causal=False):
    """Tiled forward over [B, H, N, d]; returns (O, LSE) in float64."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], _ = forward_slice(q[b, h], k[b, h], v[b, h], scale, Br, Bc, causal)
    return o, lse


def wrong_blockwise_sum(q, k, v, scale, Bc):
    """Negative control: normalise every key block on its own and add the block outputs.

    Page 3 warns against exactly this; on its worked example it gives 30 instead of 50/3.
    """
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    out = np.zeros((q.shape[0], v.shape[1]))
    for j0 in range(0, k.shape[0], Bc):
        s = (q @ k[j0:j0 + Bc].T) * scale
        m_b, l_b, u_b = block_stats(s, v[j0:j0 + Bc])
        out += u_b / l_b[:, None]
    return out


def causal_blocks_visited(N, Br, Bc):
    """Number of (query block, key block) pairs the causal tile loop visits."""
    total = 0
    for i0 in range(0, N, Br):
        i1 = min(N, i0 + Br)
        total += math.ceil(i1 / Bc)
    return total
