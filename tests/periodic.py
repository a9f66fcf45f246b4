"""Exact gradients of a periodic causal head from small oracle problems (test helper)."""
import math

import numpy as np

from oracle import attention as att


def block_problem(q64, k64, v64, do64, scale, b, nr):
    """dQ of the nr query rows of block b, and the block's gradient contributions to the keys,
    for a causal head whose rows repeat one 64-row block (Q, K, V and dO alike), from one small
    oracle problem.

    Row i = 64 b + r (r < nr) of that head holds the block's row r and sees b whole copies of the
    64-row key/value block plus the block's keys j <= r. A key seen c times enters the softmax as
    one key whose logit is raised by ln c: with one extra dimension, q' = [q, 1] and
    k' = [k, ln c / scale], the small problem below (b copies folded into 64 keys, then the nr
    keys of block b itself, causal with offset 64) has row r's exact O and LSE. Its gradients
    are then exact as well: dQ' restricted to the first d columns is row i's dQ, and a folded key
    carries the sum over its c copies, i.e. c times each copy's dK, dV.
    Returns (dq [nr, d], per-copy dK, dV of a folded key [64, d] (None if b == 0),
    dK, dV of block b's own keys [nr, d]).
    """
    d = q64.shape[1]
    qx = np.concatenate([q64[:nr], np.ones((nr, 1))], axis=1)
    own = np.concatenate([k64[:nr], np.zeros((nr, 1))], axis=1)
    if b == 0:
        dq, dk, dv = att.backward_slice(qx, own, v64[:nr], do64[:nr], scale, True)
        return dq[:, :d], None, None, dk[:, :d], dv
    folded = np.concatenate([k64, np.full((64, 1), math.log(b) / scale)], axis=1)
    kx = np.concatenate([folded, own])
    vx = np.concatenate([v64, v64[:nr]])
    dq, dk, dv = att.backward_slice(qx, kx, vx, do64[:nr], scale, True, causal_offset=64)
    return dq[:, :d], dk[:64, :d] / b, dv[:64] / b, dk[64:, :d], dv[64:]
