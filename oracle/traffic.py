"""Analytic HBM-traffic model of naive versus tiled attention (one head, one sample).

Test and report infrastructure only.

Page "从零实现 FlashAttention-2" (hands-on section) describes ``memory_work(N, d)``: count the
full N x N matrix touches and the total bytes of both designs, and print them for N = 128..4096.
It does not print the numbers, so the counts here are this model's reading of its prose:

* Naive: S = QK^T is written to HBM, read back by the softmax, P is written and read again by
  the PV product (the page's "three HBM round trips" of the N x N tensor: the score kernel's
  store, the softmax kernel's load and store, the PV kernel's load). That is 4 one-way passes of
  N*N elements, plus reading Q, K, V and writing O (4 N d elements).
* Tiled (FlashAttention): no N x N tensor touches HBM; Q, K, V are read once, O is written once
  and the per-row statistic (one fp32 LSE per row) is written: 4 N d elements + 4 N bytes.

``tiled_bytes_with_rereads`` adds what the pages leave out: every query block of Br rows reads
all of K and V again unless a cache holds them, so the tiled traffic without any cache reuse is
2 N d (N / Br) elements for K and V instead of 2 N d.

``loop_order_bytes`` counts, for either loop order (page 2, FA-1 to FA-2 section), the bytes a
kernel that keeps nothing in a cache between tiles must move, visit by visit:

* Q-outer: each query block is read once and its O (elem_bytes) and LSE (4 B) written once;
  every visited (i, j) pair reads key/value block j (2 rows x d elements per key).
* K-outer: each key/value block is read once; every visited (i, j) pair reads query block i, and
  the block's running state (u in float32 plus m and l, (d + 2) x 4 B per row) is read back
  unless it is the block's first visit and written out unless it is its last, when O and LSE
  are written instead.
"""
from __future__ import annotations

import math


def memory_work(N: int, d: int, elem_bytes: int = 2) -> dict:
    naive_touches = 4
    naive_bytes = naive_touches * N * N * elem_bytes + 4 * N * d * elem_bytes
    flash_bytes = 4 * N * d * elem_bytes + 4 * N
    return {
        "N": N,
        "d": d,
        "naive_nn_touches": naive_touches,
        "naive_nn_elements": naive_touches * N * N,
        "naive_bytes": naive_bytes,
        "flash_nn_touches": 0,
        "flash_nn_elements": 0,
        "flash_bytes": flash_bytes,
    }


def tiled_bytes_with_rereads(N: int, d: int, Br: int, elem_bytes: int = 2, causal: bool = False) -> int:
    """Tiled bytes if K/V are fetched from HBM for every query block (no cache reuse)."""
    nblk = math.ceil(N / Br)
    kv_reads = 2 * N * d * elem_bytes * nblk
    if causal:
        kv_reads = sum(2 * min(N, (i + 1) * Br) * d * elem_bytes for i in range(nblk))
    return 2 * N * d * elem_bytes + kv_reads + 4 * N


def traffic_table(seq_lengths, d: int = 64, elem_bytes: int = 2):
    return [memory_work(N, d, elem_bytes) for N in seq_lengths]


def print_traffic_table(seq_lengths=(128, 256, 512, 1024, 2048, 4096), d: int = 64, elem_bytes: int = 2):
    rows = traffic_table(seq_lengths, d, elem_bytes)
    print(f"{'N':>6} {'naive NxN elems':>16} {'naive MiB':>10} {'flash NxN':>10} {'flash MiB':>10}")
    for r in rows:
        print(f"{r['N']:>6} {r['naive_nn_elements']:>16} {r['naive_bytes'] / 2**20:>10.3f} "
              f"{r['flash_nn_elements']:>10} {r['flash_bytes'] / 2**20:>10.3f}")
    return rows


def loop_order_bytes(N: int, d: int, Br: int, Bc: int, order: str, causal: bool = False,
                     elem_bytes: int = 2) -> int:
    """HBM bytes of one head for ``order`` in {"q_outer", "k_outer"}, with no cache reuse."""
    if order not in ("q_outer", "k_outer"):
        raise ValueError(order)
    q_blocks = [(i0, min(N, i0 + Br)) for i0 in range(0, N, Br)]
    k_blocks = [(j0, min(N, j0 + Bc)) for j0 in range(0, N, Bc)]
    total = 0
    if order == "q_outer":
        for i0, i1 in q_blocks:
            rows = i1 - i0
            total += rows * d * elem_bytes                      # Q block, once
            for j0, j1 in k_blocks:
                if causal and j0 > i1 - 1:
                    break
                total += 2 * (j1 - j0) * d * elem_bytes         # K and V block, every visit
            total += rows * d * elem_bytes + rows * 4           # O and LSE, once
        return total
    for j0, j1 in k_blocks:
        total += 2 * (j1 - j0) * d * elem_bytes                 # K and V block, once
    state = (d + 2) * 4                                         # u, m, l per row, float32
    for i0, i1 in q_blocks:
        rows = i1 - i0
        visits = [j0 for j0, _ in k_blocks if not (causal and j0 > i1 - 1)]
        for n, _ in enumerate(visits):
            total += rows * d * elem_bytes                      # Q block, every visit
            if n > 0:
                total += rows * state                           # state read back
            if n < len(visits) - 1:
                total += rows * state                           # state written out
            else:
                total += rows * d * elem_bytes + rows * 4       # O and LSE at the last visit
    return total
