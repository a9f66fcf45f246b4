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
