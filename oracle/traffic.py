"""Work and traffic counts: the lesson kernels of the "fused attention" page, and the hot path.

Test infrastructure (see the package docstring).

Lesson kernels (page "fused attention" facts, block ``traffic``): one head, N
query and key rows of width d, float32 elements, no mask; tiles of B rows for
both queries and keys, G = ceil(N / B) query tiles.  Counting is done by
walking the kernels' loops (``walk_fused``, ``walk_unfused``), independently of
the closed forms the page prints (``closed_fused``, ``closed_unfused``):

* fused: each query tile loads its Q rows once, then for every key tile loads
  that tile of K and of V into shared memory (one barrier before and one after
  the tile's math), computes one score (d multiply-adds, d shared reads of K)
  and one P.V update (d multiply-adds, d shared reads of V) per (row, key),
  one exponential per (row, key) and one rescale exponential per (row, key
  tile), and finally writes its O rows;
* unfused (Algorithm 0 of the FlashAttention paper as the page quotes it):
  a scores kernel reads Q and, per query tile, K, and writes S; a softmax
  kernel reads S and writes P (one exponential per score); a P.V kernel reads
  P and, per query tile, V, and writes O.  Barrier and shared-memory counts of
  the unfused kernels depend on kernel details the page does not give and are
  not modelled.

Element counts are requests, not DRAM transactions, as on the page.
"""
from __future__ import annotations

import math


def walk_fused(N: int, d: int, B: int) -> dict:
    c = dict(globalReads=0, globalWrites=0, fma=0, exps=0, barriers=0, sharedReads=0, sharedWrites=0)
    for q0 in range(0, N, B):
        rows = min(B, N - q0)
        c["globalReads"] += rows * d  # Q rows, once per query tile
        for k0 in range(0, N, B):
            keys = min(B, N - k0)
            c["globalReads"] += 2 * keys * d  # K and V tile
            c["sharedWrites"] += 2 * keys * d
            c["barriers"] += 2
            for _r in range(rows):
                c["exps"] += 1  # rescale factor for this key tile
                c["fma"] += keys * 2 * d
                c["sharedReads"] += keys * 2 * d
                c["exps"] += keys
        c["globalWrites"] += rows * d  # O rows
    c["globalBytes"] = 4 * (c["globalReads"] + c["globalWrites"])
    c["extraMemoryBytes"] = 0
    c["sharedPerWorkgroupBytes"] = 4 * 2 * B * d
    return c


def walk_unfused(N: int, d: int, B: int) -> dict:
    c = dict(globalReads=0, globalWrites=0, fma=0, exps=0)
    # scores kernel
    for q0 in range(0, N, B):
        rows = min(B, N - q0)
        c["globalReads"] += rows * d
        for k0 in range(0, N, B):
            keys = min(B, N - k0)
            c["globalReads"] += keys * d
            c["fma"] += rows * keys * d
            c["globalWrites"] += rows * keys  # S
    # softmax kernel, one row at a time
    for _i in range(N):
        c["globalReads"] += N
        c["exps"] += N
        c["globalWrites"] += N  # P
    # P.V kernel
    for q0 in range(0, N, B):
        rows = min(B, N - q0)
        for k0 in range(0, N, B):
            keys = min(B, N - k0)
            c["globalReads"] += rows * keys + keys * d  # P tile and V tile
            c["fma"] += rows * keys * d
        c["globalWrites"] += rows * d
    c["globalBytes"] = 4 * (c["globalReads"] + c["globalWrites"])
    c["extraMemoryBytes"] = 4 * N * N
    return c


def closed_fused(N: int, d: int, B: int) -> dict:
    G = math.ceil(N / B)
    r = dict(globalReads=N * d + 2 * G * N * d, globalWrites=N * d, fma=2 * N * N * d, exps=N * N + N * G,
             barriers=2 * G * G, sharedReads=2 * N * N * d, sharedWrites=2 * G * N * d)
    r["globalBytes"] = 4 * (r["globalReads"] + r["globalWrites"])
    r["extraMemoryBytes"] = 0
    r["sharedPerWorkgroupBytes"] = 4 * 2 * B * d
    return r


def closed_unfused(N: int, d: int, B: int) -> dict:
    G = math.ceil(N / B)
    r = dict(globalReads=N * d + 2 * G * N * d + 2 * N * N, globalWrites=2 * N * N + N * d, fma=2 * N * N * d,
             exps=N * N)
    r["globalBytes"] = 4 * (r["globalReads"] + r["globalWrites"])
    r["extraMemoryBytes"] = 4 * N * N
    return r


def over_theta(kind: str, N: int, d: int, B: int, elements: int) -> float:
    """Traffic over the order of FlashAttention's Theorem 2 (M = 2 B d floats of workgroup memory)."""
    if kind == "fused":
        return elements / (N * N * d * d / (2 * B * d))
    return elements / (N * d + N * N)


def score_share(N: int, d: int, B: int) -> float:
    u = closed_unfused(N, d, B)
    return 4 * N * N / (u["globalReads"] + u["globalWrites"])
