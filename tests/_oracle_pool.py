"""Test-side drivers that evaluate the fp64 oracle over many independent units at once.

The oracle's own functions do all the arithmetic; this module only splits a workload into
units whose results do not depend on each other -- one (sequence, query head) pair of a
prefill, one sequence of a decode -- and runs them on a thread pool with single-threaded
BLAS, so that the full tensors of the larger workloads can be compared in seconds. NumPy
releases the interpreter lock inside its matrix products and element-wise loops, which is
where the time goes.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import workloads as W
from oracle import gqa_oracle as O


def pool_size() -> int:
    """Worker threads: the host's CPUs, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _blas_single_thread():
    try:
        import threadpoolctl
        return threadpoolctl.threadpool_limits(1)
    except Exception:  # no threadpoolctl: BLAS keeps its own threading
        import contextlib
        return contextlib.nullcontext()


def prefill_full(case: W.PrefillCase, window: int = 0, block_mask=None, workers: int | None = None):
    """``oracle.prefill`` of a whole case, evaluated per (sequence, query head): the prologue
    on every token (``oracle.qk_norm_rope``), then ``oracle.attend`` on each head's slice
    (one query head against its KV head g = floor(i / h)). Returns [N, H, d] float64."""
    q, k, v = case.f64("q"), case.f64("k"), case.f64("v")
    qt, kt = O.qk_norm_rope(q, k, case.positions, case.f64("q_norm_w"), case.f64("k_norm_w"),
                            case.eps, case.theta)
    h = case.H // case.G
    out = np.zeros_like(q)
    units = []
    for b in range(case.B):
        s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        if e > s:
            units += [(s, e, i) for i in range(case.H)]
    units.sort(key=lambda u: -(u[1] - u[0]))  # longest first

    def run(u):
        s, e, i = u
        g = i // h
        out[s:e, i:i + 1] = O.attend(qt[s:e, i:i + 1], kt[s:e, g:g + 1], v[s:e, g:g + 1],
                                     case.causal, None, window, block_mask)

    with _blas_single_thread(), cf.ThreadPoolExecutor(workers or pool_size()) as ex:
        list(ex.map(run, units))
    return out


def decode_all(case: W.DecodeCase, append: bool = True, workers: int | None = None):
    """``oracle.decode_one`` for every sequence of a decode case (each sequence's cache rows
    regenerated from its own seeded stream). Returns (out [B, H, d], k_slots, v_slots) with
    the appended rows per sequence (None where nothing was appended)."""
    out = np.zeros((case.B, case.H, case.d))
    k_slots = [None] * case.B
    v_slots = [None] * case.B
    q = case.f64("q")
    kn, vn = case.f64("k_new"), case.f64("v_new")
    gq, gk = case.f64("q_norm_w"), case.f64("k_norm_w")

    def run(b):
        k, v = case.cache_rows(b)
        o, ks, vs = O.decode_one(q[b], W.to_f64(k, case.dtype), W.to_f64(v, case.dtype),
                                 int(case.seq_lens[b]), gq, gk, case.eps, case.theta,
                                 k_new=kn[b] if append else None,
                                 v_new=vn[b] if append else None)
        out[b] = o
        k_slots[b], v_slots[b] = ks, vs

    order = sorted(range(case.B), key=lambda b: -int(case.seq_lens[b]))
    with _blas_single_thread(), cf.ThreadPoolExecutor(workers or pool_size()) as ex:
        list(ex.map(run, order))
    return out, k_slots, v_slots


def sample_rows(case: W.PrefillCase, n_min: int = 512, seed: int = 0, tile: int = 64,
                cols_per_block: int = 128):
    """At least ``n_min`` packed query rows of a case: in every sequence rows 0 and 1, the
    last two rows, both sides of every 16th key-tile boundary and of the first and last
    column-block boundaries (a block holds cols_per_block / h positions), then seeded
    uniform rows until the count is reached."""
    rng = np.random.default_rng(seed)
    h = case.H // case.G
    ppb = max(1, cols_per_block // h)
    rows = set()
    for b in range(case.B):
        s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        T = e - s
        if T == 0:
            continue
        fixed = [0, 1, T - 2, T - 1, ppb - 1, ppb, T - ppb - 1, T - ppb]
        for bnd in range(tile, T, 16 * tile):
            fixed += [bnd - 1, bnd]
        rows.update(s + r for r in fixed if 0 <= r < T)
    while len(rows) < min(n_min, case.N):
        rows.update(int(x) for x in rng.integers(0, case.N, size=n_min - len(rows)))
    return np.array(sorted(rows), dtype=np.int64)
