"""Whole-layer driver of the fp64 oracle: runs the per-head steps over every head.

TEST INFRASTRUCTURE (tests, smoke check, CPU-baseline timing only).  Heads are
independent (routing is per head), so they run on a thread pool; numpy
releases the interpreter lock inside its array kernels, and the BLAS thread
count is pinned to one per worker so that workers do not oversubscribe cores.
"""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import crisp_oracle as co


def _blas_limit(n):
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:  # pragma: no cover - threadpoolctl missing
        import contextlib
        return contextlib.nullcontext()


def default_workers(cap: int = 16) -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return max(1, min(cap, avail))


def layer_selection(q_bits, k_bits, *, tau=0.2, alpha=1.0, gamma=0.95, k_min_tokens=1024,
                    heads=None, force_vs=None, workers=None, floor="mean", band=False, pe_per_row=False):
    """Routing and selection of every (batch, head) pair of one layer.

    ``q_bits`` [batch][h_q][n][d], ``k_bits`` [batch][h_kv][n][d] (bf16 bits).
    ``force_vs`` maps (b, h) -> bool to override a routing decision.
    Returns {(b, h): crisp_head result}.
    """
    B, H = q_bits.shape[:2]
    G = H // k_bits.shape[1]
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    force_vs = force_vs or {}

    def one(bh):
        b, h = bh
        q = co.bf16_to_f64(q_bits[b, h])
        k = co.bf16_to_f64(k_bits[b, h // G])
        return bh, co.crisp_head(q, k, tau=tau, alpha=alpha, gamma=gamma, k_min_tokens=k_min_tokens,
                                 force_vs=force_vs.get(bh), floor=floor, band=band, pe_per_row=pe_per_row)

    workers = workers or default_workers()
    with _blas_limit(1):
        with ThreadPoolExecutor(min(workers, len(todo)) or 1) as ex:
            return dict(ex.map(one, todo))


def layer_selection_flex(q_bits, k_bits, *, tau_jsd=0.1, gamma=0.95, k_min_tokens=1024,
                         heads=None, force_vs=None, workers=None):
    """FlexPrefill's routing and selection (flex_head) of every (batch, head) pair of one layer."""
    B, H = q_bits.shape[:2]
    G = H // k_bits.shape[1]
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    force_vs = force_vs or {}

    def one(bh):
        b, h = bh
        q = co.bf16_to_f64(q_bits[b, h])
        k = co.bf16_to_f64(k_bits[b, h // G])
        return bh, co.flex_head(q, k, tau_jsd=tau_jsd, gamma=gamma, k_min_tokens=k_min_tokens,
                                force_vs=force_vs.get(bh))

    workers = workers or default_workers()
    with _blas_limit(1):
        with ThreadPoolExecutor(min(workers, len(todo)) or 1) as ex:
            return dict(ex.map(one, todo))


def layer_attention(q_bits, k_bits, v_bits, rows_of, blocks_of, *, workers=None, q_rows=None):
    """Exact block-sparse attention on chosen query blocks.

    ``rows_of[(b, h)]`` is that head's list of key-block rows; ``blocks_of`` maps
    (b, h) -> iterable of query blocks to compute.  Returns {(b, h, qb): array}.
    K and V are converted once per KV head; of Q only the requested blocks' rows
    are converted (the rest of each head's array is allocated, never touched, so
    a long layer costs memory only for what is compared).
    """
    G = q_bits.shape[1] // k_bits.shape[1]
    B = co.BLOCK
    jobs = [(bh, qb) for bh, qbs in blocks_of.items() for qb in qbs]
    kv, qs = {}, {}
    for bh, qbs in blocks_of.items():
        b, h = bh
        if (b, h // G) not in kv:
            kv[(b, h // G)] = (co.bf16_to_f64(k_bits[b, h // G]),
                               co.bf16_to_f64(v_bits[b, h // G]))
        q = np.empty(q_bits.shape[2:], dtype=np.float64)
        for qb in qbs:
            q[qb * B:(qb + 1) * B] = co.bf16_to_f64(q_bits[b, h, qb * B:(qb + 1) * B])
        qs[bh] = q

    def one(job):
        bh, qb = job
        q, (k, v) = qs[bh], kv[(bh[0], bh[1] // G)]
        o = co.block_sparse_attention(q, k, v, rows_of[bh], q_blocks=[qb], q_rows=q_rows)[qb]
        return (bh[0], bh[1], qb), o

    workers = workers or default_workers()
    with _blas_limit(1):
        with ThreadPoolExecutor(min(workers, max(1, len(jobs)))) as ex:
            out = dict(ex.map(one, jobs))
    kv.clear()
    qs.clear()
    return out


def timed(fn, *a, **kw):
    t0 = time.perf_counter()
    r = fn(*a, **kw)
    return r, time.perf_counter() - t0
