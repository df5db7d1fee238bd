"""Process-pool runner for the fp64 oracle (test infrastructure only).

Splits a problem into its independent sub-problems -- one per (batch row,
K/V head): that head's group of query heads against its K/V -- and calls
``oracle.attention.forward`` / ``backward`` on each in a freshly spawned
worker process with one BLAS thread (spawned, not forked, so workers never
inherit a GPU context from the caller).  It changes no arithmetic: every
number still comes from ``oracle.attention``.  Used by the GPU parity tests
and the benchmark's CPU baseline.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from . import attention as A


def _limit_threads():
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass


def _work(job):
    kind, b, g, q, k, v, do, docs, row_offset, scale, block_rows, rows = job
    _limit_threads()
    if kind == "fwd":
        return kind, b, g, A.forward(q, k, v, docs, row_offset, scale, block_rows=block_rows, rows=rows)
    return kind, b, g, A.backward(q, k, v, do, docs, row_offset, scale, block_rows=block_rows, rows=rows)


def default_workers():
    return max(1, min(len(os.sched_getaffinity(0)), 8))


def run(q, k, v, do, doc_lens_rows, row_offset, scale, block_rows=256, rows=None, workers=None,
        want=("fwd", "bwd")):
    """Returns a dict with 'o', 'lse' (if 'fwd' in want) and 'dq', 'dk', 'dv'
    (if 'bwd' in want), all float64, layouts as in oracle.attention."""
    B, L, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv

    def jobs():
        for kind in want:
            for b in range(B):
                for g in range(Hkv):
                    hs = slice(g * G, (g + 1) * G)
                    yield (kind, b, g, np.ascontiguousarray(q[b:b + 1, :, hs]),
                           np.ascontiguousarray(k[b:b + 1, :, g:g + 1]),
                           np.ascontiguousarray(v[b:b + 1, :, g:g + 1]),
                           None if (kind == "fwd" or do is None) else np.ascontiguousarray(do[b:b + 1, :, hs]),
                           [list(doc_lens_rows[b])], row_offset, scale, block_rows, rows)

    out = {}
    if "fwd" in want:
        out["o"] = np.zeros((B, L, Hq, d))
        out["lse"] = np.full((B, Hq, L), -np.inf)
    if "bwd" in want:
        out["dq"] = np.zeros((B, L, Hq, d))
        out["dk"] = np.zeros((B, S, Hkv, d))
        out["dv"] = np.zeros((B, S, Hkv, d))
    n_jobs = len(want) * B * Hkv
    workers = min(workers or default_workers(), n_jobs)
    pool = mp.get_context("spawn").Pool(workers) if workers > 1 else None
    try:
        results = pool.imap_unordered(_work, jobs()) if pool is not None else map(_work, jobs())
        for kind, b, g, res in results:
            hs = slice(g * G, (g + 1) * G)
            if kind == "fwd":
                out["o"][b, :, hs] = res[0][0]
                out["lse"][b, hs] = res[1][0]
            else:
                out["dq"][b, :, hs] = res[0][0]
                out["dk"][b, :, g] = res[1][0, :, 0]
                out["dv"][b, :, g] = res[2][0, :, 0]
    finally:
        if pool is not None:
            pool.close()
            pool.join()
    return out
