"""Process-pool runner for the fp64 oracle (test infrastructure only).

Splits a problem into independent sub-problems and calls
``oracle.attention.forward`` / ``backward`` on each in a freshly spawned
worker process with one BLAS thread (spawned, not forked, so workers never
inherit a GPU context from the caller).  It changes no arithmetic: every
number still comes from ``oracle.attention``; this module only slices,
re-indexes and reassembles.

A sub-problem is one batch row, one K/V head with its group of query heads,
and a contiguous range of local query rows [r_a, r_e).  Its rows attend only
keys in the window [w0, w1): w0 is the smallest document start of those rows
and w1 one past the last of them (a query never attends a key before its
document's start or after itself; Automodel page "feat(distributed):
block-diagonal varlen CP for packed sequences", Summary: block-causal per
document).  The sub-problem is therefore posed on the window alone: keys
[w0, w1) as a row of w1 - w0 tokens whose documents are the row's documents
clipped to the window (w0 is a document start, so only the last one is
cut), and the rows as a chunk at row_offset + r_a - w0.  Padding rows (past
the row's documents) are left out; they keep O = 0, LSE = -inf, dQ = 0.
dK / dV of a sub-problem are partial sums over its rows; the parent adds
them into the window's keys in job order, so the result does not depend on
the order workers finish in.
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
    idx, kind, b, g, r_a, w0, q, k, v, do, docs, row_offset, scale, block_rows, rows, drop = job
    _limit_threads()
    if kind == "fwd":
        res = A.forward(q, k, v, docs, row_offset, scale, block_rows=block_rows, rows=rows, dropout=drop)
    else:
        res = A.backward(q, k, v, do, docs, row_offset, scale, block_rows=block_rows, rows=rows, dropout=drop)
    return idx, kind, b, g, r_a, w0, res


def host_cores():
    """Cores this process may run on."""
    return len(os.sched_getaffinity(0))


def default_workers():
    """One worker per allowed core, but no more than the thread budget the
    environment sets (OMP_NUM_THREADS), when it sets one."""
    n = host_cores()
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _doc_starts(lens, seq_len):
    """doc_start of every position of the row (-1 on padding)."""
    start = np.full(seq_len, -1, np.int64)
    pos = 0
    for L in lens:
        start[pos:pos + L] = pos
        pos += L
    return start


def _clip_docs(lens, w0, w1):
    """Lengths of the row's documents clipped to the window [w0, w1)."""
    out, pos = [], 0
    for L in lens:
        lo, hi = max(pos, w0), min(pos + L, w1)
        if hi > lo:
            out.append(hi - lo)
        pos += L
    return out


def _pieces(start, row_offset, q_len, rows, n_pieces, align):
    """Split the local rows into at most n_pieces contiguous ranges of about
    equal work (allowed pairs + 1 per row), with bounds on multiples of
    align.  Returns a list of (r_a, r_b, subset or None)."""
    i = np.arange(q_len) + row_offset
    cost = np.where(start[i] >= 0, i - start[i] + 1, 0).astype(np.float64) + 1.0
    if rows is not None:
        sel = np.zeros(q_len, bool)
        sel[np.asarray(sorted(rows), np.int64)] = True
        cost = np.where(sel, cost, 0.0)
    csum = np.concatenate([[0.0], np.cumsum(cost)])
    bounds = [0]
    for p in range(1, n_pieces):
        t = int(np.searchsorted(csum, csum[-1] * p / n_pieces))
        t = min(q_len, (t // align) * align)
        if t > bounds[-1]:
            bounds.append(t)
    if bounds[-1] < q_len:
        bounds.append(q_len)
    out = []
    for r_a, r_b in zip(bounds[:-1], bounds[1:]):
        sub = None if rows is None else [t for t in rows if r_a <= t < r_b]
        if sub is None or sub:
            out.append((r_a, r_b, sub))
    return out


def run(q, k, v, do, doc_lens_rows, row_offset, scale, block_rows=256, rows=None, workers=None,
        want=("fwd", "bwd"), pieces=None, dropout=None):
    """Returns a dict with 'o', 'lse' (if 'fwd' in want) and 'dq', 'dk', 'dv'
    (if 'bwd' in want), all float64, layouts as in oracle.attention.  ``rows``
    restricts the computation to a subset of local rows (as in
    oracle.attention).  ``pieces`` fixes the number of row ranges per (batch
    row, K/V head); by default there are enough for about four jobs per
    worker.  ``dropout`` is (p, seed, offset): every job draws the mask of
    the full problem's batch row, heads and positions."""
    B, L, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    workers = workers or default_workers()
    rows = None if rows is None else sorted(set(int(t) for t in rows))
    if pieces is None:
        pieces = max(1, -(-4 * workers // (B * Hkv)))
    align = block_rows or 1

    def jobs():
        idx = 0
        for b in range(B):
            lens = list(doc_lens_rows[b])
            start = _doc_starts(lens, S)
            for r_a, r_b, sub in _pieces(start, row_offset, L, rows, pieces, align):
                t = np.arange(r_a, r_b) if sub is None else np.asarray(sub, np.int64)
                real = t[start[t + row_offset] >= 0]
                if real.size == 0:
                    continue
                r_e = int(real.max()) + 1
                w0 = int(start[real + row_offset].min())
                w1 = r_e + row_offset
                docs = [_clip_docs(lens, w0, w1)]
                ro = row_offset + r_a - w0
                sub_rows = None if sub is None else [int(x) - r_a for x in real]
                for kind in want:
                    for g in range(Hkv):
                        hs = slice(g * G, (g + 1) * G)
                        drop = None if dropout is None else A.Dropout(
                            dropout[0], dropout[1], dropout[2], Hq, b0=b, h0=g * G, pos0=w0)
                        yield (idx, kind, b, g, r_a, w0,
                               np.ascontiguousarray(q[b:b + 1, r_a:r_e, hs]),
                               np.ascontiguousarray(k[b:b + 1, w0:w1, g:g + 1]),
                               np.ascontiguousarray(v[b:b + 1, w0:w1, g:g + 1]),
                               None if (kind == "fwd" or do is None)
                               else np.ascontiguousarray(do[b:b + 1, r_a:r_e, hs]),
                               docs, ro, scale, block_rows, sub_rows, drop)
                        idx += 1

    out = {}
    if "fwd" in want:
        out["o"] = np.zeros((B, L, Hq, d))
        out["lse"] = np.full((B, Hq, L), -np.inf)
    if "bwd" in want:
        out["dq"] = np.zeros((B, L, Hq, d))
        out["dk"] = np.zeros((B, S, Hkv, d))
        out["dv"] = np.zeros((B, S, Hkv, d))
    pool = mp.get_context("spawn").Pool(workers) if workers > 1 else None
    try:
        # imap keeps job order, so the dK / dV partial sums are added in a
        # fixed order whatever order the workers finish in
        results = pool.imap(_work, jobs()) if pool is not None else map(_work, jobs())
        for _idx, kind, b, g, r_a, w0, res in results:
            hs = slice(g * G, (g + 1) * G)
            if kind == "fwd":
                o_, lse_ = res
                n = o_.shape[1]
                out["o"][b, r_a:r_a + n, hs] = o_[0]
                out["lse"][b, hs, r_a:r_a + n] = lse_[0]
            else:
                dq_, dk_, dv_ = res
                n, nw = dq_.shape[1], dk_.shape[1]
                out["dq"][b, r_a:r_a + n, hs] = dq_[0]
                out["dk"][b, w0:w0 + nw, g] += dk_[0, :, 0]
                out["dv"][b, w0:w0 + nw, g] += dv_[0, :, 0]
    finally:
        if pool is not None:
            pool.close()
            pool.join()
    return out
