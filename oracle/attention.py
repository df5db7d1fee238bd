"""fp64 dense masked attention and its hand-derived backward (oracle; test
infrastructure only).

Source: Automodel page "feat(distributed): block-diagonal varlen CP for packed
sequences".  Summary: the varlen kernel and a dense masked-SDPA fallback
compute the same thing.  Motivation: each document's attention is exactly
block-causal.  Design overview, kernels.py: the dense [B,1,L,S] mask of the L
local query rows against all S keys; batch.py / packed.py and key property 1:
the local rows are the contiguous chunk [row_offset, row_offset + L) and K/V
cover the whole row.  The forward is the plain definition (scaled dot
products, mask, softmax, weighted sum of values).  The backward is derived
from the softmax Jacobian:
    dP_ij = dO_i . v_j
    r_i   = sum_j P_ij dP_ij
    dS_ij = P_ij (dP_ij - r_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i     (summed over the query heads sharing K)
    dV_j  = sum_i P_ij dO_i             (same)
It deliberately does not use rowsum(dO * O) for r_i.

Layouts (numpy, any float dtype; cast to float64 inside):
  q, do : [B, L, Hq, d]    rows are the chunk [row_offset, row_offset + L)
  k, v  : [B, S, Hkv, d]   the whole packed row
  o     : [B, L, Hq, d]    lse: [B, Hq, L] (natural log of the softmax
                           denominator in units of scaled logits)
  dq    : like q; dk, dv: like k (zero at keys no local row attends)
Grouped-query attention: query head h reads K/V head h // (Hq // Hkv).
Readings where the page is silent: the diagonal is attended (causal includes
j = i); a position past the sum of the row's document lengths is padding and
belongs to no document, so a padding query row has O = 0, LSE = -inf and
dQ = 0, and a padding key is never attended.

Modes: ``block_rows=None`` evaluates every query row against all S keys with
the full mask (the dense definition).  ``block_rows=R`` processes R rows at a
time against the key window [doc_start of the block's first real row, last
real row + 1); the keys it drops are all masked, so the result is the same
up to summation order.  ``rows`` restricts the computation to a subset of
local query rows (for sampled checks on large workloads).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import dropout as DR


@dataclasses.dataclass(frozen=True)
class Dropout:
    """Attention dropout (oracle.dropout): probability p, 64-bit seed and
    32-bit offset of the generator's counter, and where the arrays passed to
    forward / backward sit in the full problem -- the query-head count h_q of
    the full problem, the batch row and query head of their first row and
    head (b0, h0), and the row position of their key 0 (pos0) -- so a
    sub-problem draws the same mask as the full one."""
    p: float
    seed: int
    offset: int
    h_q: int
    b0: int = 0
    h0: int = 0
    pos0: int = 0

    def keep(self, b, h, rows, keys):
        """(Z, c) for local batch row b, local head h, row / key positions
        local to the arrays."""
        z = DR.keep_mask(self.seed, self.offset, self.b0 + b, self.h0 + h, self.h_q,
                         self.pos0 + np.asarray(rows), self.pos0 + np.asarray(keys), self.p)
        return z, DR.keep_scale(self.p)[1]


def _row_doc_start(lens, seq_len):
    start = np.full(seq_len, -1, np.int64)
    pos = 0
    for L in lens:
        start[pos:pos + L] = pos
        pos += L
    return start


def block_causal_mask(doc_lens_rows, seq_len, row_offset, q_len):
    """The dense boolean mask [B, q_len, S]: M[b, t, j] is True iff query
    position i = row_offset + t and key position j lie in the same document
    and j <= i."""
    B = len(doc_lens_rows)
    M = np.zeros((B, q_len, seq_len), bool)
    j = np.arange(seq_len)
    for b, lens in enumerate(doc_lens_rows):
        doc_id = np.full(seq_len, -1, np.int64)
        pos = 0
        for d, L in enumerate(lens):
            doc_id[pos:pos + L] = d
            pos += L
        for t in range(q_len):
            i = row_offset + t
            if doc_id[i] >= 0:
                M[b, t] = (doc_id == doc_id[i]) & (j <= i)
    return M


def _blocks(rows, block_rows):
    """Split a sorted list of local rows into runs of consecutive rows of at
    most block_rows each."""
    out, cur = [], []
    for t in rows:
        if cur and (t != cur[-1] + 1 or len(cur) >= block_rows):
            out.append(cur)
            cur = []
        cur.append(t)
    if cur:
        out.append(cur)
    return out


def _plan(doc_lens_rows, seq_len, row_offset, q_len, block_rows, rows):
    """Yield (b, local rows [t0, t1), key window [w0, w1), mask block)."""
    rows = range(q_len) if rows is None else sorted(set(int(t) for t in rows))
    dense = block_rows is None
    blocks = _blocks(list(rows), q_len if dense else block_rows)
    for b, lens in enumerate(doc_lens_rows):
        start = _row_doc_start(lens, seq_len)
        doc_id = np.full(seq_len, -1, np.int64)
        pos = 0
        for d, L in enumerate(lens):
            doc_id[pos:pos + L] = d
            pos += L
        for blk in blocks:
            t0, t1 = blk[0], blk[-1] + 1
            i = np.arange(t0, t1) + row_offset
            real = start[i] >= 0
            if dense:
                w0, w1 = 0, seq_len
            elif real.any():
                w0 = int(start[i[real]].min())
                w1 = int(i[real].max()) + 1
            else:
                w0 = w1 = 0
            j = np.arange(w0, w1)
            M = (doc_id[i][:, None] == doc_id[j][None, :]) & (j[None, :] <= i[:, None]) \
                & real[:, None]
            yield b, t0, t1, w0, w1, M


def _softmax_block(s, M):
    """Masked softmax of a block of scaled logits: returns (P, lse) with
    P = 0 and lse = -inf on rows with no allowed key."""
    s = np.where(M, s, -np.inf)
    valid = M.any(axis=1)
    m = np.where(valid, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(M, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(valid, m + np.log(np.where(valid, l, 1.0)), -np.inf)
    P = np.where(M, np.exp(s - np.where(valid, lse, 0.0)[:, None]), 0.0)
    return P, lse


def _check(q, k, v):
    B, L, Hq, d = q.shape
    Bk, S, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    return B, L, Hq, d, S, Hkv, Hq // Hkv


def forward(q, k, v, doc_lens_rows, row_offset, scale, block_rows=None, rows=None, dropout=None):
    """Returns (o [B,L,Hq,d], lse [B,Hq,L]) in float64.  With ``rows``, only
    those local rows are computed (others stay O = 0, LSE = -inf).  With
    ``dropout`` (a Dropout), O uses the kept weights P * Z * c; LSE is that
    of the undropped softmax."""
    B, L, Hq, d, S, Hkv, G = _check(q, k, v)
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    o = np.zeros((B, L, Hq, d))
    lse = np.full((B, Hq, L), -np.inf)
    for b, t0, t1, w0, w1, M in _plan(doc_lens_rows, S, row_offset, L, block_rows, rows):
        if w1 <= w0:
            continue
        for h in range(Hq):
            g = h // G
            s = scale * (q[b, t0:t1, h, :] @ k[b, w0:w1, g, :].T)
            P, ls = _softmax_block(s, M)
            if dropout is not None:
                Z, c = dropout.keep(b, h, np.arange(t0, t1) + row_offset, np.arange(w0, w1))
                P = P * Z * c
            o[b, t0:t1, h, :] = P @ v[b, w0:w1, g, :]
            lse[b, h, t0:t1] = ls
    return o, lse


def backward(q, k, v, do, doc_lens_rows, row_offset, scale, block_rows=None, rows=None, dropout=None):
    """Returns (dq, dk, dv) in float64 for the loss sum(dO * O).  With
    ``rows``, only those local query rows contribute: their dQ rows are exact,
    and dK/dV hold the contributions of those rows only.  With ``dropout``,
    O = (P * Z * c) V, so dV = (P * Z * c)^T dO and the gradient reaching P
    is dP = (dO V^T) * Z * c; the softmax Jacobian step is unchanged."""
    B, L, Hq, d, S, Hkv, G = _check(q, k, v)
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); do = np.asarray(do, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b, t0, t1, w0, w1, M in _plan(doc_lens_rows, S, row_offset, L, block_rows, rows):
        if w1 <= w0:
            continue
        for h in range(Hq):
            g = h // G
            qb, kb, vb, dob = q[b, t0:t1, h], k[b, w0:w1, g], v[b, w0:w1, g], do[b, t0:t1, h]
            P, _ = _softmax_block(scale * (qb @ kb.T), M)
            dP = dob @ vb.T
            Pv = P  # the weights that multiply V
            if dropout is not None:
                Z, c = dropout.keep(b, h, np.arange(t0, t1) + row_offset, np.arange(w0, w1))
                dP = dP * Z * c
                Pv = P * Z * c
            r = (P * dP).sum(axis=1)
            dS = P * (dP - r[:, None])
            dq[b, t0:t1, h] = scale * (dS @ kb)
            dk[b, w0:w1, g] += scale * (dS.T @ qb)
            dv[b, w0:w1, g] += Pv.T @ dob
    return dq, dk, dv


def useful_pairs(doc_lens_rows, seq_len, row_offset, q_len):
    """Number of allowed (query, key) pairs over all batch rows (per query
    head): the popcount of the mask, computed per row as i - doc_start(i) + 1
    summed over the chunk's real rows."""
    total = 0
    for lens in doc_lens_rows:
        start = _row_doc_start(lens, seq_len)
        i = np.arange(row_offset, row_offset + q_len)
        real = start[i] >= 0
        total += int((i[real] - start[i[real]] + 1).sum())
    return total
