"""Pure-Python scalar loops for tiny inputs (oracle; test infrastructure only).

Same function as ``oracle.attention`` (Automodel page "feat(distributed):
block-diagonal varlen CP for packed sequences", Summary and Motivation: each
query attends only keys of its own document at or before itself), written as
independently as possible: the mask is evaluated per pair from document ids,
softmax uses ``math.exp`` over explicit lists, and the backward takes the
other well-known route through delta_i = sum_d dO_i O_i (the row sum of
P * dP equals dO_i . O_i because O_i = sum_j P_ij v_j), so agreement with
``oracle.attention`` checks both derivations.

Inputs are nested Python lists or numpy arrays with the layouts of
``oracle.attention``; outputs are nested lists of floats.
"""
from __future__ import annotations

import math


def _doc_ids(lens, seq_len):
    ids = [-1] * seq_len
    pos = 0
    for d, L in enumerate(lens):
        for i in range(pos, pos + L):
            ids[i] = d
        pos += L
    return ids


def _dot(a, b):
    return sum(float(x) * float(y) for x, y in zip(a, b))


def forward(q, k, v, doc_lens_rows, row_offset, scale):
    B, L, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    S, Hkv = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    o = [[[[0.0] * d for _ in range(Hq)] for _ in range(L)] for _ in range(B)]
    lse = [[[-math.inf] * L for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        ids = _doc_ids(doc_lens_rows[b], S)
        for h in range(Hq):
            g = h // G
            for t in range(L):
                i = row_offset + t
                keys = [j for j in range(S) if ids[i] >= 0 and ids[j] == ids[i] and j <= i]
                if not keys:
                    continue
                s = [scale * _dot(q[b][t][h], k[b][j][g]) for j in keys]
                m = max(s)
                z = sum(math.exp(x - m) for x in s)
                lse[b][h][t] = m + math.log(z)
                for c in range(d):
                    o[b][t][h][c] = sum(math.exp(x - m) / z * float(v[b][j][g][c])
                                        for x, j in zip(s, keys))
    return o, lse


def backward(q, k, v, do, doc_lens_rows, row_offset, scale):
    B, L, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    S, Hkv = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    o, _ = forward(q, k, v, doc_lens_rows, row_offset, scale)
    dq = [[[[0.0] * d for _ in range(Hq)] for _ in range(L)] for _ in range(B)]
    dk = [[[[0.0] * d for _ in range(Hkv)] for _ in range(S)] for _ in range(B)]
    dv = [[[[0.0] * d for _ in range(Hkv)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        ids = _doc_ids(doc_lens_rows[b], S)
        for h in range(Hq):
            g = h // G
            for t in range(L):
                i = row_offset + t
                keys = [j for j in range(S) if ids[i] >= 0 and ids[j] == ids[i] and j <= i]
                if not keys:
                    continue
                s = [scale * _dot(q[b][t][h], k[b][j][g]) for j in keys]
                m = max(s)
                z = sum(math.exp(x - m) for x in s)
                p = [math.exp(x - m) / z for x in s]
                delta = _dot(do[b][t][h], o[b][t][h])
                for pj, j in zip(p, keys):
                    dpj = _dot(do[b][t][h], v[b][j][g])
                    ds = pj * (dpj - delta)
                    for c in range(d):
                        dq[b][t][h][c] += scale * ds * float(k[b][j][g][c])
                        dk[b][j][g][c] += scale * ds * float(q[b][t][h][c])
                        dv[b][j][g][c] += pj * float(do[b][t][h][c])
    return dq, dk, dv
