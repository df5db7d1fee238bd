"""Attention-dropout keep masks from a counter-based generator (oracle; test
infrastructure only).

Source of the method: the Automodel page "feat(distributed): block-diagonal
varlen CP for packed sequences", Proof: the varlen attention path forwards a
dropout probability and the native kernel applies attention dropout.  The
pages give no random-number contract, so the reading taken here is:

* dropout acts on the normalised attention weights: O_i = sum_j P_ij Z_ij c
  v_j with Z_ij in {0, 1} and c = 1 / (1 - p_eff); LSE is that of the
  undropped softmax;
* Z comes from Philox4x32-10, the counter-based generator of Salmon, Moraes,
  Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): one
  call maps a 128-bit counter and a 64-bit key to four 32-bit words through
  ten rounds, each multiplying two of the words by fixed 32-bit constants
  and mixing the high and low product halves with the other words and the
  round key; the key is bumped by two Weyl constants between rounds;
* the counter of the pair (query position i, key position j) -- positions in
  the packed row, so a mask does not depend on how the rows are chunked --
  of batch row b and query head h is (j // 4, i // 4, b * H_q + h, offset)
  and the key is (seed mod 2^32, seed // 2^32); word i % 4 of the output,
  byte j % 4 of that word (least significant first), is compared with the
  8-bit threshold thr = min(255, round(256 p)): the pair is kept iff the
  byte is >= thr, so p_eff = thr / 256 and c = 256 / (256 - thr).
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57        # round multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85        # Weyl key increments
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10 over arrays of counters (uint32 values in
    int64/uint64 arrays); returns the four output words as uint64 arrays."""
    c0, c1, c2, c3 = (np.asarray(x, np.uint64) & MASK32 for x in (c0, c1, c2, c3))
    k0 = np.uint64(k0 & MASK32)
    k1 = np.uint64(k1 & MASK32)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + W0) & MASK32)
            k1 = np.uint64((int(k1) + W1) & MASK32)
        p0 = c0 * np.uint64(M0)          # < 2^64: exact in uint64
        p1 = c2 * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def threshold(p):
    """8-bit drop threshold for probability p in [0, 1)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(p * 256 + 0.5)))


def keep_scale(p):
    """(threshold, c): kept weights are multiplied by c = 256 / (256 - thr)."""
    thr = threshold(p)
    return thr, 256.0 / (256 - thr)


def keep_mask(seed, offset, b, h, h_q, rows, keys, p):
    """Boolean [len(rows), len(keys)]: Z for query positions ``rows`` and key
    positions ``keys`` (positions in the packed row) of batch row b, query
    head h."""
    thr = threshold(p)
    i = np.asarray(rows, np.int64)[:, None]
    j = np.asarray(keys, np.int64)[None, :]
    i, j = np.broadcast_arrays(i, j)
    words = philox4x32_10(j // 4, i // 4, np.full(i.shape, b * h_q + h), np.full(i.shape, offset),
                          seed & MASK32, (seed >> 32) & MASK32)
    w = np.select([i % 4 == 0, i % 4 == 1, i % 4 == 2], [words[0], words[1], words[2]], words[3])
    byte = (w >> (np.uint64(8) * (j % 4).astype(np.uint64))) & np.uint64(0xFF)
    return byte >= np.uint64(thr)
