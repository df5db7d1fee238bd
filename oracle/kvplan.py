"""Reference needed-only K/V exchange plan (oracle; test infrastructure only).

Source: Automodel page "feat(distributed): block-diagonal varlen CP for packed
sequences".  Summary: needed-only exchanges -- a left-neighbour halo
(point-to-point) or an all-to-all-v when a document spans more than two ranks
-- cut a rank's K/V from the whole row to its own chunk plus the straddling
prefix.  Design overview, batch.py: rows are padded to a multiple of cp and
every rank holds a contiguous slice; exchange.py: left-halo p2p and the
needed-only all-to-all-v.  Proof: the plan geometry is checked on the CPU.

Everything here follows from the dense block-causal mask (oracle.attention):
the keys a rank needs are exactly the keys some row of its chunk is allowed
to attend.  Nothing assumes the keys form one interval: that is checked.

Reading where the pages are silent: chunks are [r * S/cp, (r + 1) * S/cp);
the K/V window a rank's kernel takes starts at the smallest needed key (or
its own first row, if smaller), rounded down to a multiple of ``align``, and
ends at its chunk's end; a rank's mode is 0 with no halo, 1 when every halo
key belongs to rank - 1, 2 when some belongs to a rank further left; the
step's mode is the largest over the ranks (every rank runs the same
collective).
"""
from __future__ import annotations

import numpy as np

from .attention import block_causal_mask


def needed_keys(doc_lens_rows, seq_len, cp, rank):
    """Boolean [B, S]: key j of row b is attended by some row of the chunk."""
    C = seq_len // cp
    M = block_causal_mask(doc_lens_rows, seq_len, rank * C, C)
    return M.any(axis=1)


def _runs_by_owner(keys, C):
    """Split sorted key positions into (owner rank, begin, end) runs; each
    owner's keys must be one interval."""
    out = []
    for q in sorted(set(int(j) // C for j in keys)):
        ks = keys[keys // C == q]
        assert ks[-1] - ks[0] + 1 == len(ks), "needed keys of one owner are not contiguous"
        out.append((q, int(ks[0]), int(ks[-1]) + 1))
    return out


def rank_mode(doc_lens_rows, seq_len, cp, rank):
    C = seq_len // cp
    need = needed_keys(doc_lens_rows, seq_len, cp, rank)
    halo = np.nonzero(need[:, :rank * C])[1]
    if halo.size == 0:
        return 0
    return 2 if halo.min() < (rank - 1) * C else 1


def kv_plan_ref(doc_lens_rows, seq_len, cp, rank, align=64):
    """dict(kv_begin, kv_end, recv, send, rank_mode, step_mode) with recv /
    send lists of (row, peer, begin, end)."""
    assert seq_len % cp == 0
    C = seq_len // cp
    r0, r1 = rank * C, (rank + 1) * C
    need = needed_keys(doc_lens_rows, seq_len, cp, rank)
    recv, lo = [], r0
    for b in range(need.shape[0]):
        keys = np.nonzero(need[b])[0]
        if keys.size:
            lo = min(lo, int(keys.min()))
        for q, a, e in _runs_by_owner(keys[keys < r0], C):
            recv.append((b, q, a, e))
    send = []
    later = {q: needed_keys(doc_lens_rows, seq_len, cp, q) for q in range(rank + 1, cp)}
    for b in range(need.shape[0]):
        for q in range(rank + 1, cp):
            keys = np.nonzero(later[q][b, r0:r1])[0] + r0
            if keys.size:
                assert keys[-1] - keys[0] + 1 == len(keys)
                send.append((b, q, int(keys[0]), int(keys[-1]) + 1))
    return {"kv_begin": (lo // align) * align, "kv_end": r1, "recv": recv, "send": send,
            "rank_mode": rank_mode(doc_lens_rows, seq_len, cp, rank),
            "step_mode": max(rank_mode(doc_lens_rows, seq_len, cp, r) for r in range(cp))}
