"""Reference varlen metadata for block-causal packed attention (fp64 oracle;
test infrastructure only).

Source: Automodel page "feat(distributed): block-diagonal varlen CP for packed
sequences" -- Summary (per-step precomputed cu_seqlens drive the varlen
kernel), Design overview (kernels.py: varlen segmentation and host-side
validation; batch.py: contiguous per-rank slice) and key property 2 (a
document straddling the chunk's left edge gives an asymmetric first segment,
more keys than queries, bottom-right aligned).

Segment table for batch rows b = 0..B-1, chunk rows [r0, r1), r1 = r0 + q_len:
  for every document [s, e) of row b with s < r1 and e > r0, one segment with
    local query rows  [max(s, r0) - r0, min(e, r1) - r0)  (+ b * q_len)
    keys              [s, min(e, r1))                      (+ b * S)
  and, if the row's padding tail (positions >= sum of its doc lengths)
  reaches into the chunk, one padding segment covering those rows with no
  keys; its key begin is the first padding row's position (+ b * S).
Documents of length zero hold no token and produce no segment.

Outputs (all Python ints):
  cu_q   [n+1]  prefix sums of segment query lengths (0 .. B*q_len)
  cu_k   [n+1]  prefix sums of segment key lengths
  k_begin[n]    flattened key index (b*S + position) of each segment's first key
  max_q, max_k  largest segment query / key length (0 if no segment)
"""
from __future__ import annotations


class MetadataError(ValueError):
    pass


def segment_ref(doc_lens_rows, seq_len, row_offset, q_len):
    if seq_len < 0 or row_offset < 0 or q_len < 0 or row_offset + q_len > seq_len:
        raise MetadataError("chunk out of range")
    r0, r1 = row_offset, row_offset + q_len
    cu_q, cu_k, k_begin = [0], [0], []
    for b, lens in enumerate(doc_lens_rows):
        pos = 0
        for L in lens:
            if L < 0:
                raise MetadataError("negative document length")
            s, e = pos, pos + L
            pos = e
            if pos > seq_len:
                raise MetadataError("document lengths exceed the row length")
            qs, qe = max(s, r0), min(e, r1)
            if qe <= qs:  # empty document, or no row of it in the chunk
                continue
            cu_q.append(cu_q[-1] + (qe - qs))
            cu_k.append(cu_k[-1] + (qe - s))
            k_begin.append(b * seq_len + s)
        qs = max(pos, r0)
        if qs < r1:  # padding tail reaches into the chunk
            cu_q.append(cu_q[-1] + (r1 - qs))
            cu_k.append(cu_k[-1])
            k_begin.append(b * seq_len + qs)
    qlens = [cu_q[i + 1] - cu_q[i] for i in range(len(k_begin))]
    klens = [cu_k[i + 1] - cu_k[i] for i in range(len(k_begin))]
    return {
        "cu_q": cu_q, "cu_k": cu_k, "k_begin": k_begin, "n_seg": len(k_begin),
        "max_q": max(qlens, default=0), "max_k": max(klens, default=0),
    }


def token_doc_ids(lens, seq_len):
    """Document index of every position of a row; -1 on padding."""
    ids = [-1] * seq_len
    pos = 0
    for d, L in enumerate(lens):
        for i in range(pos, pos + L):
            ids[i] = d
        pos += L
    return ids


def mask_bounds(doc_lens_rows, seq_len, row_offset, q_len):
    """Per-row and per-key bounds of the block-causal mask, read off the mask
    definition itself (same document and key <= query) by scanning.

    Returns (row_lo, row_hi, key_qlo, key_qhi), lists of lists:
      row b, local query row t: keys j with row_lo <= j < row_hi are allowed
        (positions within the row); a padding row has row_lo = row_hi = 0.
      row b, key position j: local query rows t with key_qlo <= t < key_qhi
        attend it; a key no local row attends has key_qlo = key_qhi = 0.
    The allowed sets are checked to be contiguous intervals.
    """
    r0 = row_offset
    row_lo, row_hi, key_qlo, key_qhi = [], [], [], []
    for lens in doc_lens_rows:
        ids = token_doc_ids(lens, seq_len)
        lo_b, hi_b = [], []
        attend = [[] for _ in range(seq_len)]
        for t in range(q_len):
            i = r0 + t
            allowed = [j for j in range(seq_len) if ids[i] >= 0 and ids[j] == ids[i] and j <= i]
            if not allowed:
                lo_b.append(0); hi_b.append(0)
                continue
            assert allowed == list(range(allowed[0], allowed[-1] + 1))
            lo_b.append(allowed[0]); hi_b.append(allowed[-1] + 1)
            for j in allowed:
                attend[j].append(t)
        qlo_b, qhi_b = [], []
        for j in range(seq_len):
            a = attend[j]
            if not a:
                qlo_b.append(0); qhi_b.append(0)
                continue
            assert a == list(range(a[0], a[-1] + 1))
            qlo_b.append(a[0]); qhi_b.append(a[-1] + 1)
        row_lo.append(lo_b); row_hi.append(hi_b)
        key_qlo.append(qlo_b); key_qhi.append(qhi_b)
    return row_lo, row_hi, key_qlo, key_qhi


def mask_bounds_np(doc_lens_rows, seq_len, row_offset, q_len):
    """Same result as ``mask_bounds`` for large rows, written with numpy from
    each position's document start and end: since documents are contiguous,
    'same document and j <= i' is 'doc_start(i) <= j <= i', and the local rows
    attending key j are those of its document from max(j, r0) up to
    min(doc_end(j), r1).  Pinned against the scanning version on small rows.
    Returns four int64 arrays of shape [B, q_len] / [B, seq_len]."""
    import numpy as np
    B = len(doc_lens_rows)
    r0, r1 = row_offset, row_offset + q_len
    row_lo = np.zeros((B, q_len), np.int64)
    row_hi = np.zeros((B, q_len), np.int64)
    key_qlo = np.zeros((B, seq_len), np.int64)
    key_qhi = np.zeros((B, seq_len), np.int64)
    for b, lens in enumerate(doc_lens_rows):
        start = np.full(seq_len, -1, np.int64)
        end = np.full(seq_len, -1, np.int64)
        pos = 0
        for L in lens:
            start[pos:pos + L] = pos
            end[pos:pos + L] = pos + L
            pos += L
        i = np.arange(r0, r1)
        real = start[i] >= 0
        row_lo[b] = np.where(real, start[i], 0)
        row_hi[b] = np.where(real, i + 1, 0)
        j = np.arange(seq_len)
        first = np.maximum(j, r0)
        last = np.minimum(end, r1)  # exclusive
        att = (start >= 0) & (first < last)
        key_qlo[b] = np.where(att, first - r0, 0)
        key_qhi[b] = np.where(att, last - r0, 0)
    return row_lo, row_hi, key_qlo, key_qhi
