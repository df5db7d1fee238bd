"""Seeded synthetic inputs for packed block-causal attention.

This module is shared by the fp64 CPU oracle's tests, the GPU parity tests and
the benchmark.  It holds no attention arithmetic: it only draws document
lengths and N(0,1) tensors, and rounds fp32 draws to bfloat16 values.

Workloads follow the shapes and length mixes of the context-parallel
packed-sequence training described on the Automodel page "feat(distributed):
block-diagonal varlen CP for packed sequences" (Summary and Motivation: many
variable-length documents packed into one row; Design overview: contiguous
per-rank query chunks against the K/V of the whole packed row).  The
per-config numbers (sequence lengths, head counts, length distributions) are
the five benchmark workloads listed below; every random choice is seeded.

Recipe (applies to every workload):
  * document lengths: ``numpy.random.default_rng([wid, 0, attempt])``; docs
    are drawn one at a time until the row is full; a lognormal draw is
    ``int(numpy.rint(rng.lognormal(log(median), sigma)))`` clipped to
    ``[lo, hi]``; the last document is truncated so the row sums to ``S``
    exactly (no padding in the five workloads).  Rows of a batch are drawn in
    order from one generator.
  * tensors: ``numpy.random.default_rng([wid, t]).standard_normal(shape,
    dtype=float32)`` with t = 1 (Q), 2 (K), 3 (V), 4 (dO), layout
    ``[B, S, H, d]``.  Q and dO are drawn for the whole row and sliced to the
    local chunk, so a chunk's inputs are rows of the full problem.
  * bf16 workloads round the fp32 draws to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "doc_lengths", "draw_tensors",
    "round_bf16", "custom_workload",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int                 # seed key (1..5 for the named workloads)
    name: str
    dtype: str               # "f32" or "bf16"
    batch: int
    seq_len: int
    row_offset: int
    q_len: int
    h_q: int
    h_kv: int
    head_dim: int
    scale: float
    doc_lens: tuple          # tuple of tuples, one per batch row

    @property
    def n_docs(self) -> int:
        return sum(len(r) for r in self.doc_lens)


def _lognormal_row(rng, seq_len, median, sigma, lo, hi, prefix=()):
    lens = list(prefix)
    total = sum(lens)
    while total < seq_len:
        L = int(np.rint(rng.lognormal(mean=math.log(median), sigma=sigma)))
        L = min(max(L, lo), hi)
        if total + L > seq_len:
            L = seq_len - total
        lens.append(L)
        total += L
    return tuple(lens)


def _uniform_row(rng, seq_len, lo, hi):
    lens = []
    total = 0
    while total < seq_len:
        L = int(rng.integers(lo, hi + 1))
        if total + L > seq_len:
            L = seq_len - total
        lens.append(L)
        total += L
    return tuple(lens)


def _straddles(lens, chunk_bounds, inner):
    """Input-structure check for workload 3: ``inner`` lies strictly inside a
    document, and at least two distinct documents cross one of the chunk
    bounds (a bound b is crossed by [s, e) when s < b < e)."""
    starts = np.cumsum((0,) + tuple(lens[:-1]))
    ends = starts + np.asarray(lens)
    inside = any(s < inner < e for s, e in zip(starts, ends))
    crossing = {i for i, (s, e) in enumerate(zip(starts, ends))
                for b in chunk_bounds if s < b < e}
    return inside and len(crossing) >= 2


def doc_lengths(wid: int):
    """Document lengths per batch row for named workload ``wid`` (1..5)."""
    if wid == 1:
        return ((200, 37, 150, 125),)
    if wid == 2:
        rng = np.random.default_rng([2, 0, 0])
        return tuple(_lognormal_row(rng, 4096, 512, 1.0, 16, 4096) for _ in range(2))
    if wid == 3:
        attempt = 0
        while True:
            rng = np.random.default_rng([3, 0, attempt])
            row = _lognormal_row(rng, 16384, 2048, 1.0, 16, 16384)
            if _straddles(row, (4096, 8192, 12288), 8192):
                return (row,)
            attempt += 1
    if wid == 4:
        rng = np.random.default_rng([4, 0, 0])
        return (_lognormal_row(rng, 32768, 256, 1.0, 16, 4096, prefix=(24576,)),)
    if wid == 5:
        rng = np.random.default_rng([5, 0, 0])
        return (_uniform_row(rng, 49152, 16, 128),)
    raise ValueError(f"unknown workload {wid}")


_SHAPES = {
    # wid: (name, dtype, B, S, row_offset, q_len, h_q, h_kv, d)
    1: ("fp32 S=512, 4 docs, H=4, d=64", "f32", 1, 512, 0, 512, 4, 4, 64),
    2: ("bf16 packed S=4096 x2, lognormal docs (median 512), 32/8/128", "bf16", 2, 4096, 0, 4096, 32, 8, 128),
    3: ("bf16 one CP rank: S=16384, rows [8192,12288), 32/8/128", "bf16", 1, 16384, 8192, 4096, 32, 8, 128),
    4: ("bf16 long mixed S=32768: 24576-token doc + short docs, 32/8/64", "bf16", 1, 32768, 0, 32768, 32, 8, 64),
    5: ("bf16 fragmented S=49152: docs uniform in [16,128], 32/8/128", "bf16", 1, 49152, 0, 49152, 32, 8, 128),
}


def workload(wid: int) -> Workload:
    name, dt, B, S, r0, ql, hq, hkv, d = _SHAPES[wid]
    return Workload(wid, name, dt, B, S, r0, ql, hq, hkv, d, 1.0 / math.sqrt(d), doc_lengths(wid))


WORKLOADS = (1, 2, 3, 4, 5)


def custom_workload(wid, dtype, doc_lens, seq_len, row_offset, q_len, h_q, h_kv, d, scale=None, name="custom"):
    doc_lens = tuple(tuple(int(x) for x in r) for r in doc_lens)
    return Workload(wid, name, dtype, len(doc_lens), seq_len, row_offset, q_len, h_q, h_kv, d,
                    (1.0 / math.sqrt(d)) if scale is None else float(scale), doc_lens)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32.  NaN/Inf are not expected in these inputs."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def draw_tensors(w: Workload, which=("q", "k", "v", "do")):
    """fp32 numpy arrays (bf16-rounded values for bf16 workloads):
    q, do: [B, q_len, h_q, d]; k, v: [B, S, h_kv, d]."""
    tids = {"q": 1, "k": 2, "v": 3, "do": 4}
    out = {}
    for name in which:
        t = tids[name]
        heads = w.h_q if name in ("q", "do") else w.h_kv
        a = np.random.default_rng([w.wid, t]).standard_normal(
            (w.batch, w.seq_len, heads, w.head_dim), dtype=np.float32)
        if name in ("q", "do"):
            a = np.ascontiguousarray(a[:, w.row_offset:w.row_offset + w.q_len])
        if w.dtype == "bf16":
            a = round_bf16(a)
        out[name] = a
    return out
