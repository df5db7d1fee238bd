"""Block-diagonal (per-document causal) packed attention for AMD MI355X.

Python binding of ``libblockdiag.so`` (C ABI declared in
``include/blockdiag.h``).  This module only marshals arguments: every step
of the computation runs in the library's host code (segmentation,
validation) or its gfx950 kernels.  PyTorch supplies device memory and the
current stream.  There is no fallback: if the library is missing the calls
raise.

What it computes follows the Automodel page "feat(distributed):
block-diagonal varlen CP for packed sequences" (Summary, Motivation, Design
overview, key properties 1-4): a packed row holds documents back to back; a
query attends only keys of its own document at or before itself; one GPU
holds the contiguous query chunk [row_offset, row_offset + q_len) and the K/V
of the whole row; varlen metadata is computed and validated once per step.

Typical use, once per step and then per layer::

    seg = segment(doc_lens_per_row, seq_len, row_offset, q_len, device="cuda")
    out = attention(q, k, v, seg)              # autograd-aware
    o, lse = attn_fwd(q, k, v, seg)            # or the raw calls
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, seg)

Layouts: q, o, do, dq ``[B, q_len, H_q, d]``; k, v, dk, dv ``[B, S, H_kv, d]``;
lse ``[B, H_q, q_len]`` float32.  dtype float32 or bfloat16.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import numpy as np

__all__ = [
    "BlockdiagError", "MetaDesc", "Dropout", "SegTable", "segment", "validate", "doc_lens_from_ids",
    "attn_fwd", "attn_bwd", "attention", "library_path", "load_library", "KvPlan", "kv_plan",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libblockdiag.so")
_LIB = None

STATUS = {0: "BD_OK", 1: "BD_ERR_INVALID_ARG", 2: "BD_ERR_BAD_METADATA", 3: "BD_ERR_CAPACITY",
          4: "BD_ERR_WORKSPACE", 5: "BD_ERR_UNSUPPORTED", 6: "BD_ERR_HIP"}
EXPORTS = ("blockdiag_segment", "blockdiag_validate", "blockdiag_kv_plan", "blockdiag_meta_ints", "blockdiag_meta_build",
           "blockdiag_meta_build_host", "blockdiag_meta_inline_max_seg",
           "blockdiag_workspace_bytes", "blockdiag_attn_fwd", "blockdiag_attn_bwd",
           "blockdiag_attn_bwd_noalloc", "blockdiag_noalloc_scratch_bytes",
           "blockdiag_mark_main_kernel", "blockdiag_clock_probe", "blockdiag_last_error", "blockdiag_version")


class MetaDesc(ctypes.Structure):
    """``bd_meta``: host descriptor of a device metadata buffer, filled by
    ``blockdiag_meta_build`` / ``blockdiag_meta_build_host`` with the sizes
    the buffer was built for (the attention calls check them)."""
    _fields_ = [("magic", ctypes.c_uint32), ("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("row_offset", ctypes.c_int32), ("q_len", ctypes.c_int32), ("n_seg", ctypes.c_int32),
                ("kv_lo", ctypes.c_int32), ("kv_hi", ctypes.c_int32), ("max_seg_k", ctypes.c_int32),
                ("n_ints", ctypes.c_uint64), ("data", ctypes.c_void_p)]


class Dropout(ctypes.Structure):
    """``bd_dropout``: attention dropout of the attention calls (drop
    probability p, counter offset, 64-bit seed; the mask is a stated
    function of them, see include/blockdiag.h)."""
    _fields_ = [("p", ctypes.c_float), ("offset", ctypes.c_uint32), ("seed", ctypes.c_uint64)]


def _dropout_arg(dropout):
    """None or (p, seed, offset) -> a bd_dropout pointer (or None)."""
    if dropout is None:
        return None
    p, seed, offset = dropout
    return ctypes.byref(Dropout(float(p), int(offset) & 0xFFFFFFFF, int(seed) & 0xFFFFFFFFFFFFFFFF))


class KvRange(ctypes.Structure):
    """``bd_kv_range``: keys [begin, end) of batch row ``row`` exchanged with
    rank ``peer``."""
    _fields_ = [("row", ctypes.c_int32), ("peer", ctypes.c_int32), ("begin", ctypes.c_int32),
                ("end", ctypes.c_int32)]


META_MAGIC = 0x54454D42


class BlockdiagError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.message = message


def library_path():
    return _LIB_PATH


def load_library():
    """Load libblockdiag.so once and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise FileNotFoundError(
            f"{_LIB_PATH} is missing: build it with packed_sequence_attention_amd.build.build_library()")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, p, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.blockdiag_segment.argtypes = [pi32, pi32, i32, i32, i32, i32, i32, pi32, pi32, pi32, pi32, pi32, pi32]
    lib.blockdiag_segment.restype = ctypes.c_int
    lib.blockdiag_validate.argtypes = [pi32, pi32, pi32, i32, i32, i32, i32, i32]
    lib.blockdiag_validate.restype = ctypes.c_int
    prange = ctypes.POINTER(KvRange)
    lib.blockdiag_kv_plan.argtypes = [pi32, pi32, i32, i32, i32, i32, i32, pi32, pi32, i32, prange, pi32, prange,
                                      pi32, pi32, pi32]
    lib.blockdiag_kv_plan.restype = ctypes.c_int
    lib.blockdiag_meta_ints.argtypes = [i32, i32, i32]
    lib.blockdiag_meta_ints.restype = sz
    pdesc = ctypes.POINTER(MetaDesc)
    lib.blockdiag_meta_build.argtypes = [p, pi32, i32, i32, i32, i32, i32, p, sz, pdesc, p]
    lib.blockdiag_meta_build.restype = ctypes.c_int
    lib.blockdiag_meta_build_host.argtypes = [pi32, i32, i32, i32, i32, i32, p, sz, pdesc, p]
    lib.blockdiag_meta_build_host.restype = ctypes.c_int
    lib.blockdiag_meta_inline_max_seg.argtypes = []
    lib.blockdiag_meta_inline_max_seg.restype = i32
    lib.blockdiag_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, i32, i32, i32, i32]
    lib.blockdiag_workspace_bytes.restype = sz
    pdrop = ctypes.POINTER(Dropout)
    lib.blockdiag_attn_fwd.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float, pdrop, p, p, p, pdesc, p, p, p, sz, p]
    lib.blockdiag_attn_fwd.restype = ctypes.c_int
    lib.blockdiag_attn_bwd.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float, pdrop, p, p, p, p, p, p, pdesc, p, p, p, p, sz, p]
    lib.blockdiag_attn_bwd.restype = ctypes.c_int
    lib.blockdiag_attn_bwd_noalloc.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                               ctypes.c_float, pdrop, p, p, p, p, p, p, pdesc, p, p, p, p]
    lib.blockdiag_attn_bwd_noalloc.restype = ctypes.c_int
    lib.blockdiag_noalloc_scratch_bytes.argtypes = []
    lib.blockdiag_noalloc_scratch_bytes.restype = sz
    lib.blockdiag_mark_main_kernel.argtypes = [p, p]
    lib.blockdiag_mark_main_kernel.restype = ctypes.c_int
    lib.blockdiag_clock_probe.argtypes = [i32, ctypes.c_uint32, p, p]
    lib.blockdiag_clock_probe.restype = ctypes.c_int
    lib.blockdiag_last_error.argtypes = []
    lib.blockdiag_last_error.restype = ctypes.c_char_p
    lib.blockdiag_version.argtypes = []
    lib.blockdiag_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(code):
    if code != 0:
        msg = load_library().blockdiag_last_error().decode()
        raise BlockdiagError(code, msg)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


@dataclasses.dataclass
class SegTable:
    """Varlen metadata of one chunk, computed once per step.

    Host arrays (numpy int32): ``cu_q``, ``cu_k`` ([n_seg + 1]) and ``k_begin``
    ([n_seg]) as defined in include/blockdiag.h.  With a device, ``table``
    holds their concatenation on the device, ``meta`` the per-row and
    per-key mask bounds built from it by ``blockdiag_meta_build`` and
    ``desc`` the buffer's descriptor (``bd_meta``) that the attention calls
    take."""
    batch: int
    seq_len: int
    row_offset: int
    q_len: int
    cu_q: np.ndarray
    cu_k: np.ndarray
    k_begin: np.ndarray
    n_seg: int
    max_q: int
    max_k: int
    table: object = None
    meta: object = None
    desc: object = None
    _pinned: object = None

    def to(self, device, inline=None):
        """Build the device metadata on ``device``.  A table of at most
        ``blockdiag_meta_inline_max_seg()`` segments goes to the kernel in its
        launch arguments (``blockdiag_meta_build_host``, no upload); a larger
        one (or ``inline=False``) is copied to the device first
        (``blockdiag_meta_build``)."""
        import torch
        lib = load_library()
        flat = np.ascontiguousarray(np.concatenate([self.cu_q, self.cu_k, self.k_begin]), dtype=np.int32)
        n_meta = lib.blockdiag_meta_ints(self.batch, self.seq_len, self.q_len)
        meta = torch.empty(max(int(n_meta), 1), dtype=torch.int32, device=device)
        desc = MetaDesc()
        stream = torch.cuda.current_stream(meta.device).cuda_stream
        if inline is None:
            inline = self.n_seg <= lib.blockdiag_meta_inline_max_seg()
        with torch.cuda.device(meta.device):  # the library launches on the current device
            if inline:
                _check(lib.blockdiag_meta_build_host(_ptr(flat), self.n_seg, self.batch, self.seq_len,
                                                     self.row_offset, self.q_len, meta.data_ptr(), meta.numel(),
                                                     ctypes.byref(desc), stream))
                return dataclasses.replace(self, table=None, meta=meta, desc=desc, _pinned=None)
            pinned = torch.from_numpy(flat).pin_memory()
            table = pinned.to(meta.device, non_blocking=True)  # no host sync; pinned copy kept alive below
            _check(lib.blockdiag_meta_build(table.data_ptr(), _ptr(flat), self.n_seg, self.batch, self.seq_len,
                                            self.row_offset, self.q_len, meta.data_ptr(), meta.numel(),
                                            ctypes.byref(desc), stream))
        return dataclasses.replace(self, table=table, meta=meta, desc=desc, _pinned=pinned)

    def q_order(self):
        """(order, stats) views of the device metadata: the launch order of
        the 32-row query tiles (codes b * n_qt + qt, most key tiles visited
        first) and [largest, total] visits; None when the batch has more
        than 8192 query tiles (no order is built)."""
        B, S, L = self.batch, self.seq_len, self.q_len
        nq = B * ((L + 31) // 32)
        if not 0 < nq <= 8192:
            return None
        o = 2 * B * L + 2 * B * S
        return self.meta[o:o + nq], self.meta[o + nq:o + nq + 2]

    def meta_views(self):
        """(row_lo, row_hi, key_qlo, key_qhi) views of the device metadata."""
        B, S, L = self.batch, self.seq_len, self.q_len
        m = self.meta
        nr, nk = B * L, B * S
        return (m[:nr].view(B, L), m[nr:2 * nr].view(B, L),
                m[2 * nr:2 * nr + nk].view(B, S), m[2 * nr + nk:2 * nr + 2 * nk].view(B, S))


def segment(doc_lens_rows, seq_len, row_offset=0, q_len=None, device=None):
    """Segment table of the chunk [row_offset, row_offset + q_len) of every
    row (``blockdiag_segment``).  ``doc_lens_rows``: one sequence of document
    lengths per batch row; positions past a row's sum are padding."""
    lib = load_library()
    seq_len = int(seq_len)
    row_offset = int(row_offset)
    q_len = seq_len - row_offset if q_len is None else int(q_len)
    rows = [np.asarray(r, dtype=np.int64).ravel() for r in doc_lens_rows]
    batch = len(rows)
    flat = np.concatenate(rows).astype(np.int32) if batch and sum(len(r) for r in rows) else np.zeros(1, np.int32)
    per_row = np.array([len(r) for r in rows] or [0], dtype=np.int32)
    cap = int(sum(len(r) for r in rows) + batch)
    cu_q = np.zeros(cap + 1, np.int32)
    cu_k = np.zeros(cap + 1, np.int32)
    kb = np.zeros(max(cap, 1), np.int32)
    n = ctypes.c_int32(0)
    mq = ctypes.c_int32(0)
    mk = ctypes.c_int32(0)
    _check(lib.blockdiag_segment(_ptr(flat), _ptr(per_row), batch, seq_len, row_offset, q_len, cap,
                                 _ptr(cu_q), _ptr(cu_k), _ptr(kb), ctypes.byref(n), ctypes.byref(mq),
                                 ctypes.byref(mk)))
    ns = n.value
    t = SegTable(batch, seq_len, row_offset, q_len, cu_q[:ns + 1].copy(), cu_k[:ns + 1].copy(),
                 kb[:ns].copy(), ns, mq.value, mk.value)
    return t.to(device) if device is not None else t


def validate(cu_q, cu_k, k_begin, batch, seq_len, row_offset, q_len):
    """Host validation of a segment table built anywhere
    (``blockdiag_validate``); raises BlockdiagError when it is malformed."""
    lib = load_library()
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_k, dtype=np.int32)
    kb = np.ascontiguousarray(k_begin, dtype=np.int32)
    n = len(cu_q) - 1
    if n < 0 or len(cu_k) != n + 1 or len(kb) != n:
        raise BlockdiagError(2, "table arrays have inconsistent lengths")
    kb_arg = _ptr(kb) if n > 0 else _ptr(np.zeros(1, np.int32))
    _check(lib.blockdiag_validate(_ptr(cu_q), _ptr(cu_k), kb_arg, n, batch, seq_len, row_offset, q_len))


def table_from_arrays(cu_q, cu_k, k_begin, batch, seq_len, row_offset, q_len, device=None):
    """Wrap an externally built segment table after validating it."""
    validate(cu_q, cu_k, k_begin, batch, seq_len, row_offset, q_len)
    cu_q = np.asarray(cu_q, np.int32); cu_k = np.asarray(cu_k, np.int32); kb = np.asarray(k_begin, np.int32)
    n = len(kb)
    qn = np.diff(cu_q); kn = np.diff(cu_k)
    t = SegTable(batch, seq_len, row_offset, q_len, cu_q.copy(), cu_k.copy(), kb.copy(), n,
                 int(qn.max(initial=0)), int(kn.max(initial=0)))
    return t.to(device) if device is not None else t


def doc_lens_from_ids(ids):
    """Document lengths of one row from per-token document ids (a 1-D
    sequence; each maximal run of equal ids is one document; negative ids
    mark padding, which may only appear at the end)."""
    ids = np.asarray(ids).ravel()
    lens = []
    i, n = 0, len(ids)
    while i < n and ids[i] >= 0:
        j = i
        while j < n and ids[j] == ids[i]:
            j += 1
        lens.append(j - i)
        i = j
    if np.any(ids[i:] >= 0):
        raise ValueError("padding (negative ids) must only appear at the end of the row")
    return lens


# ---------------------------------------------------------------- attention calls


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    raise BlockdiagError(5, f"dtype {t.dtype} not supported (float32 or bfloat16)")


def _shapes(q, k, v, seg, kv_begin=0):
    """Checks the tensors against the segment table; k, v hold keys
    [kv_begin, kv_begin + k.shape[1]) of every row (the whole row when
    kv_begin = 0 and k.shape[1] = S)."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise BlockdiagError(1, "q must be [B, q_len, H_q, d] and k, v [B, kv_len, H_kv, d]")
    B, L, Hq, d = q.shape
    Bk, W, Hkv, dk = k.shape
    S = seg.seq_len
    if Bk != B or dk != d or B != seg.batch or L != seg.q_len or not 0 <= kv_begin <= kv_begin + W <= S:
        raise BlockdiagError(1, f"shapes q{tuple(q.shape)} k{tuple(k.shape)} (K/V from key {kv_begin}) do not "
                                f"match the segment table (B={seg.batch}, S={seg.seq_len}, q_len={seg.q_len})")
    if q.device.type != "cuda":
        raise BlockdiagError(1, "q, k, v must be contiguous device tensors of one dtype")
    for t in (q, k, v):
        if not t.is_contiguous() or t.device != q.device or t.dtype != q.dtype:
            raise BlockdiagError(1, "q, k, v must be contiguous device tensors of one dtype on one device")
    if seg.meta is None or seg.desc is None or seg.meta.device != q.device:
        raise BlockdiagError(1, "segment table has no device metadata on the tensors' device")
    return B, L, Hq, d, S, Hkv, W


def mark_main_kernel(start_event, stop_event):
    """Profiling hook (``blockdiag_mark_main_kernel``): the next attn_fwd /
    attn_bwd call records these hipEvent_t handles (ints) around its main
    kernel on its stream."""
    _check(load_library().blockdiag_mark_main_kernel(start_event, stop_event))


def clock_probe(out, ticks=2000, stream=None):
    """Measurement aid (``blockdiag_clock_probe``): launches out.numel() // 2
    one-wave workgroups that spin ``ticks`` counts of the 100 MHz real-time
    counter; ``out`` (int64, on the GPU) receives (engine cycles, ticks) per
    workgroup.  Returns nothing; read ``out`` after the stream has run."""
    import torch
    if out.dtype != torch.int64 or not out.is_cuda or not out.is_contiguous() or out.numel() < 2:
        raise BlockdiagError(1, "clock_probe needs a contiguous int64 CUDA tensor of at least 2 elements")
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    _check(load_library().blockdiag_clock_probe(out.numel() // 2, ticks, out.data_ptr(), stream.cuda_stream))


def attn_fwd(q, k, v, seg, scale=None, kv_begin=0, dropout=None):
    """O and LSE of the chunk (``blockdiag_attn_fwd``).  ``k``, ``v`` hold
    keys [kv_begin, kv_begin + k.shape[1]) of every row: the whole row
    (default) or a window with every key the chunk attends (``kv_plan``).
    ``dropout``: None or (p, seed, offset)."""
    import torch
    lib = load_library()
    B, L, Hq, d, S, Hkv, W = _shapes(q, k, v, seg, kv_begin)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    ws_bytes = lib.blockdiag_workspace_bytes(0, dt, B, S, L, Hq, Hkv, d)
    ws = torch.empty(max(int(ws_bytes), 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):  # the library launches on the current device
        _check(lib.blockdiag_attn_fwd(dt, B, S, seg.row_offset, L, kv_begin, W, Hq, Hkv, d, scale,
                                      _dropout_arg(dropout), q.data_ptr(),
                                      k.data_ptr(), v.data_ptr(), ctypes.byref(seg.desc), o.data_ptr(),
                                      lse.data_ptr(), ws.data_ptr(), ws_bytes, stream))
    return o, lse


def attn_bwd(q, k, v, o, lse, do, seg, scale=None, kv_begin=0, dropout=None):
    """dQ, dK, dV of the loss sum(dO * O) (``blockdiag_attn_bwd``); dK, dV
    cover the same keys as ``k``, ``v``; ``dropout`` as given to the
    forward."""
    import torch
    lib = load_library()
    B, L, Hq, d, S, Hkv, W = _shapes(q, k, v, seg, kv_begin)
    for t in (o, do):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise BlockdiagError(1, "o and do must match q (shape, dtype, device, contiguous)")
    if (lse.shape != (B, Hq, L) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise BlockdiagError(1, "lse must be contiguous float32 [B, H_q, q_len] on q's device")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _dtype_code(q)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws_bytes = lib.blockdiag_workspace_bytes(1, dt, B, S, L, Hq, Hkv, d)
    ws = torch.empty(max(int(ws_bytes), 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):  # the library launches on the current device
        _check(lib.blockdiag_attn_bwd(dt, B, S, seg.row_offset, L, kv_begin, W, Hq, Hkv, d, scale,
                                      _dropout_arg(dropout), q.data_ptr(),
                                      k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      do.data_ptr(), ctypes.byref(seg.desc), dq.data_ptr(), dk.data_ptr(),
                                      dv.data_ptr(), ws.data_ptr(), ws_bytes, stream))
    return dq, dk, dv


@dataclasses.dataclass
class KvPlan:
    """Needed-only K/V exchange plan of one context-parallel rank
    (``blockdiag_kv_plan``): the K/V window [kv_begin, kv_end) the rank's
    attention calls take, the ranges it receives and sends as lists of
    (row, peer, begin, end), and the rank's and the step's exchange mode
    (0 none, 1 left-neighbour halo, 2 all-to-all-v)."""
    cp: int
    rank: int
    kv_begin: int
    kv_end: int
    recv: list
    send: list
    rank_mode: int
    step_mode: int


def kv_plan(doc_lens_rows, seq_len, cp, rank, align=64):
    """Needed-only K/V plan of rank ``rank`` of ``cp`` contiguous chunks
    (``blockdiag_kv_plan``)."""
    lib = load_library()
    rows = [np.asarray(r, dtype=np.int64).ravel() for r in doc_lens_rows]
    flat = np.concatenate(rows).astype(np.int32) if rows and sum(len(r) for r in rows) else np.zeros(1, np.int32)
    per = np.array([len(r) for r in rows] or [0], dtype=np.int32)
    cap = 16
    while True:
        recv = (KvRange * cap)()
        send = (KvRange * cap)()
        vals = [ctypes.c_int32(0) for _ in range(6)]
        code = lib.blockdiag_kv_plan(_ptr(flat), _ptr(per), len(rows), int(seq_len), int(cp), int(rank), int(align),
                                     ctypes.byref(vals[0]), ctypes.byref(vals[1]), cap, recv, ctypes.byref(vals[2]),
                                     send, ctypes.byref(vals[3]), ctypes.byref(vals[4]), ctypes.byref(vals[5]))
        if code == 3:
            cap = max(vals[2].value, vals[3].value)
            continue
        _check(code)
        break
    kb, ke, nr, ns, rm, sm = (x.value for x in vals)

    def rng(arr, n):
        return [(arr[i].row, arr[i].peer, arr[i].begin, arr[i].end) for i in range(n)]

    return KvPlan(int(cp), int(rank), kb, ke, rng(recv, nr), rng(send, ns), rm, sm)


def _autograd_fn():
    import torch

    class _BlockdiagAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, seg, scale, kv_begin, dropout):
            o, lse = attn_fwd(q, k, v, seg, scale, kv_begin, dropout)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.seg = seg
            ctx.scale = scale
            ctx.kv_begin = kv_begin
            ctx.dropout = dropout
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = attn_bwd(q, k, v, o, lse, do.contiguous(), ctx.seg, ctx.scale, ctx.kv_begin, ctx.dropout)
            return dq, dk, dv, None, None, None, None

    return _BlockdiagAttention


_FN = None


def attention(q, k, v, seg, scale=None, kv_begin=0, dropout=None):
    """Drop-in attention over a packed chunk with autograd (Design overview,
    runtime.py: a drop-in SDPA; packed.py: row_offset = 0 for one GPU);
    ``kv_begin`` and ``dropout`` (None or (p, seed, offset); the backward
    reuses the forward's) as for ``attn_fwd``."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    return _FN.apply(q, k, v, seg, scale, kv_begin, dropout)
