"""CPU tests of the C ABI: the library loads and exports every function
include/blockdiag.h declares; the host segmenter is bit-exact against the
oracle's reference table; the validator rejects malformed tables; the
attention entry points reject bad arguments before launching anything.
(No kernel is launched here.)"""
import ctypes
import os
import re

import numpy as np
import pytest

import packed_sequence_attention_amd as bd
import synthetic
from oracle import segment as SEG

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session", autouse=True)
def _library():
    if not os.path.exists(bd.library_path()):
        from packed_sequence_attention_amd import build
        build.build_library()
    return bd.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "blockdiag.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(blockdiag_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = bd.load_library()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bd.EXPORTS)
    assert lib.blockdiag_version().decode().startswith("blockdiag")


def _cmp(layout, S, r0, L):
    ref = SEG.segment_ref(layout, S, r0, L)
    t = bd.segment(layout, S, r0, L)
    assert t.cu_q.tolist() == ref["cu_q"]
    assert t.cu_k.tolist() == ref["cu_k"]
    assert t.k_begin.tolist() == ref["k_begin"]
    assert (t.n_seg, t.max_q, t.max_k) == (ref["n_seg"], ref["max_q"], ref["max_k"])
    return t


@pytest.mark.parametrize("wid", synthetic.WORKLOADS)
def test_segment_bit_exact_on_workloads(wid):
    w = synthetic.workload(wid)
    t = _cmp(w.doc_lens, w.seq_len, w.row_offset, w.q_len)
    if wid == 3:  # the straddling chunk: first segment has more keys than rows
        assert (t.cu_q[1], t.cu_k[1], t.k_begin[0]) == (671, 1824, 7039)


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_segment_bit_exact_fuzz(cp):
    rng = np.random.default_rng(cp)
    for _ in range(40):
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 300))
        rows = []
        for _b in range(B):
            lens, tot = [], 0
            fill = S if rng.random() < 0.5 else int(rng.integers(0, S + 1))
            while tot < fill:
                Ln = int(min(rng.integers(0, 60), fill - tot))
                lens.append(Ln)
                tot += Ln
            rows.append(lens)
        bounds = np.linspace(0, S, cp + 1).astype(int)
        for a, b in zip(bounds[:-1], bounds[1:]):
            _cmp(rows, S, int(a), int(b - a))


def test_segment_hand_tables():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "segments_hand.json")))
    for c in g["cases"]:
        t = bd.segment(c["doc_lens"], c["seq_len"], c["row_offset"], c["q_len"])
        assert t.cu_q.tolist() == c["cu_q"] and t.cu_k.tolist() == c["cu_k"]
        assert t.k_begin.tolist() == c["k_begin"]


def test_segment_rejects_bad_input():
    with pytest.raises(bd.BlockdiagError) as e:
        bd.segment([[3, -1]], 4)
    assert e.value.code == 2
    with pytest.raises(bd.BlockdiagError) as e:
        bd.segment([[3, 2]], 4)
    assert e.value.code == 2
    with pytest.raises(bd.BlockdiagError) as e:
        bd.segment([[4]], 4, 2, 3)
    assert e.value.code == 1


def test_segment_capacity_reports_need():
    import ctypes
    lib = bd.load_library()
    docs = np.array([2, 2, 2], np.int32)
    per = np.array([3], np.int32)
    cu = np.zeros(3, np.int32); ck = np.zeros(3, np.int32); kb = np.zeros(2, np.int32)
    n, mq, mk = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    code = lib.blockdiag_segment(P(docs), P(per), 1, 8, 0, 8, 2, P(cu), P(ck), P(kb), ctypes.byref(n),
                                 ctypes.byref(mq), ctypes.byref(mk))
    assert code == 3 and n.value == 4  # three documents + padding


def test_validate_accepts_and_rejects():
    w = synthetic.workload(3)
    t = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len)
    args = (w.batch, w.seq_len, w.row_offset, w.q_len)
    bd.validate(t.cu_q, t.cu_k, t.k_begin, *args)
    bad = []
    cq = t.cu_q.copy(); cq[-1] += 1; bad.append((cq, t.cu_k, t.k_begin))          # bad terminal offset
    cq = t.cu_q.copy(); cq[1] = cq[2]; bad.append((cq, t.cu_k, t.k_begin))        # not increasing
    ck = t.cu_k.copy(); ck[1] -= 1; bad.append((t.cu_q, ck, t.k_begin))           # keys do not end at row
    kb = t.k_begin.copy(); kb[1] += 1; bad.append((t.cu_q, t.cu_k, kb))           # gap / shifted keys
    kb = t.k_begin.copy(); kb[0] = -5; bad.append((t.cu_q, t.cu_k, kb))           # outside the row
    ck = t.cu_k.copy(); ck[2:] += 3; kb = t.k_begin.copy(); kb[1] -= 3
    bad.append((t.cu_q, ck, kb))                                                   # 2nd segment starts left
    for cq, ck, kb in bad:
        with pytest.raises(bd.BlockdiagError) as e:
            bd.validate(cq, ck, kb, *args)
        assert e.value.code == 2
    # segments for an empty chunk (q_len = 0, or batch = 0): rejected before
    # any per-segment arithmetic divides by q_len
    for dims in ((1, 8, 0, 0), (0, 8, 0, 4)):
        with pytest.raises(bd.BlockdiagError) as e:
            bd.validate([0, 5, 0], [0, 5, 0], [0, 0], *dims)
        assert e.value.code == 2
    # padding segment must end the chunk and start at its first row
    t = bd.segment([[3, 4], [6, 4]], 10, 4, 4)
    bd.validate(t.cu_q, t.cu_k, t.k_begin, 2, 10, 4, 4)
    kb = t.k_begin.copy(); kb[1] += 1
    with pytest.raises(bd.BlockdiagError):
        bd.validate(t.cu_q, t.cu_k, kb, 2, 10, 4, 4)


def test_attention_entry_points_reject_before_launch():
    """Bad arguments return an error code with no kernel launched (null
    device pointers are never dereferenced because the checks come first)."""
    lib = bd.load_library()
    N = None
    fwd = lambda *a: lib.blockdiag_attn_fwd(*a)  # noqa: E731
    # h_q not a multiple of h_kv
    assert fwd(1, 1, 64, 0, 64, 0, 64, 6, 4, 64, 0.125, None, N, N, N, N, N, N, N, 0, N) == 1
    # unsupported head_dim
    assert fwd(1, 1, 64, 0, 64, 0, 64, 4, 4, 60, 0.125, None, N, N, N, N, N, N, N, 0, N) == 5
    assert fwd(1, 1, 64, 0, 64, 0, 64, 4, 4, 512, 0.125, None, N, N, N, N, N, N, N, 0, N) == 5
    # chunk out of range
    assert fwd(1, 1, 64, 32, 64, 0, 64, 4, 4, 64, 0.125, None, N, N, N, N, N, N, N, 0, N) == 1
    # unknown dtype
    assert fwd(7, 1, 64, 0, 64, 0, 64, 4, 4, 64, 0.125, None, N, N, N, N, N, N, N, 0, N) == 5
    # null tensors
    assert fwd(1, 1, 64, 0, 64, 0, 64, 4, 4, 64, 0.125, None, N, N, N, N, N, N, N, 0, N) == 1
    # empty chunk is a no-op
    assert fwd(1, 1, 64, 0, 0, 0, 64, 4, 4, 64, 0.125, None, N, N, N, N, N, N, N, 0, N) == 0
    bwd = lib.blockdiag_attn_bwd
    assert bwd(1, 1, 64, 0, 64, 0, 64, 6, 4, 64, 0.125, None, *([N] * 11), 0, N) == 1
    # backward workspace too small (checked before anything runs)
    ws = lib.blockdiag_workspace_bytes(1, 1, 1, 64, 64, 4, 4, 64)
    assert ws > 0
    p = 16  # a non-null dummy value; never dereferenced because the check fails first
    m = _desc(1, 64, 0, 64)
    assert bwd(1, 1, 64, 0, 64, 0, 64, 4, 4, 64, 0.125, None, p, p, p, p, p, p, ctypes.byref(m), p, p, p, p, ws - 1, N) == 4
    assert b"workspace" in lib.blockdiag_last_error()
    # metadata build rejects an empty table for a non-empty chunk
    desc = bd.MetaDesc()
    cap = lib.blockdiag_meta_ints(1, 64, 64)
    assert lib.blockdiag_meta_build(p, None, 0, 1, 64, 0, 64, p, cap, ctypes.byref(desc), N) == 2
    assert desc.magic == 0
    # ... a metadata buffer smaller than blockdiag_meta_ints, and a missing descriptor
    assert lib.blockdiag_meta_build(p, None, 1, 1, 64, 0, 64, p, cap - 1, ctypes.byref(desc), N) == 3
    assert lib.blockdiag_meta_build(p, None, 1, 1, 64, 0, 64, p, cap, None, N) == 1
    # bounds of rows and keys, the order of the 32-row query tiles and its two
    # statistics, then the bins: a count and 3 per bin, at most
    # batch * (2 * ceil((q_len + 127) / 128) + 1) of them
    assert lib.blockdiag_meta_ints(2, 100, 40) == 2 * 2 * 40 + 2 * 2 * 100 + 2 * 2 + 2 + 1 + 3 * 2 * (2 * 2 + 1)
    assert lib.blockdiag_meta_ints(1, 1000, 1000) == 2 * 1000 + 2 * 1000 + 32 + 2 + 1 + 3 * (2 * 9 + 1)


def test_meta_build_host_rejects_before_launch():
    """The by-value metadata entry point checks its arguments and the table
    size on the host and launches nothing when they fail."""
    lib = bd.load_library()
    N = None
    mx = lib.blockdiag_meta_inline_max_seg()
    assert mx >= 64
    table = np.zeros(3 * (mx + 1) + 2, np.int32)
    p = 16  # non-null dummy device pointer; never dereferenced because the check fails first
    cap = lib.blockdiag_meta_ints(1, 64, 64)
    desc = bd.MetaDesc()
    d = ctypes.byref(desc)
    # one segment over the limit: capacity error, the caller falls back to the device copy
    assert lib.blockdiag_meta_build_host(bd._ptr(table), mx + 1, 1, 64, 0, 64, p, cap, d, N) == 3
    assert b"segments" in lib.blockdiag_last_error()
    # empty table for a non-empty chunk; negative sizes; chunk out of range; null pointers
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 0, 1, 64, 0, 64, p, cap, d, N) == 2
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 1, -1, 64, 0, 64, p, cap, d, N) == 1
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 1, 1, 64, 32, 64, p, cap, d, N) == 1
    assert lib.blockdiag_meta_build_host(N, 1, 1, 64, 0, 64, p, cap, d, N) == 1
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 1, 1, 64, 0, 64, N, cap, d, N) == 1
    # metadata buffer too small for the sizes
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 1, 1, 64, 0, 64, p, cap - 1, d, N) == 3
    assert desc.magic == 0
    # nothing to build is a no-op that still describes the (empty) buffer
    assert lib.blockdiag_meta_build_host(N, 0, 0, 0, 0, 0, N, 0, d, N) == 0
    assert desc.magic == bd.META_MAGIC and desc.n_ints == 0


def _desc(batch, seq_len, row_offset, q_len, n_ints=None, magic=None, data=16, kv_lo=0, kv_hi=None):
    lib = bd.load_library()
    m = bd.MetaDesc()
    m.magic = bd.META_MAGIC if magic is None else magic
    m.batch, m.seq_len, m.row_offset, m.q_len = batch, seq_len, row_offset, q_len
    m.kv_lo, m.kv_hi = kv_lo, row_offset + q_len if kv_hi is None else kv_hi
    m.n_seg = 1
    m.n_ints = lib.blockdiag_meta_ints(batch, seq_len, q_len) if n_ints is None else n_ints
    m.data = data
    return m


def test_attention_rejects_metadata_built_for_other_sizes():
    """The kernels index the metadata with the call's own sizes, so a
    descriptor built for another chunk (smaller q_len, other row_offset or
    seq_len), a descriptor that was never built, one whose buffer is too
    small and a missing one are all rejected on the host with
    BD_ERR_INVALID_ARG before anything is launched (every tensor pointer
    below is a dummy that a launch would fault on)."""
    lib = bd.load_library()
    p = 16
    args = (1, 2, 256, 64, 128, 0, 256, 8, 2, 64, 0.125)  # bf16, B=2, S=256, chunk [64, 192), whole-row K/V
    ws = lib.blockdiag_workspace_bytes(1, 1, 2, 256, 128, 8, 2, 64)
    bad = [_desc(2, 256, 64, 64),                  # built for a smaller chunk
           _desc(2, 256, 0, 128),                  # other row_offset
           _desc(2, 128, 0, 128),                  # other seq_len
           _desc(1, 256, 64, 128),                 # other batch
           _desc(2, 256, 64, 128, magic=0),        # never built
           _desc(2, 256, 64, 128, n_ints=100),     # buffer smaller than the sizes need
           _desc(2, 256, 64, 128, data=None)]      # no buffer
    for m in bad:
        assert lib.blockdiag_attn_fwd(*args, None, p, p, p, ctypes.byref(m), p, p, p, 0, None) == 1
        assert b"metadata" in lib.blockdiag_last_error()
        assert lib.blockdiag_attn_bwd(*args, None, p, p, p, p, p, p, ctypes.byref(m), p, p, p, p, ws, None) == 1
        assert b"metadata" in lib.blockdiag_last_error()
    assert lib.blockdiag_attn_fwd(*args, None, p, p, p, None, p, p, p, 0, None) == 1
    assert lib.blockdiag_attn_bwd(*args, None, p, p, p, p, p, p, None, p, p, p, p, ws, None) == 1


def test_doc_lens_from_ids():
    assert bd.doc_lens_from_ids([0, 0, 0, 1, 2, 2, -1, -1]) == [3, 1, 2]
    assert bd.doc_lens_from_ids([5, 5, 5, 5]) == [4]
    assert bd.doc_lens_from_ids([-1, -1]) == []
    with pytest.raises(ValueError):
        bd.doc_lens_from_ids([0, -1, 1])


def test_attention_rejects_bad_kv_windows():
    """K/V windows (kv_begin, kv_len) are checked on the host before any
    launch: start a multiple of 64, at most row_offset, inside the row,
    reaching the chunk's end, and holding every key the descriptor says the
    chunk attends [kv_lo, kv_hi)."""
    lib = bd.load_library()
    p = 16
    B, S, r0, L, Hq, Hkv, d = 1, 512, 256, 128, 4, 1, 64
    ws = lib.blockdiag_workspace_bytes(1, 1, B, S, L, Hq, Hkv, d)
    m = _desc(B, S, r0, L, kv_lo=200, kv_hi=384)   # the chunk attends keys [200, 384)

    def fwd(kb, kl):
        return lib.blockdiag_attn_fwd(1, B, S, r0, L, kb, kl, Hq, Hkv, d, 0.125, None, p, p, p, ctypes.byref(m), p, p, p,
                                      0, None)

    def bwd(kb, kl):
        return lib.blockdiag_attn_bwd(1, B, S, r0, L, kb, kl, Hq, Hkv, d, 0.125, None, p, p, p, p, p, p, ctypes.byref(m),
                                      p, p, p, p, ws, None)

    bad = [(100, 284),   # start not a multiple of 64
           (256, 128),   # starts after key 200, which row 256 attends
           (-64, 512),   # negative start
           (128, 200),   # ends at 328 < 384: misses the chunk's end
           (0, 576),     # past the row
           (320, 64)]    # after row_offset
    for kb, kl in bad:
        assert fwd(kb, kl) == 1, (kb, kl)
        assert bwd(kb, kl) == 1, (kb, kl)
    m2 = _desc(B, S, r0, L, kv_lo=200, kv_hi=400)  # attends past the window end
    assert lib.blockdiag_attn_fwd(1, B, S, r0, L, 192, 192, Hq, Hkv, d, 0.125, None, p, p, p, ctypes.byref(m2), p, p, p,
                                  0, None) == 1
    assert b"misses keys" in lib.blockdiag_last_error()


def test_attention_rejects_bad_dropout():
    """A dropout probability outside [0, 1) (or NaN) is refused on the host."""
    lib = bd.load_library()
    p = 16
    m = _desc(1, 64, 0, 64)
    for prob in (-0.1, 1.0, 1.5, float("nan")):
        dr = ctypes.byref(bd.Dropout(prob, 0, 1))
        assert lib.blockdiag_attn_fwd(1, 1, 64, 0, 64, 0, 64, 4, 4, 64, 0.125, dr, p, p, p, ctypes.byref(m), p, p,
                                      p, 0, None) == 1
        assert b"dropout" in lib.blockdiag_last_error()


def test_clock_probe_rejects_before_launch():
    """The clock probe checks its arguments on the host and launches
    nothing when they fail."""
    lib = bd.load_library()
    p = 16
    assert lib.blockdiag_clock_probe(0, 2000, p, None) == 1
    assert lib.blockdiag_clock_probe(65537, 2000, p, None) == 1
    assert lib.blockdiag_clock_probe(8, 0, p, None) == 1
    assert lib.blockdiag_clock_probe(8, 10000001, p, None) == 1
    assert lib.blockdiag_clock_probe(8, 2000, None, None) == 1
    assert b"clock_probe" in lib.blockdiag_last_error()
