"""CPU tests of the C ABI: the library loads and exports every function
include/blockdiag.h declares; the host segmenter is bit-exact against the
oracle's reference table; the validator rejects malformed tables; the
attention entry points reject bad arguments before launching anything.
(No kernel is launched here.)"""
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
    assert fwd(1, 1, 64, 0, 64, 6, 4, 64, 0.125, N, N, N, N, N, N, N, 0, N) == 1
    # unsupported head_dim
    assert fwd(1, 1, 64, 0, 64, 4, 4, 60, 0.125, N, N, N, N, N, N, N, 0, N) == 5
    assert fwd(1, 1, 64, 0, 64, 4, 4, 512, 0.125, N, N, N, N, N, N, N, 0, N) == 5
    # chunk out of range
    assert fwd(1, 1, 64, 32, 64, 4, 4, 64, 0.125, N, N, N, N, N, N, N, 0, N) == 1
    # unknown dtype
    assert fwd(7, 1, 64, 0, 64, 4, 4, 64, 0.125, N, N, N, N, N, N, N, 0, N) == 5
    # null tensors
    assert fwd(1, 1, 64, 0, 64, 4, 4, 64, 0.125, N, N, N, N, N, N, N, 0, N) == 1
    # empty chunk is a no-op
    assert fwd(1, 1, 64, 0, 0, 4, 4, 64, 0.125, N, N, N, N, N, N, N, 0, N) == 0
    bwd = lib.blockdiag_attn_bwd
    assert bwd(1, 1, 64, 0, 64, 6, 4, 64, 0.125, *([N] * 11), 0, N) == 1
    # backward workspace too small (checked before anything runs)
    ws = lib.blockdiag_workspace_bytes(1, 1, 1, 64, 64, 4, 4, 64)
    assert ws > 0
    p = 16  # a non-null dummy value; never dereferenced because the check fails first
    assert bwd(1, 1, 64, 0, 64, 4, 4, 64, 0.125, *([p] * 10), p, ws - 1, N) == 4
    assert b"workspace" in lib.blockdiag_last_error()
    # metadata build rejects an empty table for a non-empty chunk
    assert lib.blockdiag_meta_build(p, 0, 1, 64, 0, 64, p, N) == 2
    # bounds of rows and keys, then the order of the 32-row query tiles and its two statistics
    assert lib.blockdiag_meta_ints(2, 100, 40) == 2 * 2 * 40 + 2 * 2 * 100 + 2 * 2 + 2


def test_meta_build_host_rejects_before_launch():
    """The by-value metadata entry point checks its arguments and the table
    size on the host and launches nothing when they fail."""
    lib = bd.load_library()
    N = None
    mx = lib.blockdiag_meta_inline_max_seg()
    assert mx >= 64
    table = np.zeros(3 * (mx + 1) + 2, np.int32)
    p = 16  # non-null dummy device pointer; never dereferenced because the check fails first
    # one segment over the limit: capacity error, the caller falls back to the device copy
    assert lib.blockdiag_meta_build_host(bd._ptr(table), mx + 1, 1, 64, 0, 64, p, N) == 3
    assert b"segments" in lib.blockdiag_last_error()
    # empty table for a non-empty chunk; negative sizes; chunk out of range; null pointers
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 0, 1, 64, 0, 64, p, N) == 2
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 1, -1, 64, 0, 64, p, N) == 1
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 1, 1, 64, 32, 64, p, N) == 1
    assert lib.blockdiag_meta_build_host(N, 1, 1, 64, 0, 64, p, N) == 1
    assert lib.blockdiag_meta_build_host(bd._ptr(table), 1, 1, 64, 0, 64, N, N) == 1
    # nothing to build is a no-op
    assert lib.blockdiag_meta_build_host(N, 0, 0, 0, 0, 0, N, N) == 0


def test_doc_lens_from_ids():
    assert bd.doc_lens_from_ids([0, 0, 0, 1, 2, 2, -1, -1]) == [3, 1, 2]
    assert bd.doc_lens_from_ids([5, 5, 5, 5]) == [4]
    assert bd.doc_lens_from_ids([-1, -1]) == []
    with pytest.raises(ValueError):
        bd.doc_lens_from_ids([0, -1, 1])
