"""The host segmenter and validator (segment.cpp, no HIP dependency) built
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run over
the segmenter and validator cases of the ABI tests plus a seeded fuzz of
valid and corrupted tables (CPU only).  Every case must run clean, and its
result must equal the normal library's result through the Python binding
(bit-exact tables, same status codes)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import packed_sequence_attention_amd as bd
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def replay(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("san") / "replay")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "packed_sequence_attention_amd", "csrc", "segment.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "replay.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("sanitizer build unavailable: " + r.stderr[-500:])
    return out


def _seg_line(rows, S, r0, L, cap):
    per = [len(r) for r in rows]
    flat = [int(x) for r in rows for x in r]
    return " ".join(map(str, ["S", len(rows), S, r0, L, cap, *per, *flat]))


def _val_line(cu_q, cu_k, kb, B, S, r0, L):
    n = len(cu_q) - 1
    return " ".join(map(str, ["V", n, B, S, r0, L, *cu_q, *cu_k, *kb]))


def _binding_seg(rows, S, r0, L, cap):
    import ctypes
    lib = bd.load_library()
    per = np.array([len(r) for r in rows] or [0], np.int32)
    flat = np.array([int(x) for r in rows for x in r] or [0], np.int32)
    cu_q = np.zeros(cap + 1, np.int32); cu_k = np.zeros(cap + 1, np.int32); kb = np.zeros(max(cap, 1), np.int32)
    n, mq, mk = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = lib.blockdiag_segment(bd._ptr(flat), bd._ptr(per), len(rows), S, r0, L, cap, bd._ptr(cu_q), bd._ptr(cu_k),
                               bd._ptr(kb), ctypes.byref(n), ctypes.byref(mq), ctypes.byref(mk))
    out = [st]
    if st == 0:
        k = n.value
        out += [k, mq.value, mk.value, *cu_q[:k + 1], *cu_k[:k + 1], *kb[:k]]
    elif st == 3:
        out.append(n.value)
    return " ".join(map(str, out))


def _binding_val(cu_q, cu_k, kb, B, S, r0, L):
    try:
        bd.validate(cu_q, cu_k, kb, B, S, r0, L)
        return "0"
    except bd.BlockdiagError as e:
        return str(e.code)


def _cases():
    rng = np.random.default_rng(2024)
    seg, val = [], []
    for wid in synthetic.WORKLOADS:
        w = synthetic.workload(wid)
        seg.append((w.doc_lens, w.seq_len, w.row_offset, w.q_len, w.n_docs + w.batch))
    seg += [([[3, -1]], 4, 0, 4, 3), ([[3, 2]], 4, 0, 4, 3), ([[4]], 4, 2, 3, 2),   # rejected inputs
            ([[2, 2, 2]], 8, 0, 8, 2), ([[0, 5, 0, 3]], 10, 2, 8, 5), ([[40]], 128, 64, 64, 2),
            ([[7]], 7, 7, 0, 1), ([], 0, 0, 0, 0)]
    for _ in range(150):
        B = int(rng.integers(1, 4)); S = int(rng.integers(1, 200))
        rows = []
        for _b in range(B):
            lens, tot = [], 0
            fill = S if rng.random() < 0.5 else int(rng.integers(0, S + 1))
            while tot < fill:
                Ln = int(min(rng.integers(0, 50), fill - tot)); lens.append(Ln); tot += Ln
            rows.append(lens)
        a = int(rng.integers(0, S)); b = int(rng.integers(a, S + 1))
        cap = sum(len(r) for r in rows) + B
        seg.append((rows, S, a, b - a, cap if rng.random() < 0.8 else int(rng.integers(0, cap + 1))))
        t = bd.segment(rows, S, a, b - a)
        args = (B, S, a, b - a)
        val.append((list(t.cu_q), list(t.cu_k), list(t.k_begin), *args))
        for _m in range(3):  # corrupt one entry of one array
            cq, ck, kb = list(t.cu_q), list(t.cu_k), list(t.k_begin)
            arr = [cq, ck, kb][int(rng.integers(0, 3))]
            if arr:
                i = int(rng.integers(0, len(arr)))
                arr[i] += int(rng.choice([-3, -1, 1, 2, 1000, -1000]))
            val.append((cq, ck, kb, *args))
    # the empty-chunk divisions the validator must refuse before dividing
    val += [([0, 5, 0], [0, 5, 0], [0, 0], 1, 8, 0, 0), ([0, 5, 0], [0, 5, 0], [0, 0], 0, 8, 0, 4),
            ([0], [0], [], 0, 0, 0, 0)]
    return seg, val


def test_segmenter_and_validator_clean_under_sanitizers(replay):
    seg, val = _cases()
    lines = [_seg_line(*c) for c in seg] + [_val_line(*c) for c in val]
    expect = [_binding_seg(*c) for c in seg] + [_binding_val(*c) for c in val]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([replay], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-2000:]
    got = r.stdout.strip().split("\n")
    assert len(got) == len(expect)
    for i, (g, e) in enumerate(zip(got, expect)):
        assert g == e, (i, lines[i][:200], g[:200], e[:200])
