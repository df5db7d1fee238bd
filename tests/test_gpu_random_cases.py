"""Seeded random configurations against the fp64 oracle (Automodel page,
Proof: forward/backward parity on packed varlen inputs).

Eight cases drawn once from a fixed generator: dtype, GQA ratio 1-8, one or two
batch rows, document lengths from single tokens to the whole row with
optional padding tails, and a chunk [row_offset, row_offset + q_len) placed
anywhere in the row, each head_dim path (the matrix-core 64 / 128 / 256,
the generic 96) twice -- combinations the hand-picked cases do not reach.
Tolerances as for every parity case (tests/helpers.py)."""
import sys

import numpy as np
import pytest

from tests import helpers as H

gpu = pytest.mark.gpu


def _draw_cases(seed=4242, n=8):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        dtype = "f32" if k == 0 else "bf16"
        d = (64, 128, 256, 96)[k % 4]  # every head_dim path twice
        h_kv = int(rng.choice([1, 2]))
        h_q = h_kv * int(rng.choice([1, 2, 4, 8]))
        batch = int(rng.choice([1, 2]))
        S = int(rng.integers(96, 600))
        rows = []
        for _ in range(batch):
            fill = S if rng.random() < 0.6 else int(rng.integers(S // 2, S + 1))
            hi = int(rng.choice([8, 64, 256, S]))
            lens, tot = [], 0
            while tot < fill:
                ln = int(min(rng.integers(1, hi + 1), fill - tot))
                lens.append(ln)
                tot += ln
            rows.append(lens)
        r0 = int(rng.integers(0, S // 2 + 1))
        q_len = int(rng.integers(1, S - r0 + 1))
        cases.append((dtype, rows, S, r0, q_len, h_q, h_kv, d))
    return cases


CASES = _draw_cases()


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@gpu
@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_case_parity(i):
    dtype, docs, S, r0, L, hq, hkv, d = CASES[i]
    _log(f"random case {i}: {dtype} B={len(docs)} S={S} r0={r0} L={L} H={hq}/{hkv} d={d} "
         f"docs={[len(r) for r in docs]}")
    w, t = H.small_case(200 + i, dtype, docs, S, r0, L, hq, hkv, d)
    gpu_out = H.run_gpu(w, t)
    ref = H.oracle(w, t, block_rows=None)
    errs = H.check(w, gpu_out, ref)
    _log("  errors", {k: f"{v:.3g}" for k, v in errs.items()})


def test_random_cases_are_valid_layouts():
    """The drawn layouts are what the segmenter accepts (CPU check)."""
    for dtype, docs, S, r0, L, hq, hkv, d in CASES:
        assert all(sum(r) <= S for r in docs)
        assert 0 <= r0 and r0 + L <= S and L >= 1
        assert hq % hkv == 0 and d % 8 == 0
