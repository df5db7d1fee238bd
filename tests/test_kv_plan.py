"""The needed-only K/V exchange plan (blockdiag_kv_plan), CPU only: the
oracle (oracle/kvplan.py, from the dense block-causal mask) pinned to plans
derived by hand (tests/golden/kv_plan_hand.json), then the library's
planner bit-exact against the oracle for cp in {2, 3, 4, 8} on random
layouts (padding tails, zero-length documents, all-padding ranks, documents
spanning several ranks) and on the S = 16384 workload whose chunk at 8192
straddles a document; plus the plan's own consistency: every rank's receive
ranges are the send ranges addressed to it, and receive plus own chunk cover
every key its rows attend."""
import json
import os

import numpy as np
import pytest

import packed_sequence_attention_amd as bd
import synthetic
from oracle import kvplan as KP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _as_lists(r):
    return [list(x) for x in r]


def test_oracle_matches_hand_worked_plans():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "kv_plan_hand.json")))
    for c in g["cases"]:
        for rank, want in enumerate(c["ranks"]):
            got = KP.kv_plan_ref(c["doc_lens"], c["seq_len"], c["cp"], rank, c["align"])
            assert got["kv_begin"] == want["kv_begin"] and got["kv_end"] == want["kv_end"], (c["why"], rank)
            assert _as_lists(got["recv"]) == want["recv"], (c["why"], rank)
            assert _as_lists(got["send"]) == want["send"], (c["why"], rank)
            assert got["rank_mode"] == want["rank_mode"] and got["step_mode"] == c["step_mode"]


def _check_same(rows, S, cp, align=64):
    for rank in range(cp):
        ref = KP.kv_plan_ref(rows, S, cp, rank, align)
        got = bd.kv_plan(rows, S, cp, rank, align)
        assert (got.kv_begin, got.kv_end) == (ref["kv_begin"], ref["kv_end"]), (rows, S, cp, rank)
        assert got.recv == ref["recv"] and got.send == ref["send"], (rows, S, cp, rank)
        assert (got.rank_mode, got.step_mode) == (ref["rank_mode"], ref["step_mode"])


def test_library_matches_oracle_on_hand_cases():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "kv_plan_hand.json")))
    for c in g["cases"]:
        _check_same(c["doc_lens"], c["seq_len"], c["cp"], c["align"])


@pytest.mark.parametrize("cp", [2, 3, 4, 8])
def test_library_matches_oracle_random(cp):
    rng = np.random.default_rng(100 + cp)
    for _ in range(25):
        B = int(rng.integers(1, 4))
        S = cp * int(rng.integers(1, 40))
        rows = []
        for _b in range(B):
            lens, tot = [], 0
            fill = S if rng.random() < 0.5 else int(rng.integers(0, S + 1))
            long_docs = rng.random() < 0.3
            while tot < fill:
                Ln = int(min(rng.integers(0, S if long_docs else 12), fill - tot))
                lens.append(Ln)
                tot += Ln
            rows.append(lens)
        _check_same(rows, S, cp, align=int(rng.choice([1, 4, 64])))


def test_straddling_workload_plan():
    """Workload 3's packing (S = 16384, cp = 4): every chunk bound lies inside
    a document, each straddle reaches only the left neighbour (halo p2p)."""
    w = synthetic.workload(3)
    rows = [list(r) for r in w.doc_lens]
    _check_same(rows, w.seq_len, 4)
    p2 = bd.kv_plan(rows, w.seq_len, 4, 2)
    assert p2.recv == [(0, 1, 7039, 8192)] and p2.kv_begin == 6976 and p2.kv_end == 12288
    assert p2.rank_mode == 1 and p2.step_mode == 1


def test_plan_is_consistent_across_ranks():
    rng = np.random.default_rng(5)
    for cp in (2, 4, 8):
        S = 64 * cp
        rows = [[int(x) for x in rng.integers(1, 3 * S // cp, size=20)] for _ in range(2)]
        rows = [[x for x in r if x > 0] for r in rows]
        rows = [r[:int(np.searchsorted(np.cumsum(r), S, side="right"))] for r in rows]
        plans = [bd.kv_plan(rows, S, cp, r) for r in range(cp)]
        for r, p in enumerate(plans):
            sent_to_r = sorted((row, src.rank, a, e) for src in plans for (row, peer, a, e) in src.send if peer == r)
            assert sorted(p.recv) == sent_to_r
            need = KP.needed_keys(rows, S, cp, r)
            for b in range(len(rows)):
                have = np.zeros(S, bool)
                have[r * S // cp:(r + 1) * S // cp] = True
                for (row, _q, a, e) in p.recv:
                    if row == b:
                        have[a:e] = True
                assert not np.any(need[b] & ~have)
                assert np.all(np.nonzero(need[b])[0] >= p.kv_begin)


def test_plan_rejects_bad_input():
    with pytest.raises(bd.BlockdiagError):
        bd.kv_plan([[4, 4]], 9, 2, 0)      # seq_len not a multiple of cp
    with pytest.raises(bd.BlockdiagError):
        bd.kv_plan([[4, 4]], 8, 2, 2)      # rank out of range
    with pytest.raises(bd.BlockdiagError) as e:
        bd.kv_plan([[6, 6]], 8, 2, 0)      # documents longer than the row
    assert e.value.code == 2
