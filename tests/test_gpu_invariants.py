"""GPU invariants of the HIP path that hold at any size:

* chunk concatenation (key property 1 of the Automodel page "feat(
  distributed): block-diagonal varlen CP for packed sequences"): O and LSE of
  contiguous chunks concatenated equal the single full call bit for bit
  (key tiles are anchored at fixed positions of the row, so a row's
  arithmetic does not depend on the chunk), and so does dQ from the tile
  kernels (its rows are computed independently, over the same key tiles;
  these tests keep every call on the tile kernels, since a chunk of only
  short documents would otherwise take the short-document kernel, which sums
  in another order); dK/dV sum over chunks to the full call's within
  tolerance;
* forward and backward are bitwise deterministic (a replayed forward under
  activation checkpointing equals the original, Design overview, packed.py);
* documents are independent: changing one document's inputs leaves every
  other document's O, LSE, dK and dV bit for bit unchanged;
* the launch order does not change a result: the forward and dQ kernels
  run their query tiles longest first when the metadata's statistics say
  so, otherwise in a fixed order; both give the same bits;
* the autograd wrapper returns the raw calls' results;
* window-only K/V (the needed-only exchange's buffers, built from the
  planner's ranges) gives the whole-row call's bits.
"""
import numpy as np
import pytest

import synthetic
from tests import helpers as H

gpu = pytest.mark.gpu


def _w2_small():
    # workload-2-like packing at S = 2048 (lognormal doc lengths), bf16 32/8/128
    rng = np.random.default_rng(7)
    lens, tot = [], 0
    while tot < 2048:
        Ln = int(min(max(int(np.rint(rng.lognormal(np.log(300), 1.0))), 16), 2048 - tot)); lens.append(Ln); tot += Ln
    return lens


@gpu
@pytest.mark.parametrize("cp", [2, 4, 8])
def test_chunk_concatenation(cp):
    import torch
    import packed_sequence_attention_amd as bd
    docs = [_w2_small()]
    S = 2048
    w, t = H.small_case(200 + cp, "bf16", docs, S, 0, S, 32, 8, 128)
    d = H.to_device(w, t)
    full = H.tile_path(bd.segment(docs, S, 0, S, device="cuda"))
    o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], full)
    dq, dk, dv = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], full)
    dk_sum = torch.zeros_like(dk, dtype=torch.float32)
    dv_sum = torch.zeros_like(dv, dtype=torch.float32)
    bounds = np.linspace(0, S, cp + 1).astype(int)
    for a, b in zip(bounds[:-1], bounds[1:]):
        seg = H.tile_path(bd.segment(docs, S, int(a), int(b - a), device="cuda"))
        qc = d["q"][:, a:b].contiguous(); doc_ = d["do"][:, a:b].contiguous()
        oc, lc = bd.attn_fwd(qc, d["k"], d["v"], seg)
        assert torch.equal(oc, o[:, a:b]), "O differs from the full call"
        assert torch.equal(lc, lse[:, :, a:b]), "LSE differs from the full call"
        dqc, dkc, dvc = bd.attn_bwd(qc, d["k"], d["v"], oc, lc, doc_, seg)
        assert torch.equal(dqc, dq[:, a:b]), "dQ differs from the full call"
        dk_sum += dkc.float(); dv_sum += dvc.float()
    assert H.rel_fro(dk_sum.double().cpu().numpy(), dk.double().cpu().numpy()) < 1e-2
    assert H.rel_fro(dv_sum.double().cpu().numpy(), dv.double().cpu().numpy()) < 1e-2


@gpu
def test_chunk_concatenation_head_dim_256():
    """The head_dim 256 kernels keep the same key-tile anchoring: uneven
    chunks (bounds not multiples of the 32-row tile) give O, LSE and dQ
    equal bit for bit to the single full call."""
    import torch
    import packed_sequence_attention_amd as bd
    docs = [_w2_small()[:6]]
    S = sum(docs[0])
    w, t = H.small_case(260, "bf16", docs, S, 0, S, 8, 2, 256)
    d = H.to_device(w, t)
    full = bd.segment(docs, S, 0, S, device="cuda")
    o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], full)
    dq, _, _ = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], full)
    bounds = [0, S // 3 + 5, (2 * S) // 3 - 7, S]
    for a, b in zip(bounds[:-1], bounds[1:]):
        seg = bd.segment(docs, S, int(a), int(b - a), device="cuda")
        qc = d["q"][:, a:b].contiguous(); doc_ = d["do"][:, a:b].contiguous()
        oc, lc = bd.attn_fwd(qc, d["k"], d["v"], seg)
        assert torch.equal(oc, o[:, a:b]), "O differs from the full call"
        assert torch.equal(lc, lse[:, :, a:b]), "LSE differs from the full call"
        dqc, _, _ = bd.attn_bwd(qc, d["k"], d["v"], oc, lc, doc_, seg)
        assert torch.equal(dqc, dq[:, a:b]), "dQ differs from the full call"


@gpu
def test_determinism():
    import torch
    import packed_sequence_attention_amd as bd
    w = synthetic.workload(2)
    t = synthetic.draw_tensors(w)
    d = H.to_device(w, t)
    seg = bd.segment(w.doc_lens, w.seq_len, 0, w.q_len, device="cuda")
    o1, l1 = bd.attn_fwd(d["q"], d["k"], d["v"], seg)
    o2, l2 = bd.attn_fwd(d["q"], d["k"], d["v"], seg)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = bd.attn_bwd(d["q"], d["k"], d["v"], o1, l1, d["do"], seg)
    g2 = bd.attn_bwd(d["q"], d["k"], d["v"], o1, l1, d["do"], seg)
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])


@gpu
@pytest.mark.parametrize("wid", [2, 3])
def test_launch_order_does_not_change_results(wid):
    """Workloads 2 and 3 meet the condition for the longest-first order of the
    query tiles; overwriting the metadata's visit statistics with values no
    kernel follows ({0, 2^31 - 1}) makes the same calls run in the fixed
    order, and every output is identical bit for bit."""
    import torch
    import packed_sequence_attention_amd as bd
    w = synthetic.workload(wid)
    t = synthetic.draw_tensors(w)
    d = H.to_device(w, t)
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device="cuda")
    _, stats = seg.q_order()
    st = stats.cpu().numpy()
    n_hg, slots = w.h_q // 4, 256 * 2  # the dQ kernel's slots on 256 CUs (the forward has more)
    assert 2 * int(st[0]) * slots >= int(st[1]) * n_hg, "the sorted order is expected to be followed here"
    o1, l1 = bd.attn_fwd(d["q"], d["k"], d["v"], seg)
    g1 = bd.attn_bwd(d["q"], d["k"], d["v"], o1, l1, d["do"], seg)
    stats.copy_(torch.tensor([0, 2**31 - 1], dtype=torch.int32, device=stats.device))
    o2, l2 = bd.attn_fwd(d["q"], d["k"], d["v"], seg)
    g2 = bd.attn_bwd(d["q"], d["k"], d["v"], o2, l2, d["do"], seg)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@gpu
def test_document_independence():
    import torch
    import packed_sequence_attention_amd as bd
    docs = [[300, 257, 500, 91, 400]]
    S = 1548
    w, t = H.small_case(300, "bf16", docs, S, 0, S, 8, 2, 128)
    lo, hi = 300, 557
    t2 = {k: v.copy() for k, v in t.items()}
    rng = np.random.default_rng(1)
    for k in t2:
        t2[k][:, lo:hi] = synthetic.round_bf16(t2[k][:, lo:hi] + rng.standard_normal(t2[k][:, lo:hi].shape,
                                                                                     dtype=np.float32))
    seg = bd.segment(docs, S, 0, S, device="cuda")
    outs = []
    for tt in (t, t2):
        d = H.to_device(w, tt)
        o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], seg)
        dq, dk, dv = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], seg)
        outs.append((o, lse, dk, dv))
    keep = torch.ones(S, dtype=torch.bool); keep[lo:hi] = False
    (o1, l1, k1, v1), (o2, l2, k2, v2) = outs
    assert torch.equal(o1[:, keep], o2[:, keep])
    assert torch.equal(l1[:, :, keep], l2[:, :, keep])
    assert torch.equal(k1[:, keep], k2[:, keep]) and torch.equal(v1[:, keep], v2[:, keep])
    assert not torch.equal(o1[:, lo:hi], o2[:, lo:hi])


@gpu
def test_autograd_wrapper_matches_raw_calls():
    import torch
    import packed_sequence_attention_amd as bd
    docs = [[100, 156]]
    w, t = H.small_case(400, "bf16", docs, 256, 0, 256, 8, 2, 64)
    d = H.to_device(w, t)
    seg = bd.segment(docs, 256, 0, 256, device="cuda")
    q = d["q"].clone().requires_grad_(); k = d["k"].clone().requires_grad_(); v = d["v"].clone().requires_grad_()
    out = bd.attention(q, k, v, seg)
    out.backward(d["do"])
    o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], seg)
    dq, dk, dv = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], seg)
    assert torch.equal(out.detach(), o)
    assert torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
    assert H.rel_fro(q.grad.double().cpu().numpy(), dq.double().cpu().numpy()) < 1e-3


WINDOW_CASES = [
    # (dtype, doc_lens rows, S, cp, rank, h_q, h_kv, d): chunk = rank's rows
    ("bf16", [[40, 200, 120, 152]], 512, 4, 2, 8, 2, 128),
    ("bf16", [[300, 20, 100], [64] * 6 + [36]], 448, 2, 1, 8, 2, 64),      # padding tail in row 0
    ("bf16", [[130, 500, 70, 324]], 1024, 4, 3, 8, 2, 256),
    ("bf16", [[50, 600, 94]], 768, 8, 6, 4, 2, 96),                         # generic kernels (d = 96)
    ("f32", [[90, 230, 64, 128]], 512, 2, 1, 4, 4, 64),                     # generic kernels (float32)
    ("bf16", [[1000, 24]], 1024, 4, 3, 8, 1, 128),                          # all-to-all-v: halo from 3 ranks
]


def _window_inputs(t_full, plan, S):
    """The K / V a rank holds after the needed-only exchange: its window
    [kv_begin, kv_end) of every row, filled from the plan's receive ranges
    and its own chunk, zeros elsewhere."""
    kb, ke = plan.kv_begin, plan.kv_end
    C = S // plan.cp
    r0 = plan.rank * C
    out = {}
    for name in ("k", "v"):
        full = t_full[name]
        win = np.zeros((full.shape[0], ke - kb) + full.shape[2:], full.dtype)
        win[:, r0 - kb:ke - kb] = full[:, r0:ke]
        for (row, _peer, a, e) in plan.recv:
            win[row, a - kb:e - kb] = full[row, a:e]
        out[name] = win
    return out


def _run_window(w, t, plan=None):
    """Whole-row call and window-only call on the same chunk."""
    import torch
    import packed_sequence_attention_amd as bd
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device="cuda")
    d = H.to_device(w, t)
    o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], seg, w.scale)
    dq, dk, dv = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], seg, w.scale)
    tw = _window_inputs(t, plan, w.seq_len)
    dw = H.to_device(w, tw)
    ow, lw = bd.attn_fwd(d["q"], dw["k"], dw["v"], seg, w.scale, kv_begin=plan.kv_begin)
    dqw, dkw, dvw = bd.attn_bwd(d["q"], dw["k"], dw["v"], ow, lw, d["do"], seg, w.scale, kv_begin=plan.kv_begin)
    torch.cuda.synchronize()
    return (o, lse, dq, dk, dv), (ow, lw, dqw, dkw, dvw)


@gpu
@pytest.mark.parametrize("case", range(len(WINDOW_CASES) + 1))
def test_window_only_kv_is_bitwise_whole_row(case):
    """The needed-only exchange (Automodel page, Summary and Design overview,
    exchange.py): a rank that holds only its plan's K/V window -- received
    halo ranges, its own chunk, zeros elsewhere -- gets bit for bit the O,
    LSE and dQ of the whole-row call, and dK / dV equal to the whole-row
    call's on the window, which is zero outside it.  The last case is the
    S = 16384 workload's straddling chunk (rank 2 of 4) at full size."""
    import torch
    import packed_sequence_attention_amd as bd
    if case < len(WINDOW_CASES):
        dtype, docs, S, cp, rank, hq, hkv, d = WINDOW_CASES[case]
        C = S // cp
        w, t = H.small_case(600 + case, dtype, docs, S, rank * C, C, hq, hkv, d)
        t_full = t
    else:
        w = synthetic.workload(3)
        cp, rank = 4, 2
        t_full = synthetic.draw_tensors(w)
        t = t_full
    plan = bd.kv_plan(w.doc_lens, w.seq_len, cp, rank)
    print(f"window case {case}: {w.dtype} S={w.seq_len} cp={cp} rank={rank} d={w.head_dim} "
          f"window=[{plan.kv_begin},{plan.kv_end}) mode={plan.rank_mode}/{plan.step_mode}", flush=True)
    full, win = _run_window(w, t_full, plan)
    kb, ke = plan.kv_begin, plan.kv_end
    for name, a, b in (("o", full[0], win[0]), ("lse", full[1], win[1]), ("dq", full[2], win[2]),
                       ("dk", full[3][:, kb:ke], win[3]), ("dv", full[4][:, kb:ke], win[4])):
        assert torch.equal(a, b), f"{name} differs with window-only K/V"
    assert not full[3][:, :kb].any() and not full[3][:, ke:].any()
    assert not full[4][:, :kb].any() and not full[4][:, ke:].any()
    if case == len(WINDOW_CASES) - 1:
        assert plan.rank_mode == 2  # the 1000-token document spans all four ranks


@gpu
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (8, 4, 64), (6, 2, 128)])
def test_chunk_concatenation_any_gqa_ratio(hq, hkv, d):
    """Query heads from groups of 1, 2 or 3: workgroups of the matrix-core
    forward and dQ kernels take several query tiles and visit the union of
    their key ranges; a row's result still depends only on its own tiles, so
    chunks concatenate bit for bit (O, LSE, dQ) and dK / dV sum to the full
    call's within tolerance."""
    import torch
    import packed_sequence_attention_amd as bd
    docs = [_w2_small()]
    S, cp = 2048, 4
    w, t = H.small_case(250 + hq + d, "bf16", docs, S, 0, S, hq, hkv, d)
    dd = H.to_device(w, t)
    full = H.tile_path(bd.segment(docs, S, 0, S, device="cuda"))
    o, lse = bd.attn_fwd(dd["q"], dd["k"], dd["v"], full)
    dq, dk, dv = bd.attn_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], full)
    dk_sum = torch.zeros_like(dk, dtype=torch.float32)
    bounds = [0, 500, 1100, 1600, 2048]   # uneven chunks, not multiples of 32
    for a, b in zip(bounds[:-1], bounds[1:]):
        seg = H.tile_path(bd.segment(docs, S, a, b - a, device="cuda"))
        qc, doc_ = dd["q"][:, a:b].contiguous(), dd["do"][:, a:b].contiguous()
        oc, lc = bd.attn_fwd(qc, dd["k"], dd["v"], seg)
        assert torch.equal(oc, o[:, a:b]) and torch.equal(lc, lse[:, :, a:b])
        dqc, dkc, _dvc = bd.attn_bwd(qc, dd["k"], dd["v"], oc, lc, doc_, seg)
        assert torch.equal(dqc, dq[:, a:b])
        dk_sum += dkc.float()
    torch.cuda.synchronize()
    rel = float((dk_sum - dk.float()).norm() / dk.float().norm())
    assert rel <= 1e-2, rel
