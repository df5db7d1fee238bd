"""The short-document backward (every segment at most 128 keys: one kernel
computes dQ, dK and dV over the metadata's bins of whole documents), through
the C ABI:

* the bins the metadata build writes are bit-exact against the greedy walk
  of the host table (none when a segment has more than 128 keys);
* parity with the oracle (Automodel page, Proof: forward/backward parity)
  on packings of short documents: padding tails, chunks that start inside a
  document, B = 2, head_dim 64 and 128, GQA groups of 1, 2, 3, 4 and 8,
  documents of exactly 128 tokens and of one token, attention dropout; the
  worst per-document gradient error is gated as well;
* against the tile kernels on the same inputs (within the tolerance: the
  two sum in different orders), and bitwise replay and window-only K/V;
* chunks: O and LSE concatenate bit for bit (the forward is unchanged), dQ
  within tolerance of the full call, dK / dV sum to it."""
import sys

import numpy as np
import pytest

import synthetic
from tests import helpers as H

gpu = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _short(seed, S, fill=None, lo=16, hi=128):
    rng = np.random.default_rng(seed)
    fill = S if fill is None else fill
    lens, tot = [], 0
    while tot < fill:
        Ln = int(min(rng.integers(lo, hi + 1), fill - tot))
        lens.append(Ln)
        tot += Ln
    return lens


BIN_LAYOUTS = [
    # (doc_lens rows, S, row_offset, q_len)
    ([_short(1, 2048)], 2048, 0, 2048),
    ([_short(2, 2048)], 2048, 700, 900),                          # starts inside a document
    ([_short(3, 1024, fill=900), _short(4, 1024)], 1024, 0, 1024),  # padding tail, B = 2
    ([[128] * 8, [1] * 300 + [64] * 4], 1024, 0, 1024),          # exactly 128; many 1-token docs
    ([_short(5, 4096, lo=1, hi=8)], 4096, 1000, 3000),             # tiny documents
    ([[64, 129, 64]], 257, 0, 257),                                # one document of 129: no bins
    ([_short(6, 2048)], 2048, 1900, 148),
]


@gpu
@pytest.mark.parametrize("i", range(len(BIN_LAYOUTS)))
def test_bins_match_greedy_walk(i):
    import packed_sequence_attention_amd as bd
    rows, S, a, L = BIN_LAYOUTS[i]
    for inline in (True, False):
        seg = bd.segment(rows, S, a, L)
        if inline and seg.n_seg > bd.load_library().blockdiag_meta_inline_max_seg():
            continue
        seg = seg.to("cuda", inline=inline)
        ref = H.greedy_bins(seg)
        got = H.device_bins(seg)
        _log(f"bins layout {i} inline={inline}: {len(got)} bins, max_seg_k {seg.desc.max_seg_k}")
        assert got == (ref or []), (got[:5], (ref or [])[:5])
        assert (seg.desc.max_seg_k <= 128) == (ref is not None)


PARITY = [
    # (doc_lens rows, S, row_offset, q_len, h_q, h_kv, d, dropout p)
    ([_short(11, 2048, fill=1900), _short(12, 2048)], 2048, 0, 2048, 32, 8, 128, 0.0),
    ([_short(13, 3000)], 3000, 1111, 1200, 16, 4, 128, 0.0),
    ([_short(14, 1500)], 1500, 0, 1500, 16, 4, 64, 0.0),
    ([_short(15, 1200)], 1200, 37, 1100, 8, 8, 128, 0.0),        # multi-head
    ([_short(16, 1000)], 1000, 0, 1000, 6, 2, 64, 0.0),           # groups of 3
    ([[128] * 6 + [1] * 50 + [77, 128]], 1024, 0, 1024, 8, 4, 128, 0.0),
    ([_short(17, 2000, lo=1, hi=12)], 2000, 300, 1500, 16, 2, 128, 0.0),  # groups of 8
    ([_short(18, 1500, fill=1400)], 1500, 5, 1450, 8, 2, 128, 0.2),      # dropout
    ([_short(19, 1000)], 1000, 0, 1000, 8, 2, 64, 0.1),
]


@gpu
@pytest.mark.parametrize("i", range(len(PARITY)))
def test_short_document_parity(i):
    rows, S, r0, L, hq, hkv, d, p = PARITY[i]
    w, t = H.small_case(1500 + i, "bf16", rows, S, r0, L, hq, hkv, d)
    _log(f"short-document case {i}: S={S} r0={r0} L={L} H={hq}/{hkv} d={d} p={p} docs={len(rows[0])}")
    import torch
    import packed_sequence_attention_amd as bd
    seg = bd.segment(w.doc_lens, S, r0, L, device="cuda")
    assert 0 <= seg.desc.max_seg_k <= 128 and len(H.device_bins(seg)) > 0
    drop = (p, 0xC0FFEE + i, 5) if p > 0 else None
    dd = H.to_device(w, t)
    o, lse = bd.attn_fwd(dd["q"], dd["k"], dd["v"], seg, w.scale, dropout=drop)
    dq, dk, dv = bd.attn_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], seg, w.scale, dropout=drop)
    torch.cuda.synchronize()
    g = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    g = {k_: v_.double().cpu().numpy() for k_, v_ in g.items()}
    ref = H.oracle(w, t, block_rows=None, dropout=drop)
    grads = ("dq", "dk", "dv")
    errs = H.check(w, {k_: g[k_] for k_ in grads}, {k_: ref[k_] for k_ in grads})
    worst = H.per_doc_grad_errors(w, g, ref)
    _log("  errors", {k_: f"{v_:.3g}" for k_, v_ in errs.items()}, "worst per document",
         {k_: f"{v_:.3g}" for k_, v_ in worst.items()})
    for name, e in worst.items():
        assert e <= H.TOL["bf16"]["grad_rel_fro"], name


@gpu
def test_short_documents_against_tile_kernels_replay_and_window():
    import torch
    import packed_sequence_attention_amd as bd
    rows = [_short(31, 2048, fill=2000), _short(32, 2048)]
    S, r0, L = 2048, 640, 1200
    w, t = H.small_case(1600, "bf16", rows, S, r0, L, 16, 4, 128)
    dd = H.to_device(w, t)
    seg = bd.segment(rows, S, r0, L, device="cuda")
    o, lse = bd.attn_fwd(dd["q"], dd["k"], dd["v"], seg)
    g1 = bd.attn_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], seg)
    g2 = bd.attn_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], seg)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b), "replay differs"
    # the needed-only K/V window gives the same bits
    kb = (int(seg.desc.kv_lo) // 64) * 64
    kw, vw = dd["k"][:, kb:r0 + L].contiguous(), dd["v"][:, kb:r0 + L].contiguous()
    gw = bd.attn_bwd(dd["q"], kw, vw, o, lse, dd["do"], seg, kv_begin=kb)
    assert torch.equal(gw[0], g1[0])
    assert torch.equal(gw[1], g1[1][:, kb:r0 + L]) and torch.equal(gw[2], g1[2][:, kb:r0 + L])
    # the tile kernels on the same inputs: equal within the tolerance
    seg_t = H.tile_path(bd.segment(rows, S, r0, L, device="cuda"))
    gt = bd.attn_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], seg_t)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g1, gt):
        rel = H.rel_fro(a.double().cpu().numpy(), b.double().cpu().numpy())
        _log(f"  short vs tile kernels {name}: {rel:.3g}")
        assert rel <= 1e-2, name
    assert not g1[1][:, r0 + L:].any() and not g1[2][:, r0 + L:].any()


@gpu
def test_short_documents_chunks():
    import torch
    import packed_sequence_attention_amd as bd
    rows = [_short(41, 2048)]
    S = 2048
    w, t = H.small_case(1700, "bf16", rows, S, 0, S, 8, 2, 128)
    dd = H.to_device(w, t)
    full = bd.segment(rows, S, 0, S, device="cuda")
    o, lse = bd.attn_fwd(dd["q"], dd["k"], dd["v"], full)
    dq, dk, dv = bd.attn_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], full)
    dk_sum = torch.zeros_like(dk, dtype=torch.float32)
    dv_sum = torch.zeros_like(dv, dtype=torch.float32)
    bounds = [0, 333, 1000, 1500, 2048]
    for a, b in zip(bounds[:-1], bounds[1:]):
        seg = bd.segment(rows, S, a, b - a, device="cuda")
        qc, doc_ = dd["q"][:, a:b].contiguous(), dd["do"][:, a:b].contiguous()
        oc, lc = bd.attn_fwd(qc, dd["k"], dd["v"], seg)
        assert torch.equal(oc, o[:, a:b]) and torch.equal(lc, lse[:, :, a:b])
        dqc, dkc, dvc = bd.attn_bwd(qc, dd["k"], dd["v"], oc, lc, doc_, seg)
        rel = H.rel_fro(dqc.double().cpu().numpy(), dq[:, a:b].double().cpu().numpy())
        assert rel <= 1e-2, rel
        dk_sum += dkc.float()
        dv_sum += dvc.float()
    torch.cuda.synchronize()
    assert H.rel_fro(dk_sum.double().cpu().numpy(), dk.double().cpu().numpy()) < 1e-2
    assert H.rel_fro(dv_sum.double().cpu().numpy(), dv.double().cpu().numpy()) < 1e-2
