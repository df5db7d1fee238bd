"""Attention dropout on the GPU (Automodel page, Proof: the varlen path
forwards a dropout probability and the native kernel applies it), through
the C ABI:

* parity with the oracle drawing the same stated mask (Philox4x32-10 over
  the (key / 4, row / 4, b * h_q + h, offset) counter) at p = 0.1 and 0.3,
  on the matrix-core kernels (head_dim 64 / 128 / 256) and the generic ones
  (float32, head_dim 96), with chunks whose row_offset is not a multiple of
  4, padding tails, and the S = 4096 x 2 workload at full size; the same
  outputs without dropout are far outside the tolerance (the mask matters);
* a replayed forward and backward are bitwise identical;
* masks follow row positions: chunks concatenate bit for bit, and
  window-only K/V give the whole-row bits;
* p = 0 is bitwise the call without dropout."""
import sys

import numpy as np
import pytest

import synthetic
from tests import helpers as H

gpu = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _gpu(w, t, dropout, kv=None):
    import torch
    import packed_sequence_attention_amd as bd
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device="cuda")
    d = H.to_device(w, t)
    o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], seg, w.scale, dropout=dropout)
    dq, dk, dv = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], seg, w.scale, dropout=dropout)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _np(out):
    return {k: v.double().cpu().numpy() for k, v in out.items()}


def _check_dropout(w, g, ref, t, p):
    """The tolerances of the undropped path, except bf16 O: the fixed bf16
    bound is stated for the undropped output only, so here it is derived per element from the
    arithmetic -- the output's round-to-nearest (at most 2^-8 |O| for bf16)
    plus the bf16 rounding of the kept weights P * c that multiply V (at most
    2^-9 c max|v| summed over a row), plus 1e-3 for the float32 sums.  The
    scale c = 1 / (1 - p) raises |O|, so the fixed 2e-2 of the undropped path
    does not carry over."""
    if w.dtype != "bf16":
        return H.check(w, g, ref)
    from oracle import dropout as DR
    c = DR.keep_scale(p)[1]
    bound = 2.0 ** -8 * np.abs(ref["o"]) + 2.0 ** -9 * c * np.abs(t["v"]).max() + 1e-3
    err = np.abs(g["o"] - ref["o"])
    assert np.all(err <= bound), f"O error {err.max():.3g} above the derived bound"
    errs = {"o": float(err.max()), "o_share_of_bound": float((err / bound).max())}
    errs["lse"] = H.lse_diff(g["lse"], ref["lse"])
    assert errs["lse"] <= H.TOL["bf16"]["lse"], errs["lse"]
    grads = ("dq", "dk", "dv")
    errs.update(H.check(w, {k: g[k] for k in grads}, {k: ref[k] for k in grads}))
    return errs


CASES = [
    # (dtype, doc_lens rows, S, row_offset, q_len, h_q, h_kv, d, p)
    ("bf16", [[200, 37, 150, 125], [512]], 512, 0, 512, 8, 2, 128, 0.1),
    ("bf16", [[300, 250, 90]], 700, 101, 503, 8, 2, 64, 0.3),          # row_offset % 4 = 1, padding tail
    ("bf16", [[130, 400, 90]], 640, 34, 400, 8, 2, 256, 0.1),           # head_dim 256, row_offset % 4 = 2
    ("f32", [[90, 170, 60]], 320, 3, 300, 4, 2, 64, 0.3),              # generic kernels, float32
    ("bf16", [[70, 120, 66]], 256, 0, 256, 4, 4, 96, 0.1),             # generic kernels, bf16
]


@gpu
@pytest.mark.parametrize("i", range(len(CASES)))
def test_dropout_parity_with_oracle(i):
    dtype, docs, S, r0, L, hq, hkv, d, p = CASES[i]
    w, t = H.small_case(800 + i, dtype, docs, S, r0, L, hq, hkv, d)
    seed, offset = 0x1234_5678_9ABC_DEF0 + i, 17 + i
    _log(f"dropout case {i}: {dtype} S={S} r0={r0} L={L} H={hq}/{hkv} d={d} p={p}")
    g = _np(_gpu(w, t, (p, seed, offset)))
    ref = H.oracle(w, t, block_rows=None, dropout=(p, seed, offset))
    errs = _check_dropout(w, g, ref, t, p)
    _log("  errors", {k: f"{v:.3g}" for k, v in errs.items()})
    # the mask matters: against the undropped oracle O is far off
    ref0 = H.oracle(w, t, block_rows=None, want=("fwd",))
    assert np.abs(g["o"] - ref0["o"]).max() > 20 * H.TOL[w.dtype]["o"]


@gpu
def test_dropout_parity_workload2_full_size():
    w = synthetic.workload(2)
    t = synthetic.draw_tensors(w)
    drop = (0.1, 20241203, 7)
    _log("dropout workload 2: gpu ...")
    g = _np(_gpu(w, t, drop))
    _log("  oracle ...")
    ref = H.oracle(w, t, block_rows=256, dropout=drop)
    errs = _check_dropout(w, g, ref, t, drop[0])
    worst = H.per_doc_grad_errors(w, g, ref)
    _log("  errors", {k: f"{v:.3g}" for k, v in errs.items()}, "worst per document",
         {k: f"{v:.3g}" for k, v in worst.items()})
    for name, e in worst.items():
        assert e <= H.TOL["bf16"]["grad_rel_fro"], name


@gpu
def test_dropout_replay_chunks_window_and_zero_probability():
    import torch
    import packed_sequence_attention_amd as bd
    docs = [[300, 500, 120, 104], [1024]]
    S, cp = 1024, 4
    w, t = H.small_case(900, "bf16", docs, S, 0, S, 8, 2, 128)
    drop = (0.2, 99, 3)
    a = _gpu(w, t, drop)
    b = _gpu(w, t, drop)
    for name in a:
        assert torch.equal(a[name], b[name]), f"{name}: replay differs"
    # p = 0 through the struct is the call without dropout
    z0 = _gpu(w, t, (0.0, 99, 3))
    n0 = _gpu(w, t, None)
    for name in z0:
        assert torch.equal(z0[name], n0[name]), f"{name}: p = 0 differs from no dropout"
    # chunks (and each chunk on its needed-only K/V window) reproduce the full call's rows
    d = H.to_device(w, t)
    C = S // cp
    for r in range(cp):
        r0 = r * C
        seg = bd.segment(docs, S, r0, C, device="cuda")
        qc, doc_ = d["q"][:, r0:r0 + C].contiguous(), d["do"][:, r0:r0 + C].contiguous()
        oc, lc = bd.attn_fwd(qc, d["k"], d["v"], seg, w.scale, dropout=drop)
        dqc, _dk, _dv = bd.attn_bwd(qc, d["k"], d["v"], oc, lc, doc_, seg, w.scale, dropout=drop)
        assert torch.equal(oc, a["o"][:, r0:r0 + C]) and torch.equal(lc, a["lse"][:, :, r0:r0 + C])
        assert torch.equal(dqc, a["dq"][:, r0:r0 + C])
        plan = bd.kv_plan(docs, S, cp, r)
        kb = plan.kv_begin
        kw, vw = d["k"][:, kb:r0 + C].contiguous(), d["v"][:, kb:r0 + C].contiguous()
        ow, lw = bd.attn_fwd(qc, kw, vw, seg, w.scale, kv_begin=kb, dropout=drop)
        dqw, dkw, dvw = bd.attn_bwd(qc, kw, vw, ow, lw, doc_, seg, w.scale, kv_begin=kb, dropout=drop)
        assert torch.equal(ow, oc) and torch.equal(dqw, dqc)
        assert torch.equal(dkw, _dk[:, kb:r0 + C]) and torch.equal(dvw, _dv[:, kb:r0 + C])
    torch.cuda.synchronize()
