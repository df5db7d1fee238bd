"""Shared helpers of the GPU parity tests: seeded inputs, calls through the
C ABI (Python binding), the oracle and the tolerance checks.

Tolerances (float32 workloads / bfloat16 workloads):
  O:            max-abs <= 1e-5 / 2e-2 (bf16 O: float32 accumulation, output
                rounded to nearest even)
  LSE:          max-abs <= 1e-5 / 2e-2
  dQ, dK, dV:   max-abs <= 1e-4 / relative Frobenius norm <= 5e-2 per tensor
Segment tables and per-row / per-key bounds: bit-exact.
"""
from __future__ import annotations

import numpy as np

import synthetic

TOL = {
    "f32": {"o": 1e-5, "lse": 1e-5, "grad_abs": 1e-4},
    "bf16": {"o": 2e-2, "lse": 2e-2, "grad_rel_fro": 5e-2},
}


def torch_dtype(w):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def to_device(w, arrays, device="cuda"):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=torch_dtype(w))
            for k, a in arrays.items()}


def run_gpu(w, t, device="cuda", want_bwd=True):
    """Runs the library on workload w with numpy inputs t; returns float64
    numpy outputs."""
    import torch
    import packed_sequence_attention_amd as bd
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device=device)
    d = to_device(w, t, device)
    o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], seg, w.scale)
    out = {"o": o, "lse": lse}
    if want_bwd:
        dq, dk, dv = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], seg, w.scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in out.items()}


def oracle(w, t, rows=None, want=("fwd", "bwd"), block_rows=256, dropout=None):
    from oracle import parallel
    return parallel.run(t["q"], t["k"], t["v"], t.get("do"), w.doc_lens, w.row_offset, w.scale,
                        block_rows=block_rows, rows=rows, want=want, dropout=dropout)


def lse_diff(a, b):
    """max |a - b| over finite entries; the -inf pattern must agree."""
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb), "LSE -inf pattern differs"
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    return float(np.abs(a[fa] - b[fb]).max(initial=0.0))


def rel_fro(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def check(w, gpu, ref, rows=None, keys=None, report=None):
    """Assert the tolerances; ``rows`` / ``keys`` restrict the comparison
    (local query rows / key positions) for sampled checks.  Returns the
    observed errors."""
    tol = TOL[w.dtype]
    sel_r = slice(None) if rows is None else np.asarray(rows)
    sel_k = slice(None) if keys is None else np.asarray(keys)
    errs = {}
    if "o" in ref:
        errs["o"] = float(np.abs(gpu["o"][:, sel_r] - ref["o"][:, sel_r]).max(initial=0.0))
        errs["lse"] = lse_diff(gpu["lse"][:, :, sel_r], ref["lse"][:, :, sel_r])
    if "dq" in ref:
        pairs = (("dq", gpu["dq"][:, sel_r], ref["dq"][:, sel_r]), ("dk", gpu["dk"][:, sel_k], ref["dk"][:, sel_k]),
                 ("dv", gpu["dv"][:, sel_k], ref["dv"][:, sel_k]))
        for name, x, r in pairs:
            if w.dtype == "f32":
                errs[name] = float(np.abs(x - r).max(initial=0.0))
            else:
                errs[name] = rel_fro(x, r)
    if report is not None:
        report.update(errs)
    if "o" in errs:
        assert errs["o"] <= tol["o"], f"O max-abs {errs['o']:.3g} > {tol['o']}"
        assert errs["lse"] <= tol["lse"], f"LSE max-abs {errs['lse']:.3g} > {tol['lse']}"
    for name in ("dq", "dk", "dv"):
        if name in errs:
            lim = tol["grad_abs"] if w.dtype == "f32" else tol["grad_rel_fro"]
            assert errs[name] <= lim, f"{name} error {errs[name]:.3g} > {lim}"
    return errs


def small_case(i, dtype, doc_lens, seq_len, row_offset, q_len, h_q, h_kv, d, scale=None):
    w = synthetic.custom_workload(1000 + i, dtype, doc_lens, seq_len, row_offset, q_len, h_q, h_kv, d,
                                  scale, name=f"case{i}")
    return w, synthetic.draw_tensors(w)


def per_doc_grad_errors(w, gpu, ref, heads=None, kv_heads=None):
    """Worst per-document relative Frobenius error of dQ (the document's rows
    in the chunk, all query heads) and of dK, dV (the document's keys that
    the chunk attends, all K/V heads), over every batch row and document: an
    error confined to a few short documents is not diluted by the others.
    Keys no chunk row attends must be exactly zero.  ``heads`` / ``kv_heads``
    select the head slices the arrays hold (default: all)."""
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    r0, r1 = w.row_offset, w.row_offset + w.q_len
    for b, lens in enumerate(w.doc_lens):
        for name in ("dk", "dv"):  # keys after the chunk's last row: never attended
            assert not np.any(gpu[name][b, r1:]), f"{name} nonzero at keys past the chunk"
        pos = 0
        for Ln in lens:
            s, e = pos, pos + Ln
            pos = e
            if Ln == 0:
                continue
            qa, qb = max(s, r0) - r0, min(e, r1) - r0
            if qb <= qa:  # no row of the chunk in this document: its keys are unattended
                for name in ("dk", "dv"):
                    assert not np.any(gpu[name][b, s:e]), f"{name} nonzero at unattended keys [{s},{e})"
                continue
            for name, x, r in (("dq", gpu["dq"][b, qa:qb], ref["dq"][b, qa:qb]),
                               ("dk", gpu["dk"][b, s:min(e, r1)], ref["dk"][b, s:min(e, r1)]),
                               ("dv", gpu["dv"][b, s:min(e, r1)], ref["dv"][b, s:min(e, r1)])):
                den = np.linalg.norm(r)
                if den > 0:
                    worst[name] = max(worst[name], float(np.linalg.norm(x - r) / den))
    return worst


def tile_path(seg):
    """Makes the backward of this segment table take the tile kernels (dQ
    pass, then dK/dV pass) even when every segment is short: the descriptor
    then says the longest segment is unknown.  Returns seg."""
    seg.desc.max_seg_k = -1
    return seg


def greedy_bins(seg, cap=128):
    """The short-document bins of a host segment table, walked in order
    (documents of one batch row grouped while their keys span at most cap
    positions; padding and a new batch row start a new bin): a list of
    (first row, end row, first key) or None when a segment has more than cap
    keys.  Written from the bins' definition in include/blockdiag.h."""
    out, cur = [], None
    for s in range(seg.n_seg):
        q0, q1 = int(seg.cu_q[s]), int(seg.cu_q[s + 1])
        kn = int(seg.cu_k[s + 1] - seg.cu_k[s])
        k0 = int(seg.k_begin[s])
        if kn == 0:
            if cur is not None:
                out.append(tuple(cur))
            cur = None
            continue
        if kn > cap:
            return None
        if cur is not None and q0 // seg.q_len == cur[0] // seg.q_len and k0 + kn - cur[2] <= cap:
            cur[1] = q1
            continue
        if cur is not None:
            out.append(tuple(cur))
        cur = [q0, q1, k0]
    if cur is not None:
        out.append(tuple(cur))
    return out


def device_bins(seg):
    """The bins the metadata build wrote (the section after the bounds and
    the query-tile order), as a list of (first row, end row, first key)."""
    m = seg.meta.cpu().numpy()
    B, S, L = seg.batch, seg.seq_len, seg.q_len
    off = 2 * B * L + 2 * B * S
    nq = B * ((L + 31) // 32)
    if 1 <= nq <= 8192:
        off += nq + 2
    n = int(m[off])
    return [tuple(int(x) for x in m[off + 1 + 3 * i: off + 4 + 3 * i]) for i in range(n)]
