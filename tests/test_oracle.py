"""Pins of the fp64 oracle against values independent of its own code.

Each test names what it pins.  Sources: Automodel page "feat(distributed):
block-diagonal varlen CP for packed sequences" -- Summary/Motivation (dense
masked SDPA is the plain definition; block-causal per document, exact parity
with the non-CP mask), Design overview (kernels.py: [B,1,L,S] mask; batch.py:
contiguous chunk; exchange.py: K/V gradients are summed back over ranks) and
key properties 1-2 (per-rank outputs concatenated over ranks equal the full
attention; straddling documents are bottom-right aligned).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as A
from oracle import brute
from oracle import segment as SEG

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layout(rng, B, S, allow_pad=True):
    rows = []
    for _ in range(B):
        lens, total = [], 0
        fill = S if (not allow_pad or rng.random() < 0.5) else int(rng.integers(1, S + 1))
        while total < fill:
            L = int(rng.integers(1, max(2, S // 2) + 1))
            L = min(L, fill - total)
            lens.append(L)
            total += L
        rows.append(tuple(lens))
    return tuple(rows)


def rand_case(seed, B=None, S=None, Hq=None, Hkv=None, d=None, allow_pad=True):
    rng = np.random.default_rng(seed)
    B = B or int(rng.integers(1, 3))
    S = S or int(rng.integers(2, 17))
    Hkv = Hkv or int(rng.choice([1, 2]))
    Hq = Hq or Hkv * int(rng.choice([1, 2]))
    d = d or int(rng.integers(1, 5))
    layout = rand_layout(rng, B, S, allow_pad)
    q = rng.standard_normal((B, S, Hq, d))
    k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d))
    do = rng.standard_normal((B, S, Hq, d))
    return layout, S, q, k, v, do, float(rng.uniform(0.3, 1.5))


# ---------------------------------------------------------------- hand-worked


def test_hand_example_forward_backward():
    """Pin: values worked by hand (tests/golden/hand_example.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    S = g["seq_len"]
    q = np.array(g["q"]).reshape(1, S, 1, 1)
    k = np.array(g["k"]).reshape(1, S, 1, 1)
    v = np.array(g["v"]).reshape(1, S, 1, 1)
    do = np.array(g["do"]).reshape(1, S, 1, 1)
    for key, r0, L in (("full", 0, S), ("chunk_row_offset_2", 2, 1)):
        exp = g[key]
        o, lse = A.forward(q[:, r0:r0 + L], k, v, g["doc_lens"], r0, g["scale"])
        dq, dk, dv = A.backward(q[:, r0:r0 + L], k, v, do[:, r0:r0 + L], g["doc_lens"], r0, g["scale"])
        np.testing.assert_allclose(o.ravel(), exp["o"], atol=1e-14)
        np.testing.assert_allclose(lse.ravel(), exp["lse"], atol=1e-14)
        np.testing.assert_allclose(dq.ravel(), exp["dq"], atol=1e-14)
        np.testing.assert_allclose(dk.ravel(), exp["dk"], atol=1e-14)
        np.testing.assert_allclose(dv.ravel(), exp["dv"], atol=1e-14)


def test_segment_ref_hand_tables():
    """Pin: segment tables worked by hand (tests/golden/segments_hand.json)."""
    g = json.load(open(os.path.join(GOLDEN, "segments_hand.json")))
    for c in g["cases"]:
        t = SEG.segment_ref(c["doc_lens"], c["seq_len"], c["row_offset"], c["q_len"])
        assert t["cu_q"] == c["cu_q"]
        assert t["cu_k"] == c["cu_k"]
        assert t["k_begin"] == c["k_begin"]
        assert (t["max_q"], t["max_k"]) == (c["max_q"], c["max_k"])


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_all_chunkings(seed):
    """Pin: pure-Python scalar loops (per-pair document-id mask, delta-route
    backward) on tiny inputs, every contiguous chunk [r0, r0+L)."""
    layout, S, q, k, v, do, scale = rand_case(seed)
    rng = np.random.default_rng(1000 + seed)
    chunks = [(0, S)] + [tuple(sorted(rng.integers(0, S + 1, 2))) for _ in range(2)]
    for a, b in chunks:
        L = b - a
        qc, doc_ = q[:, a:b], do[:, a:b]
        o, lse = A.forward(qc, k, v, layout, a, scale)
        if L == 0:  # empty chunk: nothing to compute
            assert o.size == 0 and lse.size == 0
            continue
        ob, lseb = brute.forward(qc.tolist(), k.tolist(), v.tolist(), layout, a, scale)
        np.testing.assert_allclose(o, np.array(ob).reshape(o.shape), atol=1e-12)
        np.testing.assert_allclose(lse, np.array(lseb).reshape(lse.shape), atol=1e-12)
        dq, dk, dv = A.backward(qc, k, v, doc_, layout, a, scale)
        dqb, dkb, dvb = brute.backward(qc.tolist(), k.tolist(), v.tolist(), doc_.tolist(), layout, a, scale)
        np.testing.assert_allclose(dq, np.array(dqb), atol=1e-12)
        np.testing.assert_allclose(dk, np.array(dkb), atol=1e-12)
        np.testing.assert_allclose(dv, np.array(dvb), atol=1e-12)


# ---------------------------------------------------------------- library special cases


def _torch_sdpa(q, k, v, do, layout, r0, scale):
    """fp64 CPU torch SDPA with an explicit boolean [B,1,L,S] mask built from
    document ids; GQA by repeating K/V heads; gradients by torch autograd."""
    B, L, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    mask = torch.zeros(B, 1, L, S, dtype=torch.bool)
    for b, lens in enumerate(layout):
        ids = torch.full((S,), -1)
        pos = 0
        for di, Ln in enumerate(lens):
            ids[pos:pos + Ln] = di
            pos += Ln
        for t in range(L):
            i = r0 + t
            if ids[i] >= 0:
                mask[b, 0, t] = (ids == ids[i]) & (torch.arange(S) <= i)
    tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    tk = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_()
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), attn_mask=mask, scale=scale)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    return (out.detach().permute(0, 2, 1, 3).numpy(), tq.grad.permute(0, 2, 1, 3).numpy(),
            tk.grad.permute(0, 2, 1, 3).numpy(), tv.grad.permute(0, 2, 1, 3).numpy())


@pytest.mark.parametrize("seed", range(6))
def test_matches_torch_sdpa_multi_doc(seed):
    """Pin: torch.nn.functional.scaled_dot_product_attention (fp64, CPU) with
    a boolean [B,1,L,S] mask, multi-document rows, GQA, chunks; autograd
    gradients.  No padding rows (torch gives NaN on an all-masked row)."""
    rng = np.random.default_rng(50 + seed)
    S = int(rng.integers(8, 40))
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([3, 8]))
    layout = rand_layout(rng, 2, S, allow_pad=False)
    q = rng.standard_normal((2, S, Hq, d)); k = rng.standard_normal((2, S, Hkv, d))
    v = rng.standard_normal((2, S, Hkv, d)); do = rng.standard_normal((2, S, Hq, d))
    a = int(rng.integers(0, S // 2)); b = int(rng.integers(a + 1, S + 1))
    scale = 0.7
    o, lse = A.forward(q[:, a:b], k, v, layout, a, scale)
    dq, dk, dv = A.backward(q[:, a:b], k, v, do[:, a:b], layout, a, scale)
    to, tdq, tdk, tdv = _torch_sdpa(q[:, a:b], k, v, do[:, a:b], layout, a, scale)
    for x, y in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        np.testing.assert_allclose(x, y, atol=1e-12)


def test_single_document_is_causal_attention():
    """Pin: one document spanning the row is ordinary causal attention
    (torch SDPA is_causal=True, no mask built), incl. the LSE via logsumexp."""
    rng = np.random.default_rng(7)
    B, S, Hq, Hkv, d = 1, 33, 4, 2, 16
    q = rng.standard_normal((B, S, Hq, d)); k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d)); do = rng.standard_normal((B, S, Hq, d))
    scale = 1 / math.sqrt(d)
    o, lse = A.forward(q, k, v, [[S]], 0, scale)
    dq, dk, dv = A.backward(q, k, v, do, [[S]], 0, scale)
    tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    tk = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_()
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(2, 1), tv.repeat_interleave(2, 1), is_causal=True, scale=scale)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    np.testing.assert_allclose(o, out.detach().permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    logits = scale * torch.einsum("bhid,bhjd->bhij", tq.detach(), tk.detach().repeat_interleave(2, 1))
    logits = logits.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), atol=1e-12)


# ---------------------------------------------------------------- closed forms


def test_closed_forms():
    """Pin: closed forms of the definition.
    * the first token of each document attends only itself: O = v, LSE =
      scale q.k, dQ = 0;
    * Q = 0: O_i is the mean of v over the document prefix and LSE_i the log
      of its length;
    * K -> K + c: O unchanged, LSE_i += scale q_i.c;  V -> V + c: O += c."""
    rng = np.random.default_rng(3)
    layout = ((5, 1, 7, 3), (16,))
    S, Hq, Hkv, d, scale = 16, 4, 2, 6, 0.4
    q = rng.standard_normal((2, S, Hq, d)); k = rng.standard_normal((2, S, Hkv, d))
    v = rng.standard_normal((2, S, Hkv, d)); do = rng.standard_normal((2, S, Hq, d))
    o, lse = A.forward(q, k, v, layout, 0, scale)
    dq, _, _ = A.backward(q, k, v, do, layout, 0, scale)
    for b, lens in enumerate(layout):
        starts = np.cumsum((0,) + lens[:-1])
        for s in starts:
            for h in range(Hq):
                g = h // 2
                np.testing.assert_allclose(o[b, s, h], v[b, s, g], atol=1e-14)
                np.testing.assert_allclose(lse[b, h, s], scale * q[b, s, h] @ k[b, s, g], atol=1e-14)
                np.testing.assert_allclose(dq[b, s, h], 0.0, atol=1e-14)
    o0, lse0 = A.forward(np.zeros_like(q), k, v, layout, 0, scale)
    for b, lens in enumerate(layout):
        pos = 0
        for Ln in lens:
            for i in range(pos, pos + Ln):
                n = i - pos + 1
                for h in range(Hq):
                    np.testing.assert_allclose(o0[b, i, h], v[b, pos:i + 1, h // 2].mean(0), atol=1e-14)
                    np.testing.assert_allclose(lse0[b, h, i], math.log(n), atol=1e-14)
            pos += Ln
    c = rng.standard_normal(d)
    o1, lse1 = A.forward(q, k + c, v, layout, 0, scale)
    np.testing.assert_allclose(o1, o, atol=1e-12)
    np.testing.assert_allclose(lse1, lse + scale * np.einsum("bihd,d->bhi", q, c), atol=1e-12)
    o2, lse2 = A.forward(q, k, v + c, layout, 0, scale)
    np.testing.assert_allclose(o2, o + c, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)


def test_useful_pairs_closed_form():
    """Pin: for row_offset 0 the pair count is sum L(L+1)/2 over documents
    (workload 1: 40,003 per head) and equals the mask's popcount."""
    w = synthetic.workload(1)
    assert A.useful_pairs(w.doc_lens, 512, 0, 512) == sum(L * (L + 1) // 2 for L in w.doc_lens[0]) == 40003
    rng = np.random.default_rng(11)
    for _ in range(10):
        S = int(rng.integers(1, 30))
        layout = rand_layout(rng, 2, S)
        a = int(rng.integers(0, S)); b = int(rng.integers(a, S + 1))
        M = A.block_causal_mask(layout, S, a, b - a)
        assert A.useful_pairs(layout, S, a, b - a) == int(M.sum())


# ---------------------------------------------------------------- finite differences


def test_backward_finite_differences():
    """Pin: central finite differences of L = sum(dO * O) in fp64."""
    rng = np.random.default_rng(5)
    layout = ((3, 4, 2), (9,))
    S, Hq, Hkv, d, scale, a, b = 9, 2, 1, 3, 0.8, 2, 9
    q = rng.standard_normal((2, S, Hq, d))[:, a:b].copy(); k = rng.standard_normal((2, S, Hkv, d))
    v = rng.standard_normal((2, S, Hkv, d)); do = rng.standard_normal((2, b - a, Hq, d))
    dq, dk, dv = A.backward(q, k, v, do, layout, a, scale)
    eps = 1e-6

    def loss(qq, kk, vv):
        return float((A.forward(qq, kk, vv, layout, a, scale)[0] * do).sum())

    for x, gx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = [q, k, v]; args_m = [q, k, v]
            args_p[which] = xp; args_m[which] = xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(gx, num, atol=1e-7, rtol=1e-6)


# ---------------------------------------------------------------- invariants


def test_gradient_invariants():
    """Pin: (i) each softmax row's dS sums to zero, so for a document whose
    rows are all local, sum over its keys of dK is zero; (ii) each row's
    weights sum to one, so sum over keys of dV equals sum over real rows of
    dO, summed over the query heads sharing a K/V head."""
    rng = np.random.default_rng(9)
    layout = ((6, 9, 5),)
    S, Hq, Hkv, d, scale = 24, 4, 2, 5, 0.5   # 4 padding positions at the end
    q = rng.standard_normal((1, S, Hq, d)); k = rng.standard_normal((1, S, Hkv, d))
    v = rng.standard_normal((1, S, Hkv, d)); do = rng.standard_normal((1, S, Hq, d))
    dq, dk, dv = A.backward(q, k, v, do, layout, 0, scale)
    pos = 0
    for Ln in layout[0]:
        np.testing.assert_allclose(dk[0, pos:pos + Ln].sum(0), 0.0, atol=1e-12)
        pos += Ln
    for g in range(Hkv):
        np.testing.assert_allclose(dv[0, :, g].sum(0), do[0, :20, 2 * g:2 * g + 2].sum((0, 1)), atol=1e-12)
    # padding: rows give zero dQ, keys zero dK/dV; forward gives O=0, LSE=-inf
    o, lse = A.forward(q, k, v, layout, 0, scale)
    assert np.all(o[0, 20:] == 0) and np.all(np.isneginf(lse[0, :, 20:]))
    assert np.all(dq[0, 20:] == 0) and np.all(dk[0, 20:] == 0) and np.all(dv[0, 20:] == 0)


@pytest.mark.parametrize("cp", [2, 3, 4, 8])
def test_chunk_concatenation(cp):
    """Pin (key property 1): per-chunk outputs concatenated over contiguous
    chunks equal the full call; per-chunk dK/dV summed over chunks equal the
    full dK/dV (the reduce-scatter SUM of the exchange)."""
    rng = np.random.default_rng(20 + cp)
    S = 48
    layout = rand_layout(rng, 2, S)
    q = rng.standard_normal((2, S, 4, 8)); k = rng.standard_normal((2, S, 2, 8))
    v = rng.standard_normal((2, S, 2, 8)); do = rng.standard_normal((2, S, 4, 8))
    o, lse = A.forward(q, k, v, layout, 0, 0.5)
    dq, dk, dv = A.backward(q, k, v, do, layout, 0, 0.5)
    bounds = np.linspace(0, S, cp + 1).astype(int) if cp != 3 else np.array([0, 5, 30, 48])
    dk_sum = np.zeros_like(dk); dv_sum = np.zeros_like(dv)
    for a, b in zip(bounds[:-1], bounds[1:]):
        oc, lc = A.forward(q[:, a:b], k, v, layout, a, 0.5)
        dqc, dkc, dvc = A.backward(q[:, a:b], k, v, do[:, a:b], layout, a, 0.5)
        np.testing.assert_allclose(oc, o[:, a:b], atol=1e-13)
        np.testing.assert_array_equal(np.isneginf(lc), np.isneginf(lse[:, :, a:b]))
        np.testing.assert_allclose(np.where(np.isinf(lc), 0, lc), np.where(np.isinf(lse[:, :, a:b]), 0, lse[:, :, a:b]), atol=1e-13)
        np.testing.assert_allclose(dqc, dq[:, a:b], atol=1e-13)
        dk_sum += dkc; dv_sum += dvc
    np.testing.assert_allclose(dk_sum, dk, atol=1e-12)
    np.testing.assert_allclose(dv_sum, dv, atol=1e-12)


def test_document_independence():
    """Pin: perturbing one document's inputs changes only that document's
    outputs (rows) and gradients (rows and keys) -- bit for bit elsewhere."""
    rng = np.random.default_rng(13)
    layout = ((7, 10, 6, 9),)
    S = 32
    q = rng.standard_normal((1, S, 2, 4)); k = rng.standard_normal((1, S, 1, 4))
    v = rng.standard_normal((1, S, 1, 4)); do = rng.standard_normal((1, S, 2, 4))
    base = A.forward(q, k, v, layout, 0, 0.9) + A.backward(q, k, v, do, layout, 0, 0.9)
    lo, hi = 7, 17
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[0, lo:hi] += rng.standard_normal(x[0, lo:hi].shape)
    pert = A.forward(q2, k2, v2, layout, 0, 0.9) + A.backward(q2, k2, v2, do2, layout, 0, 0.9)
    outside = np.r_[0:lo, hi:S]
    o, lse, dq, dk, dv = base
    o2, lse2, dq2, dk2, dv2 = pert
    np.testing.assert_array_equal(o[0, outside], o2[0, outside])
    np.testing.assert_array_equal(lse[0][:, outside], lse2[0][:, outside])
    for x, y in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_array_equal(x[0, outside], y[0, outside])
    assert np.abs(o[0, lo:hi] - o2[0, lo:hi]).min() > 0


def test_windowed_and_row_subset_match_dense():
    """The windowed mode and the row-subset mode are the dense definition up
    to summation order (workload 1 plus random layouts with padding)."""
    w = synthetic.workload(1)
    t = synthetic.draw_tensors(w)
    o, lse = A.forward(t["q"], t["k"], t["v"], w.doc_lens, 0, w.scale)
    dq, dk, dv = A.backward(t["q"], t["k"], t["v"], t["do"], w.doc_lens, 0, w.scale)
    for R in (1, 7, 64, 512):
        ow, lw = A.forward(t["q"], t["k"], t["v"], w.doc_lens, 0, w.scale, block_rows=R)
        g = A.backward(t["q"], t["k"], t["v"], t["do"], w.doc_lens, 0, w.scale, block_rows=R)
        np.testing.assert_allclose(ow, o, atol=1e-12)
        np.testing.assert_allclose(lw, lse, atol=1e-12)
        for x, y in zip(g, (dq, dk, dv)):
            np.testing.assert_allclose(x, y, atol=1e-12)
    rows = [0, 5, 199, 200, 236, 237, 511]
    os_, ls_ = A.forward(t["q"], t["k"], t["v"], w.doc_lens, 0, w.scale, block_rows=3, rows=rows)
    np.testing.assert_allclose(os_[:, rows], o[:, rows], atol=1e-12)
    np.testing.assert_allclose(ls_[:, :, rows], lse[:, :, rows], atol=1e-12)
    # dK/dV of keys attended only by the given rows are exact: keys 237..386
    # (third document) attended by rows 237..386 only
    rows3 = list(range(237, 387))
    _, dk3, dv3 = A.backward(t["q"], t["k"], t["v"], t["do"], w.doc_lens, 0, w.scale, rows=rows3, block_rows=16)
    np.testing.assert_allclose(dk3[:, 237:387], dk[:, 237:387], atol=1e-12)
    np.testing.assert_allclose(dv3[:, 237:387], dv[:, 237:387], atol=1e-12)
    rng = np.random.default_rng(2)
    for _ in range(5):
        layout, S, q, k, v, do, scale = rand_case(int(rng.integers(1 << 30)), S=20)
        a = int(rng.integers(0, 10))
        ref = A.forward(q[:, a:], k, v, layout, a, scale)
        win = A.forward(q[:, a:], k, v, layout, a, scale, block_rows=4)
        for x, y in zip(ref, win):
            np.testing.assert_allclose(np.where(np.isinf(x), 0, x), np.where(np.isinf(y), 0, y), atol=1e-12)


# ---------------------------------------------------------------- segment reference


@pytest.mark.parametrize("seed", range(20))
def test_segment_ref_against_mask(seed):
    """Pin: segments read off the dense mask by brute force -- they partition
    the local rows in order; each segment's rows see exactly the keys
    [k_begin, k_begin + t + k_len - q_len] (bottom-right alignment); padding
    segments see none; the segment pair count equals the mask popcount."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4)); S = int(rng.integers(1, 25))
    layout = rand_layout(rng, B, S)
    if seed % 3 == 0:  # zero-length documents are allowed and ignored
        layout = tuple(tuple(list(r) + [0]) for r in layout)
    a = int(rng.integers(0, S + 1)); b = int(rng.integers(a, S + 1))
    L = b - a
    t = SEG.segment_ref(layout, S, a, L)
    M = A.block_causal_mask(layout, S, a, L)
    cu_q, cu_k, kb = t["cu_q"], t["cu_k"], t["k_begin"]
    assert cu_q[0] == 0 and cu_q[-1] == B * L
    pairs = 0
    for s in range(t["n_seg"]):
        qn, kn = cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s]
        assert qn > 0
        for r in range(cu_q[s], cu_q[s + 1]):
            bb, tt = divmod(r, L)
            allowed = np.flatnonzero(M[bb, tt]) + bb * S
            if kn == 0:
                assert allowed.size == 0
            else:
                expect = np.arange(kb[s], kb[s] + (r - cu_q[s]) + kn - qn + 1)
                np.testing.assert_array_equal(allowed, expect)
                pairs += allowed.size
    assert pairs == int(M.sum())


def test_segment_ref_rejects_bad_input():
    with pytest.raises(SEG.MetadataError):
        SEG.segment_ref([[3, -1]], 4, 0, 4)
    with pytest.raises(SEG.MetadataError):
        SEG.segment_ref([[3, 2]], 4, 0, 4)
    with pytest.raises(SEG.MetadataError):
        SEG.segment_ref([[4]], 4, 2, 3)


@pytest.mark.parametrize("seed", range(10))
def test_mask_bounds_numpy_matches_scan(seed):
    """The numpy per-row / per-key bounds equal the ones read off the mask by
    scanning (which asserts the allowed sets are intervals)."""
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 30))
    layout = rand_layout(rng, 2, S)
    a = int(rng.integers(0, S + 1)); b = int(rng.integers(a, S + 1))
    scan = SEG.mask_bounds(layout, S, a, b - a)
    fast = SEG.mask_bounds_np(layout, S, a, b - a)
    for x, y in zip(scan, fast):
        np.testing.assert_array_equal(np.array(x).reshape(y.shape), y)


def test_live_tile_ranges_are_exact():
    """Skipping fully masked tiles: for a query tile, the key tiles holding at
    least one allowed pair are exactly the contiguous range from the tile of
    the first real row's document start to the tile of the last real row;
    for a key tile, the query tiles are the range spanned by its keys'
    attending rows.  Checked against the mask on workload-shaped layouts at
    several tile sizes."""
    rng = np.random.default_rng(1)
    cases = [(synthetic.workload(1).doc_lens, 512, 0, 512)]
    for _ in range(6):
        S = int(rng.integers(40, 300))
        layout = rand_layout(rng, 2, S)
        a = int(rng.integers(0, S // 2)); b = int(rng.integers(a + 1, S + 1))
        cases.append((layout, S, a, b - a))
    for layout, S, a, L in cases:
        M = A.block_causal_mask(layout, S, a, L)
        lo, hi, qlo, qhi = SEG.mask_bounds_np(layout, S, a, L)
        for BM, BN in ((32, 64), (32, 32), (16, 64), (64, 128)):
            for bb in range(len(layout)):
                for t0 in range(0, L, BM):
                    t1 = min(t0 + BM, L)
                    live = {j // BN for t in range(t0, t1) for j in np.flatnonzero(M[bb, t])}
                    real = [t for t in range(t0, t1) if hi[bb, t] > lo[bb, t]]
                    rng_ = set(range(lo[bb, real[0]] // BN, (hi[bb, real[-1]] - 1) // BN + 1)) if real else set()
                    assert live == rng_
                for j0 in range(0, S, BN):
                    j1 = min(j0 + BN, S)
                    live = {t // BM for j in range(j0, j1) for t in np.flatnonzero(M[bb, :, j])}
                    att = [j for j in range(j0, j1) if qhi[bb, j] > qlo[bb, j]]
                    rng_ = set(range(qlo[bb, att[0]] // BM, (qhi[bb, att[-1]] - 1) // BM + 1)) if att else set()
                    assert live == rng_


# ---------------------------------------------------------------- generator


def test_generator_reference_draws_and_bf16_rounding():
    """The seeded generator reproduces its documented draws; round_bf16 is
    round-to-nearest-even as torch's float32 -> bfloat16 conversion."""
    assert synthetic.doc_lengths(2) == ((619, 304, 339, 45, 2789), (1608, 370, 1110, 678, 294, 36))
    assert synthetic.doc_lengths(3) == ((3913, 3126, 1824, 1649, 4238, 1634),)
    d4 = synthetic.doc_lengths(4)[0]
    assert d4[:4] == (24576, 133, 215, 1351) and sum(d4) == 32768 and len(d4) == 19
    d5 = synthetic.doc_lengths(5)[0]
    assert len(d5) == 694 and sum(d5) == 49152 and d5[:4] == (91, 106, 18, 107)
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]  # exact ties
    r = synthetic.round_bf16(x)
    t = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(r, t)


@pytest.mark.parametrize("block_rows", [None, 16])
def test_parallel_runner_matches_direct_calls(block_rows):
    """oracle.parallel.run re-poses each (batch row, K/V head, row range) job
    on its key window and reassembles the results; pinned against the direct
    oracle.attention calls on a chunked GQA problem (B = 2, a padding tail, a
    document straddling the chunk's left edge), with the rows split into
    several ranges per head and into a sampled subset, to <= 1e-12."""
    rng = np.random.default_rng(11)
    layout = ((37, 5, 60, 18), (90, 20, 6))   # row 1 ends in 4 padding tokens
    S, r0, L, Hq, Hkv, d = 120, 23, 90, 6, 2, 8
    q = rng.standard_normal((2, L, Hq, d))
    k = rng.standard_normal((2, S, Hkv, d))
    v = rng.standard_normal((2, S, Hkv, d))
    do = rng.standard_normal((2, L, Hq, d))
    scale = 0.3
    from oracle import parallel
    o, lse = A.forward(q, k, v, layout, r0, scale)
    dq, dk, dv = A.backward(q, k, v, do, layout, r0, scale)
    for pieces, workers in ((1, 1), (5, 1), (3, 2)):
        got = parallel.run(q, k, v, do, layout, r0, scale, block_rows=block_rows, workers=workers,
                           pieces=pieces)
        assert np.array_equal(np.isneginf(got["lse"]), np.isneginf(lse))
        fin = np.isfinite(lse)
        assert np.abs(got["lse"][fin] - lse[fin]).max() <= 1e-12
        for name, ref in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
            assert np.abs(got[name] - ref).max() <= 1e-12, (name, pieces)
    rows = [0, 1, 13, 14, 40, 41, 42, 77, 88, 89]
    o_s, lse_s = A.forward(q, k, v, layout, r0, scale, rows=rows)
    dq_s, dk_s, dv_s = A.backward(q, k, v, do, layout, r0, scale, rows=rows)
    got = parallel.run(q, k, v, do, layout, r0, scale, block_rows=block_rows, rows=rows, workers=1, pieces=4)
    for name, ref in (("o", o_s), ("dq", dq_s), ("dk", dk_s), ("dv", dv_s)):
        assert np.abs(got[name] - ref).max() <= 1e-12, name
    assert np.array_equal(np.isneginf(got["lse"]), np.isneginf(lse_s))
