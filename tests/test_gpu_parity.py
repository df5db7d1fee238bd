"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

* metadata: per-row / per-key bounds built on the device are bit-exact
  against the oracle's bounds;
* small cases (seconds for the dense oracle) spanning several tiles with
  ragged tails: float32 and bfloat16, head_dim 64 / 128 (matrix-core path)
  and others (generic path), grouped-query ratios 1..8, chunks at a
  row_offset with straddling documents, padding, empty and all-padding
  chunks, a single document, many tiny documents;
* a batch row past 31-bit buffer offsets (2^24 tokens, 2 GiB K and V):
  the generic kernels' 64-bit indexing, checked on the chunk's documents;
* the five named workloads at full size: 1, 2, 3 and 5 against the full
  oracle, with the bf16 gradient bound also applied to every document on
  its own; 4 (a 24576-token document) against the full oracle for one K/V
  head and its query heads (every row and key), on sampled rows for the
  other heads, plus full-size invariants.
Tolerances are in tests/helpers.py.
"""
import sys

import numpy as np
import pytest

import synthetic
from tests import helpers as H

gpu = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@gpu
@pytest.mark.parametrize("wid", synthetic.WORKLOADS)
def test_metadata_bit_exact(wid):
    import packed_sequence_attention_amd as bd
    from oracle import segment as SEG
    w = synthetic.workload(wid)
    _log(f"meta workload {wid}")
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device="cuda")
    got = [x.cpu().numpy() for x in seg.meta_views()]
    ref = SEG.mask_bounds_np(w.doc_lens, w.seq_len, w.row_offset, w.q_len)
    for g_, r_ in zip(got, ref):
        np.testing.assert_array_equal(g_, r_)


@gpu
def test_metadata_bit_exact_random_layouts():
    import packed_sequence_attention_amd as bd
    from oracle import segment as SEG
    rng = np.random.default_rng(0)
    for i in range(30):
        B = int(rng.integers(1, 4)); S = int(rng.integers(1, 400))
        rows = []
        for _ in range(B):
            lens, tot = [], 0
            fill = S if rng.random() < 0.5 else int(rng.integers(0, S + 1))
            while tot < fill:
                Ln = int(min(rng.integers(0, 80), fill - tot)); lens.append(Ln); tot += Ln
            rows.append(lens)
        a = int(rng.integers(0, S)); b = int(rng.integers(a + 1, S + 1))
        seg = bd.segment(rows, S, a, b - a, device="cuda")
        got = [x.cpu().numpy() for x in seg.meta_views()]
        ref = SEG.mask_bounds_np(rows, S, a, b - a)
        for g_, r_ in zip(got, ref):
            np.testing.assert_array_equal(g_, r_)


def _work_bin(w):
    """Work bins of the launch orders: exact below 128, then 16 per octave."""
    w = np.maximum(np.asarray(w, np.int64), 0)
    e = np.floor(np.log2(np.maximum(w, 1))).astype(np.int64)
    hi = 128 + (e - 7) * 16 + ((w >> np.maximum(e - 4, 0)) & 15)
    return np.where(w < 128, w, np.minimum(hi, 255))


def _expected_visits(bounds, row_offset):
    """Key tiles of 32 each 32-row query tile visits (from doc_start of its
    first real row to its last real row; 0 for an all-padding tile), from the
    oracle's mask bounds, in tile-code order b * n_qt + qt."""
    row_lo, row_hi = bounds[0], bounds[1]
    out = []
    for b in range(row_lo.shape[0]):
        for t0 in range(0, row_lo.shape[1], 32):
            real = np.nonzero(row_hi[b, t0:t0 + 32] > row_lo[b, t0:t0 + 32])[0]
            out.append(0 if len(real) == 0 else
                       (row_offset + t0 + real.max()) // 32 - row_lo[b, t0 + real.min()] // 32 + 1)
    return np.array(out, np.int64)


@gpu
@pytest.mark.parametrize("case", range(7))
def test_query_tile_order(case):
    """The metadata's query-tile launch order: a permutation of the tile
    codes, visit bins non-increasing along it with ties in ascending code
    order, and statistics [largest, total] equal to those of the visit counts
    computed from the oracle's mask bounds (five workloads and two chunked,
    padded layouts)."""
    import packed_sequence_attention_amd as bd
    from oracle import segment as SEG
    if case < 5:
        w = synthetic.workload(synthetic.WORKLOADS[case])
        rows, S, r0, L = w.doc_lens, w.seq_len, w.row_offset, w.q_len
    elif case == 5:
        rows, S, r0, L = [[300, 40, 500, 100], [1000], [7, 9, 600]], 1024, 256, 512
    else:
        rows, S, r0, L = [[5000, 3000, 100], [64] * 100], 9000, 4000, 4200
    _log(f"query-tile order case {case}")
    seg = bd.segment(rows, S, r0, L, device="cuda")
    order, stats = seg.q_order()
    visits = _expected_visits(SEG.mask_bounds_np(rows, S, r0, L), r0)
    g = order.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(np.sort(g), np.arange(len(visits)))
    bins = _work_bin(visits)[g]
    assert np.all(np.diff(bins) <= 0)
    same = np.diff(bins) == 0
    assert np.all(np.diff(g)[same] > 0)
    np.testing.assert_array_equal(stats.cpu().numpy(), [visits.max(), visits.sum()])


@gpu
def test_metadata_inline_and_device_tables_agree():
    """The table passed by value in the launch arguments and the table copied
    to the device give the same metadata, bit for bit, at the size limit of
    the by-value path and on both sides of it, and both match the oracle."""
    import packed_sequence_attention_amd as bd
    from oracle import segment as SEG
    mx = bd.load_library().blockdiag_meta_inline_max_seg()
    rng = np.random.default_rng(7)
    layouts = [([[4] * mx], 4 * mx, 0, 4 * mx), ([[4] * mx], 4 * mx, 100, 200),
               ([[3] * (mx + 1)], 3 * (mx + 1), 0, 3 * (mx + 1))]
    for _ in range(6):
        B = int(rng.integers(1, 4)); S = int(rng.integers(64, 600))
        rows = [[int(x) for x in rng.integers(1, 40, size=int(rng.integers(1, 40)))] for _ in range(B)]
        rows = [r if sum(r) <= S else [S] for r in rows]
        a = int(rng.integers(0, S)); b = int(rng.integers(a + 1, S + 1))
        layouts.append((rows, S, a, b - a))
    for rows, S, a, L in layouts:
        _log(f"meta inline/device S={S} chunk=[{a},{a + L}) rows={len(rows)}")
        t = bd.segment(rows, S, a, L)
        ref = SEG.mask_bounds_np(rows, S, a, L)
        dev = [x.cpu().numpy() for x in t.to("cuda", inline=False).meta_views()]
        for g_, r_ in zip(dev, ref):
            np.testing.assert_array_equal(g_, r_)
        if t.n_seg <= mx:
            inl = [x.cpu().numpy() for x in t.to("cuda", inline=True).meta_views()]
            for g_, r_ in zip(inl, dev):
                np.testing.assert_array_equal(g_, r_)
        else:
            with pytest.raises(bd.BlockdiagError):
                t.to("cuda", inline=True)


def _rand_docs(seed, S, fill=None, lo=1, hi=None):
    rng = np.random.default_rng(seed)
    fill = S if fill is None else fill
    hi = hi or S
    lens, tot = [], 0
    while tot < fill:
        Ln = int(min(rng.integers(lo, hi + 1), fill - tot)); lens.append(Ln); tot += Ln
    return lens


SMALL = [
    # (dtype, doc_lens rows, S, row_offset, q_len, h_q, h_kv, d)
    ("f32", [[200, 37, 150, 125]], 512, 0, 512, 4, 4, 64),
    ("f32", [_rand_docs(1, 333, fill=300)], 333, 45, 250, 8, 2, 128),
    ("f32", [_rand_docs(2, 200)], 200, 0, 200, 3, 1, 40),
    ("bf16", [_rand_docs(3, 300), _rand_docs(4, 300, fill=260)], 300, 0, 300, 8, 2, 128),
    ("bf16", [_rand_docs(5, 700, hi=300)], 700, 100, 513, 8, 2, 64),
    ("bf16", [_rand_docs(6, 450)], 450, 0, 450, 16, 2, 128),
    ("bf16", [_rand_docs(7, 260)], 260, 30, 200, 4, 2, 96),
    ("bf16", [_rand_docs(8, 257)], 257, 0, 257, 4, 4, 128),
    ("bf16", [[600]], 600, 0, 600, 8, 2, 128),
    ("bf16", [[600]], 600, 0, 600, 4, 1, 64),
    ("bf16", [_rand_docs(9, 800, lo=1, hi=9)], 800, 0, 800, 4, 1, 128),
    ("bf16", [[100, 50]], 400, 200, 200, 4, 1, 128),
    ("bf16", [_rand_docs(10, 500, fill=120, hi=40)], 500, 0, 500, 4, 1, 64),
    ("bf16", [[70], [300], [129, 1]], 300, 64, 129, 8, 2, 64),
    ("bf16", [[1000]], 1000, 967, 33, 4, 1, 128),
    ("f32", [_rand_docs(11, 380, fill=350)], 380, 0, 380, 4, 1, 64),
    # head_dim 256 (matrix-core forward and backward) and GQA 8:1, padding
    # tail; float32 head_dim 256 on the generic kernels
    ("bf16", [_rand_docs(12, 300, fill=280)], 300, 20, 250, 8, 1, 256),
    ("f32", [_rand_docs(13, 200)], 200, 0, 200, 2, 2, 256),
    ("bf16", [_rand_docs(14, 700, hi=400)], 700, 0, 700, 8, 2, 256),
    ("bf16", [[500, 300], [150, 650]], 800, 300, 421, 4, 1, 256),
    # matrix-core kernels at GQA ratios that are not a multiple of 4: two
    # heads and two query tiles per workgroup (ratio 2, 6), one head and four
    # query tiles (ratio 1, 3); ragged tails, chunks, padding, head_dim 256
    ("bf16", [_rand_docs(15, 900, hi=500)], 900, 0, 900, 8, 8, 128),
    ("bf16", [_rand_docs(16, 700, fill=650, hi=300), _rand_docs(17, 700)], 700, 77, 555, 8, 4, 128),
    ("bf16", [_rand_docs(18, 1000, hi=600)], 1000, 200, 700, 6, 2, 64),
    ("bf16", [_rand_docs(19, 640, hi=200)], 640, 0, 640, 12, 2, 128),
    ("bf16", [_rand_docs(20, 500, hi=300)], 500, 37, 400, 4, 4, 256),
    ("bf16", [_rand_docs(21, 600, hi=250)], 600, 0, 600, 4, 2, 256),
    ("bf16", [[1, 2, 3, 300, 1, 200]], 520, 0, 520, 2, 2, 64),
    # GQA 16:1 (the dK/dV kernel's four rounds of four heads), three batch
    # rows with a one-row chunk, and a 32:1 group at head_dim 64
    ("bf16", [_rand_docs(22, 300, hi=200)], 300, 0, 300, 16, 1, 128),
    ("bf16", [_rand_docs(23, 260), _rand_docs(24, 260, fill=200), _rand_docs(25, 260)], 260, 13, 1, 4, 2, 64),
    ("bf16", [_rand_docs(26, 330, hi=150), _rand_docs(27, 330)], 330, 0, 330, 32, 1, 64),
    # generic kernels at head_dims past 128 that are not multiples of 64: a
    # partial third block of 64 columns and a fourth wholly past the row
    # (float32, and bf16 at a head_dim the matrix-core kernels do not take)
    ("f32", [_rand_docs(28, 220)], 220, 0, 220, 2, 1, 136),
    ("bf16", [_rand_docs(29, 180, fill=170)], 180, 20, 160, 4, 4, 200),
]


@gpu
@pytest.mark.parametrize("i", range(len(SMALL)))
def test_small_case_parity(i):
    dtype, docs, S, r0, L, hq, hkv, d = SMALL[i]
    w, t = H.small_case(i, dtype, docs, S, r0, L, hq, hkv, d)
    _log(f"small case {i}: {dtype} S={S} r0={r0} L={L} H={hq}/{hkv} d={d} docs={len(docs[0])}")
    gpu_out = H.run_gpu(w, t)
    ref = H.oracle(w, t, block_rows=None)
    errs = H.check(w, gpu_out, ref)
    _log("  errors", {k: f"{v:.3g}" for k, v in errs.items()})


@gpu
def test_empty_chunk_and_zero_gradients():
    """q_len = 0 is a no-op forward and zero dK/dV; an all-padding chunk gives
    O = 0, LSE = -inf and zero gradients."""
    import torch
    import packed_sequence_attention_amd as bd
    w, t = H.small_case(90, "bf16", [[40]], 128, 64, 64, 4, 1, 128)
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device="cuda")
    dv = H.to_device(w, t)
    o, lse = bd.attn_fwd(dv["q"], dv["k"], dv["v"], seg)
    dq, dk, dvv = bd.attn_bwd(dv["q"], dv["k"], dv["v"], o, lse, dv["do"], seg)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dvv == 0)
    seg0 = bd.segment(w.doc_lens, w.seq_len, 10, 0, device="cuda")
    q0 = dv["q"][:, :0].contiguous()
    o0, lse0 = bd.attn_fwd(q0, dv["k"], dv["v"], seg0)
    dq0, dk0, dv0 = bd.attn_bwd(q0, dv["k"], dv["v"], o0, lse0, q0, seg0)
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.all(dk0 == 0) and torch.all(dv0 == 0)



@gpu
def test_row_past_31_bit_offsets():
    """Largest sizes: a batch row of 2^24 tokens whose K and V are 2 GiB each
    (h_kv = 1, head_dim 64), more than 31-bit buffer offsets address, so
    every kernel takes its 64-bit-indexed generic form.  The chunk is the
    row's last 256 rows (two documents after one long one); O, LSE and dQ
    match the oracle on those two documents alone, dK and dV match it on
    their keys and are exactly zero on the long document's keys."""
    import torch
    import packed_sequence_attention_amd as bd
    S, tail = 1 << 24, [100, 156]
    n = sum(tail)
    w_s, t = H.small_case(95, "bf16", [tail], n, 0, n, 4, 1, 64)
    ref = H.oracle(w_s, t, block_rows=None)
    _log(f"row of {S} tokens, chunk of the last {n} rows")
    seg = bd.segment([[S - n] + tail], S, S - n, n, device="cuda")
    dev = H.to_device(w_s, t)
    k = torch.zeros((1, S, 1, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    k[:, S - n:] = dev["k"]
    v[:, S - n:] = dev["v"]
    o, lse = bd.attn_fwd(dev["q"], k, v, seg, w_s.scale)
    dq, dk, dv = bd.attn_bwd(dev["q"], k, v, o, lse, dev["do"], seg, w_s.scale)
    torch.cuda.synchronize()
    zero_k = bool((dk[:, :S - n] == 0).all().item()) and bool((dv[:, :S - n] == 0).all().item())
    got = {"o": o, "lse": lse, "dq": dq, "dk": dk[:, S - n:], "dv": dv[:, S - n:]}
    got = {name: x.double().cpu().numpy() for name, x in got.items()}
    del k, v, dk, dv
    torch.cuda.empty_cache()
    assert zero_k, "dK / dV must be zero at keys no row of the chunk attends"
    errs = H.check(w_s, got, ref)
    _log("  errors", {name: f"{e:.3g}" for name, e in errs.items()})


FULL_REPORT = {}


@gpu
@pytest.mark.parametrize("wid", [1, 2, 3, 5])
def test_workload_full_parity(wid):
    w = synthetic.workload(wid)
    _log(f"workload {wid}: {w.name}")
    t = synthetic.draw_tensors(w)
    gpu_out = H.run_gpu(w, t)
    _log("  gpu done; oracle ...")
    ref = H.oracle(w, t, block_rows=None if wid == 1 else 256)
    errs = H.check(w, gpu_out, ref)
    FULL_REPORT[wid] = errs
    _log("  errors", {k: f"{v:.3g}" for k, v in errs.items()})
    if w.dtype == "bf16":
        # the bf16 gradient bound, applied to every document on its own
        worst = H.per_doc_grad_errors(w, gpu_out, ref)
        _log("  worst per-document relative Frobenius", {k: f"{v:.3g}" for k, v in worst.items()})
        for name, e in worst.items():
            assert e <= H.TOL["bf16"]["grad_rel_fro"], f"{name}: a document's error {e:.3g}"


@gpu
def test_workload4_full_group_parity_and_invariants():
    """Workload 4 (S = 32768, one 24576-token document then short ones).
    K/V head 0 with its four query heads, every row and every key, against
    the oracle: O and LSE by max-abs, dQ, dK, dV by relative Frobenius over
    the group and per document -- this covers all 24576 keys of the long
    document, whose key tiles run the longest query sweeps.  The other heads:
    O, LSE and dQ on sampled rows, and the full-size invariant that each
    row's attention weights sum to one, so sum_j dV_j equals the sum of dO
    over the group's rows (per K/V head)."""
    w = synthetic.workload(4)
    t = synthetic.draw_tensors(w)
    _log("workload 4: gpu ...")
    g = H.run_gpu(w, t)
    G = w.h_q // w.h_kv
    tg = {"q": t["q"][:, :, :G], "k": t["k"][:, :, :1], "v": t["v"][:, :, :1], "do": t["do"][:, :, :G]}
    wg = synthetic.custom_workload(w.wid, w.dtype, w.doc_lens, w.seq_len, w.row_offset, w.q_len, G, 1,
                                   w.head_dim, w.scale, name="workload 4, K/V head 0")
    _log("  oracle, K/V head 0 (all rows and keys) ...")
    ref = H.oracle(wg, tg, block_rows=256)
    gg = {"o": g["o"][:, :, :G], "lse": g["lse"][:, :G], "dq": g["dq"][:, :, :G],
          "dk": g["dk"][:, :, :1], "dv": g["dv"][:, :, :1]}
    errs = H.check(wg, gg, ref)
    _log("  errors (K/V head 0)", {k: f"{v:.3g}" for k, v in errs.items()})
    worst = H.per_doc_grad_errors(wg, gg, ref)
    _log("  worst per-document relative Frobenius", {k: f"{v:.3g}" for k, v in worst.items()})
    for name, e in worst.items():
        assert e <= H.TOL["bf16"]["grad_rel_fro"], f"{name}: a document's error {e:.3g}"
    rng = np.random.default_rng(44)
    starts = np.cumsum((0,) + w.doc_lens[0][:-1])
    rows = sorted(set([0, 1, 31, 32, 63, 64, 24575, 24576, 24577, 32767] + list(starts)
                      + list(rng.integers(0, 32768, 24))))
    _log(f"  oracle, all heads on {len(rows)} rows ...")
    refr = H.oracle(w, t, rows=rows, block_rows=64)
    H.check(w, {"o": g["o"], "lse": g["lse"]}, {"o": refr["o"], "lse": refr["lse"]}, rows=rows)
    e_dq = H.rel_fro(g["dq"][:, rows], refr["dq"][:, rows])
    assert e_dq <= 5e-2, e_dq
    do = t["do"].astype(np.float64)
    for gh in range(w.h_kv):
        lhs = g["dv"][0, :, gh].sum(0)
        rhs = do[0, :, gh * G:(gh + 1) * G].sum((0, 1))
        assert np.linalg.norm(lhs - rhs) <= 1e-2 * np.linalg.norm(rhs) + 1e-3
    _log("  sampled dQ (all heads)", f"{e_dq:.3g}")


@gpu
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_single_document_spanning_every_chunk(dtype, d):
    """One document fills the row and is split into 4 contiguous chunks (the
    context-parallel layout of the Automodel page's Design overview): every
    chunk after the first has a long asymmetric first segment (more keys than
    queries).  Each chunk's O, LSE and dQ match the oracle on its rows, and
    the chunks' partial dK/dV summed over the chunks match the oracle's
    gradients of the whole row (what the reduce-scatter of dK/dV returns)."""
    S, cp = 1536, 4
    w_full, t = H.small_case(400 + d, dtype, [[S]], S, 0, S, 8, 2, d)
    full = H.oracle(w_full, t, block_rows=256)
    L = S // cp
    dk_sum = np.zeros_like(full["dk"])
    dv_sum = np.zeros_like(full["dv"])
    for c in range(cp):
        a = c * L
        wc = synthetic.custom_workload(400 + d, dtype, [[S]], S, a, L, 8, 2, d, name=f"chunk{c}")
        tc = {"q": t["q"][:, a:a + L], "k": t["k"], "v": t["v"], "do": t["do"][:, a:a + L]}
        _log(f"single document {dtype} d={d}: chunk {c} rows [{a}, {a + L})")
        g = H.run_gpu(wc, tc)
        ref_c = {"o": full["o"][:, a:a + L], "lse": full["lse"][:, :, a:a + L], "dq": full["dq"][:, a:a + L]}
        errs = H.check(wc, {"o": g["o"], "lse": g["lse"], "dq": g["dq"], "dk": g["dk"], "dv": g["dv"]},
                       {**ref_c, "dk": g["dk"], "dv": g["dv"]})
        _log("  errors", {k: f"{v:.3g}" for k, v in errs.items() if k not in ("dk", "dv")})
        dk_sum += g["dk"]
        dv_sum += g["dv"]
    errs = H.check(w_full, {"dk": dk_sum, "dv": dv_sum, "dq": full["dq"]},
                   {"dk": full["dk"], "dv": full["dv"], "dq": full["dq"]})
    _log("  summed dK/dV errors", {k: f"{v:.3g}" for k, v in errs.items() if k != "dq"})


@gpu
def test_binding_rejects_mismatched_tensors_before_launch():
    """The Python binding checks every tensor's shape, dtype, layout and
    device against q before any kernel is enqueued; nothing is written."""
    import torch

    import packed_sequence_attention_amd as bd
    _log("binding argument checks")
    seg = bd.segment([[40, 24], [64]], 64, 0, 64, device="cuda")
    q = torch.randn(2, 64, 4, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(2, 64, 2, 64, device="cuda", dtype=torch.bfloat16)
    v = torch.randn_like(k)
    o, lse = bd.attn_fwd(q, k, v, seg)
    do = torch.randn_like(q)
    bad_fwd = [
        (q.cpu(), k, v),                      # q off the device
        (q, k.cpu(), v),                      # k off q's device
        (q, k, v.float()),                    # dtype mismatch
        (q, k.transpose(1, 2), v),            # non-contiguous / wrong shape
        (q[:, :32], k, v),                    # q_len differs from the table
    ]
    for args in bad_fwd:
        with pytest.raises(bd.BlockdiagError):
            bd.attn_fwd(*args, seg)
    bad_bwd = [
        (o.cpu(), lse, do),                   # o off q's device
        (o, lse.cpu(), do),                   # lse off q's device
        (o, lse, do.cpu()),                   # dO off q's device
        (o, lse.double(), do),                # lse dtype
        (o, lse, do.float()),                 # dO dtype
        (o, lse[:, :, :32], do),              # lse shape
    ]
    for o_, l_, d_ in bad_bwd:
        with pytest.raises(bd.BlockdiagError):
            bd.attn_bwd(q, k, v, o_, l_, d_, seg)
    # through the C ABI: metadata built on the device for a smaller chunk is
    # rejected by its descriptor before any launch
    import ctypes
    lib = bd.load_library()
    small = bd.segment([[40, 24], [64]], 64, 0, 32, device="cuda")
    ws = lib.blockdiag_workspace_bytes(1, 1, 2, 64, 64, 4, 2, 64)
    wsb = torch.empty(ws, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    code = lib.blockdiag_attn_fwd(1, 2, 64, 0, 64, 0, 64, 4, 2, 64, 0.125, None, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  ctypes.byref(small.desc), o.data_ptr(), lse.data_ptr(), None, 0, st)
    assert code == 1 and b"metadata" in lib.blockdiag_last_error()
    code = lib.blockdiag_attn_bwd(1, 2, 64, 0, 64, 0, 64, 4, 2, 64, 0.125, None, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  o.data_ptr(), lse.data_ptr(), do.data_ptr(), ctypes.byref(small.desc),
                                  do.data_ptr(), k.data_ptr(), v.data_ptr(), wsb.data_ptr(), ws, st)
    assert code == 1 and b"metadata" in lib.blockdiag_last_error()
    torch.cuda.synchronize()
    # the good call still works after the rejected ones
    dq, dk, dv = bd.attn_bwd(q, k, v, o, lse, do, seg)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t.float()).all().item() for t in (dq, dk, dv))
