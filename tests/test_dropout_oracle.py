"""Pins of the oracle's attention dropout (oracle/dropout.py and the dropout
path of oracle/attention.py), CPU only:

* Philox4x32-10 against the generator's published known-answer vectors;
* the counter layout (which counter fields, which word, which byte) against
  keep decisions worked out by hand from those vectors;
* keep statistics: the dropped fraction matches thr / 256;
* p = 0 reduces to no dropout;
* the backward with dropout against central finite differences (the mask
  does not depend on the inputs) and against torch autograd through the same
  mask applied explicitly;
* masks follow row positions: chunks concatenate to the full call, and the
  process-pool runner (re-indexed sub-problems) equals the direct call."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import dropout as DR
from oracle import parallel

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dropout_hand.json")))


def _h(x):
    return int(x, 16) if isinstance(x, str) else int(x)


def test_philox_known_answers():
    for case in GOLDEN["philox"]:
        c = [np.array([_h(x)]) for x in case["counter"]]
        k0, k1 = (_h(x) for x in case["key"])
        out = DR.philox4x32_10(*c, k0, k1)
        assert ["%08x" % int(w[0]) for w in out] == case["out"]


def test_keep_layout_hand_blocks():
    for blk in GOLDEN["blocks"]:
        rows = np.arange(blk["row0"], blk["row0"] + 4)
        keys = np.arange(blk["key0"], blk["key0"] + 4)
        z = DR.keep_mask(int(blk["seed"], 16), blk["offset"], blk["b"], blk["h"], blk["h_q"], rows, keys, blk["p"])
        assert z.astype(int).tolist() == blk["keep"], blk["why"]


@pytest.mark.parametrize("p", [0.1, 0.3, 0.5])
def test_keep_statistics(p):
    thr, c = DR.keep_scale(p)
    z = DR.keep_mask(12345, 7, 1, 3, 8, np.arange(512), np.arange(1024), p)
    n = z.size
    drop = 1.0 - z.mean()
    sd = np.sqrt(thr / 256 * (1 - thr / 256) / n)
    assert abs(drop - thr / 256) < 5 * sd
    assert c == 256.0 / (256 - thr)
    # rows, heads, offsets and seeds draw different masks
    z2 = DR.keep_mask(12345, 8, 1, 3, 8, np.arange(512), np.arange(1024), p)
    assert (z != z2).mean() > 0.05


def _case(seed=0):
    rng = np.random.default_rng(seed)
    layout = ((5, 7, 4), (9, 7))
    S, r0, L, Hq, Hkv, d = 16, 3, 12, 4, 2, 3
    q = rng.standard_normal((2, L, Hq, d)); k = rng.standard_normal((2, S, Hkv, d))
    v = rng.standard_normal((2, S, Hkv, d)); do = rng.standard_normal((2, L, Hq, d))
    return layout, S, r0, L, Hq, Hkv, d, q, k, v, do


def test_zero_probability_is_no_dropout():
    layout, S, r0, L, Hq, Hkv, d, q, k, v, do = _case()
    drop = A.Dropout(0.0, 99, 5, Hq)
    o0, l0 = A.forward(q, k, v, layout, r0, 0.7)
    o1, l1 = A.forward(q, k, v, layout, r0, 0.7, dropout=drop)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = A.backward(q, k, v, do, layout, r0, 0.7)
    g1 = A.backward(q, k, v, do, layout, r0, 0.7, dropout=drop)
    assert all(np.array_equal(a, b) for a, b in zip(g0, g1))


def test_backward_with_dropout_finite_differences():
    layout, S, r0, L, Hq, Hkv, d, q, k, v, do = _case(1)
    drop = A.Dropout(0.3, 2024, 11, Hq)
    scale = 0.7

    def loss(q_, k_, v_):
        o, _ = A.forward(q_, k_, v_, layout, r0, scale, dropout=drop)
        return float((o * do).sum())

    dq, dk, dv = A.backward(q, k, v, do, layout, r0, scale, dropout=drop)
    eps = 1e-6
    rng = np.random.default_rng(3)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            fp = loss(**{**{"q_": args["q"], "k_": args["k"], "v_": args["v"]}, f"{name}_": xp})
            fm = loss(**{**{"q_": args["q"], "k_": args["k"], "v_": args["v"]}, f"{name}_": xm})
            num = (fp - fm) / (2 * eps)
            assert abs(num - g[idx]) <= 1e-6 * max(1.0, abs(num)), (name, idx, num, g[idx])


def test_backward_with_dropout_matches_torch_autograd():
    layout, S, r0, L, Hq, Hkv, d, q, k, v, do = _case(2)
    scale = 0.5
    drop = A.Dropout(0.25, 77, 3, Hq)
    G = Hq // Hkv
    M = torch.from_numpy(A.block_causal_mask(layout, S, r0, L))          # [B, L, S]
    Z = np.zeros((2, Hq, L, S))
    for b in range(2):
        for h in range(Hq):
            Z[b, h] = drop.keep(b, h, np.arange(L) + r0, np.arange(S))[0]
    c = DR.keep_scale(0.25)[1]
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kq = kt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)             # [B, Hq, S, d]
    vq = vt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    s = scale * qt.permute(0, 2, 1, 3) @ kq.transpose(-1, -2)           # [B, Hq, L, S]
    s = s.masked_fill(~M[:, None], float("-inf"))
    P = torch.softmax(s, dim=-1).nan_to_num(0.0)
    o = (P * torch.from_numpy(Z) * c) @ vq                                # [B, Hq, L, d]
    o = o.permute(0, 2, 1, 3)
    (o * torch.from_numpy(do)).sum().backward()
    o_ref, _ = A.forward(q, k, v, layout, r0, scale, dropout=drop)
    dq, dk, dv = A.backward(q, k, v, do, layout, r0, scale, dropout=drop)
    assert np.abs(o.detach().numpy() - o_ref).max() <= 1e-12
    for g_ref, g_t in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.abs(g_ref - g_t.numpy()).max() <= 1e-12


def test_dropout_masks_follow_row_positions():
    """Chunks of the row draw the same mask as the full call (O, LSE, dQ
    concatenate, dK / dV sum), and the runner's re-indexed jobs equal the
    direct call."""
    rng = np.random.default_rng(4)
    layout = ((30, 50, 20, 28), (64, 64))
    S, Hq, Hkv, d, scale = 128, 4, 2, 8, 0.4
    q = rng.standard_normal((2, S, Hq, d)); k = rng.standard_normal((2, S, Hkv, d))
    v = rng.standard_normal((2, S, Hkv, d)); do = rng.standard_normal((2, S, Hq, d))
    drop = A.Dropout(0.2, 31337, 9, Hq)
    o, lse = A.forward(q, k, v, layout, 0, scale, dropout=drop)
    dq, dk, dv = A.backward(q, k, v, do, layout, 0, scale, dropout=drop)
    dks, dvs = np.zeros_like(dk), np.zeros_like(dv)
    for a, e in ((0, 40), (40, 100), (100, 128)):
        oc, lc = A.forward(q[:, a:e], k, v, layout, a, scale, dropout=drop)
        qc, kc, vc = A.backward(q[:, a:e], k, v, do[:, a:e], layout, a, scale, dropout=drop)
        assert np.abs(oc - o[:, a:e]).max() <= 1e-12 and np.abs(qc - dq[:, a:e]).max() <= 1e-12
        fin = np.isfinite(lc)
        assert np.abs(lc[fin] - lse[:, :, a:e][fin]).max() <= 1e-12
        dks += kc; dvs += vc
    assert np.abs(dks - dk).max() <= 1e-12 and np.abs(dvs - dv).max() <= 1e-12
    got = parallel.run(q[:, 20:], k, v, do[:, 20:], layout, 20, scale, block_rows=16, workers=1, pieces=3,
                       dropout=(0.2, 31337, 9))
    o2, _ = A.forward(q[:, 20:], k, v, layout, 20, scale, dropout=drop)
    g2 = A.backward(q[:, 20:], k, v, do[:, 20:], layout, 20, scale, dropout=drop)
    assert np.abs(got["o"] - o2).max() <= 1e-12
    for name, ref in zip(("dq", "dk", "dv"), g2):
        assert np.abs(got[name] - ref).max() <= 1e-12, name
