"""The allocation-free backward entry point (blockdiag_attn_bwd_noalloc)
against blockdiag_attn_bwd, through the C ABI: two calls in a row on one
GPU, the second with a smaller input, each bit for bit equal to the
workspace entry point's result; and its size limit, rejected on the host
before anything is launched."""
import ctypes
import sys

import numpy as np
import pytest

import synthetic
from tests import helpers as H

gpu = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _call_both(w, t):
    import torch
    import packed_sequence_attention_amd as bd
    lib = bd.load_library()
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device="cuda")
    d = H.to_device(w, t)
    o, lse = bd.attn_fwd(d["q"], d["k"], d["v"], seg, w.scale)
    ref = bd.attn_bwd(d["q"], d["k"], d["v"], o, lse, d["do"], seg, w.scale)
    outs = [torch.full_like(d["q"], float("nan")), torch.full_like(d["k"], float("nan")),
            torch.full_like(d["v"], float("nan"))]
    dt = 0 if w.dtype == "f32" else 1
    st = torch.cuda.current_stream().cuda_stream
    code = lib.blockdiag_attn_bwd_noalloc(dt, w.batch, w.seq_len, w.row_offset, w.q_len, 0, w.seq_len, w.h_q, w.h_kv,
                                          w.head_dim, w.scale, None, d["q"].data_ptr(), d["k"].data_ptr(),
                                          d["v"].data_ptr(), o.data_ptr(), lse.data_ptr(), d["do"].data_ptr(),
                                          ctypes.byref(seg.desc), outs[0].data_ptr(), outs[1].data_ptr(),
                                          outs[2].data_ptr(), st)
    assert code == 0, lib.blockdiag_last_error()
    torch.cuda.synchronize()
    return ref, outs


@gpu
def test_noalloc_backward_matches_workspace_entry_point():
    cases = [
        # larger first, then a smaller input on the same GPU (the array keeps
        # the first call's contents)
        ("bf16", [[300, 200, 12, 500], [1024]], 1024, 0, 1024, 8, 2, 128),
        ("bf16", [[90, 40, 126]], 256, 32, 200, 4, 1, 64),
        ("f32", [[50, 70]], 128, 0, 120, 4, 2, 64),
    ]
    for i, (dtype, docs, S, r0, L, hq, hkv, d) in enumerate(cases):
        _log(f"no-alloc case {i}: {dtype} S={S} r0={r0} L={L} H={hq}/{hkv} d={d}")
        w, t = H.small_case(700 + i, dtype, docs, S, r0, L, hq, hkv, d)
        ref, got = _call_both(w, t)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert bool(torch_equal(a, b)), f"{name} differs from blockdiag_attn_bwd"


def torch_equal(a, b):
    import torch
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_noalloc_rejects_sizes_past_the_static_scratch():
    """Checked on the host before the device is touched (dummy pointers)."""
    import packed_sequence_attention_amd as bd
    lib = bd.load_library()
    cap = lib.blockdiag_noalloc_scratch_bytes()
    assert cap == 16 << 20
    rows = cap // 8  # row-statistics pairs that fit
    p = 16
    m = bd.MetaDesc()
    # batch * q_len * h_q = rows + 32 > rows
    q_len = rows // 32 + 1
    code = lib.blockdiag_attn_bwd_noalloc(1, 1, q_len, 0, q_len, 0, q_len, 32, 8, 128, 0.088, None, p, p, p, p, p, p,
                                          ctypes.byref(m), p, p, p, None)
    assert code == 4 and b"scratch" in lib.blockdiag_last_error()
