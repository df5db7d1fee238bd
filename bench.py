"""Benchmark of the block-diagonal packed attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
host segmentation of the document lengths (blockdiag_segment), the device
metadata build (blockdiag_meta_build_host with the table in the launch
arguments, or a pinned upload and blockdiag_meta_build for tables of more
than 126 segments), the forward (blockdiag_attn_fwd) and the backward
(blockdiag_attn_bwd).  Inputs are
resident in HBM before the timed region starts.

Metric: useful (unmasked-pair) attention TFLOP/s, counting 4*d*H_q FLOP per
allowed (query, key) pair for the forward and 2.5 times that for the
backward; `value` divides that by the whole step's wall time.  The default
workload is bf16 B=2, S=4096 per row, H_q=32, H_kv=8, d=128, lognormal
document lengths (median 512), row_offset 0.

Printed: one JSON line (rank 0), with
  roofline      the backward's main kernel: the short-document kernel
                (dQ, dK and dV in one pass; taken when no segment has more
                than 128 keys, bf16, head_dim 64 / 128) or else the dK/dV
                kernel (the dominant one of the tile kernels).  achieved =
                algorithmic FLOP per launch (short-document kernel: all
                five products, 10 * d FLOP per allowed pair and query head;
                dK/dV kernel: the four products S, dP, dV, dK, 8 * d -- dQ
                is credited to the dQ kernel and its recomputation of S and
                dP is not counted) / its mean duration from HIP events
                recorded around that kernel on its stream in ten of the
                timed steps (spread over the timed region), against the bf16
                dense matrix-core peak (the fp32 vector-ALU peak, bound
                "alu", for shapes on the generic kernels, e.g. the float32
                workload 1); where that kernel's FLOP per algorithmic byte
                is below the machine balance (short documents, e.g. the
                fragmented S=49152 workload) it is priced in GB/s against
                the 8 TB/s HBM peak instead (bound "hbm"); `traffic` from
                the committed rocprofv3 counter summary when it was taken on
                the current kernel source, else null;
  hbm           algorithmic bytes of the forward and backward entry points
                (each tensor touched once) and the HBM rate they imply;
  roofs_us      one step's lower bounds from the matrix-core, HBM and exp
                roofs next to the measured step;
  gpu_clock     the engine clock (MHz) read by clock probes launched right
                after each of ten extra steps; the peaks above assume
                2.4 GHz;
  flushed       (--flush-mib) the step timed with a buffer written before
                each one, so inputs come from HBM rather than L2 / the
                Infinity Cache;
  cpu_baseline  the fp64 oracle timed on this host's cores over a bounded
                sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz
PEAK_FP32_VALU_TFLOPS = 157.3  # 256 CU x 4 SIMD x 64 fp32 FLOP/clk x 2.4 GHz (vector ALU)
PEAK_HBM_GBS = 8000.0
# exp throughput: v_exp_f32 issues at quarter rate (8 clk per wave64
# instruction per SIMD, measured) -> 8 exp/clk/SIMD x 1024 SIMDs x 2.4 GHz
PEAK_EXP_PER_S = 1024 * 8 * 2.4e9
METRIC = "unmasked-pair attention TFLOP/s fwd+bwd (bf16, packed S=4k) and % MFMA peak"


def useful_pairs(seg):
    """Allowed (query, key) pairs per query head, from the segment table:
    segment rows t = 0..q-1 see t + (k - q) + 1 keys (bottom-right aligned),
    padding segments (k = 0) none."""
    total = 0
    for s in range(seg.n_seg):
        qn = int(seg.cu_q[s + 1] - seg.cu_q[s])
        kn = int(seg.cu_k[s + 1] - seg.cu_k[s])
        if kn > 0:
            total += qn * (kn - qn + 1) + qn * (qn - 1) // 2
    return total


class HipEvents:
    """Minimal hipEvent_t handling through the HIP runtime's C API."""

    # Timing-only events: recording one then skips the system-scope fence
    # (cache write-back and invalidate) that a default event performs, which
    # stalls the stream for microseconds between the kernels it brackets.
    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev.value

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def kernel_source_digest(name):
    """sha256 prefix of a kernel's source file followed by the shared device
    header every kernel includes (its reductions and helpers are part of the
    kernel's code)."""
    h = hashlib.sha256()
    for f in (name, "device_common.h"):
        h.update(open(os.path.join(ROOT, "packed_sequence_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, kernel_file, workload_tag):
    """HBM bytes per launch from profiles/<kernel>_<workload>_traffic.md when
    its recorded source digest matches the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_tag}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_d = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_d or not m_b or m_d.group(1) != kernel_source_digest(kernel_file):
        return None
    return float(m_b.group(1))


def observed_clock(bd, step, dev, reps=10, n_wg=64):
    """The engine clock while the hot path runs: after each of `reps`
    steps, a clock probe (blockdiag_clock_probe: n_wg one-wave workgroups,
    each spinning 20 us and counting engine cycles against the 100 MHz
    real-time counter) on the same stream, while the steps' load still
    holds the clock.  Returns the median, min and max over all probes (MHz)."""
    import numpy as np
    import torch
    out = torch.zeros(reps, 2 * n_wg, dtype=torch.int64, device=dev)
    for r in range(reps):
        step()
        bd.clock_probe(out[r], ticks=2000)
    torch.cuda.synchronize()
    c = out.view(-1, 2).cpu().numpy().astype(np.float64)
    mhz = c[:, 0] / c[:, 1] * 100.0
    return {"mhz_median": round(float(np.median(mhz)), 1), "mhz_min": round(float(mhz.min()), 1),
            "mhz_max": round(float(mhz.max()), 1), "probes": int(mhz.size),
            "source": "engine cycles / 100 MHz real-time ticks over 20 us, right after each of "
                      f"{reps} steps"}


def cpu_baseline(w, t, flops_per_pair, budget_s=10.0):
    """The fp64 oracle (windowed, unchanged) timed on this host: batch rows
    are run one after another (each row split into (K/V head, query-row
    range) sub-problems, forward and backward, in a pool of one worker
    process per allowed core -- capped by OMP_NUM_THREADS when set -- with
    one BLAS thread each) until the rows done so far have taken `budget_s`
    seconds or the whole workload is done."""
    import numpy as np
    from oracle import parallel
    from oracle import attention as A
    workers = parallel.default_workers()
    dt = 0.0
    flops = 0
    rows = 0
    for b in range(w.batch):
        sub = {k: np.ascontiguousarray(t[k][b:b + 1]) for k in ("q", "k", "v", "do")}
        t0 = time.perf_counter()
        parallel.run(sub["q"], sub["k"], sub["v"], sub["do"], w.doc_lens[b:b + 1], w.row_offset, w.scale,
                     block_rows=256, workers=workers)
        dt += time.perf_counter() - t0
        pairs = A.useful_pairs(w.doc_lens[b:b + 1], w.seq_len, w.row_offset, w.q_len)
        flops += flops_per_pair * w.h_q * pairs
        rows += 1
        if dt >= budget_s:
            break
    what = "the whole workload" if rows == w.batch else f"batch rows 0..{rows - 1} of {w.batch}"
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
            "host_cores": parallel.host_cores(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{what} (all {w.h_q} query heads), forward+backward, fp64 numpy windowed oracle, "
                      f"jobs of (K/V head, row range) on {workers} worker processes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="named workload 1..5 (default 2)")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="run the named workload's packing and head counts at this head_dim instead "
                         "(e.g. 256); not the headline configuration")
    ap.add_argument("--h-kv", type=int, default=None,
                    help="run the named workload's packing with this many K/V heads instead (e.g. 32 for "
                         "multi-head attention, 16 for GQA 2:1); not the headline configuration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the engine-clock reading")
    ap.add_argument("--whole-row", action="store_true",
                    help="pass K/V for the whole row instead of the chunk's K/V window")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="also time steps with a buffer of this many MiB written before each one "
                         "(evicts Q/K/V/dO from L2 and the Infinity Cache; e.g. 512)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (3 launches): a known-size "
                         "reference for HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU's share only: run it with --gpus 1 (the library holds the "
              "single-GPU kernels; the multi-GPU K/V exchange around them is not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import packed_sequence_attention_amd as bd
    import synthetic

    if not os.path.exists(bd.library_path()):
        from packed_sequence_attention_amd import build
        build.build_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synthetic.workload(args.workload)
    if args.head_dim is not None and args.head_dim != w.head_dim:
        w = synthetic.custom_workload(w.wid, w.dtype, w.doc_lens, w.seq_len, w.row_offset, w.q_len, w.h_q,
                                      w.h_kv, args.head_dim,
                                      name=w.name.replace(f"/{w.head_dim}", f"/{args.head_dim}"))
    if args.h_kv is not None and args.h_kv != w.h_kv:
        w = synthetic.custom_workload(w.wid, w.dtype, w.doc_lens, w.seq_len, w.row_offset, w.q_len, w.h_q,
                                      args.h_kv, w.head_dim, w.scale,
                                      name=w.name.replace(f"/{w.h_kv}/", f"/{args.h_kv}/"))
    t = synthetic.draw_tensors(w)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    d = {k: torch.from_numpy(v).to(dev, dt) for k, v in t.items()}
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    seg0 = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len)
    # K/V as a context-parallel rank holds them after the needed-only
    # exchange: keys [kv_begin, row_offset + q_len), kv_begin the first key
    # any row of the chunk attends rounded down to 64 (the whole row up to
    # the chunk's end when the chunk starts the row).  --whole-row keeps all
    # seq_len keys.
    if args.whole_row:
        kv_begin, kv_end = 0, w.seq_len
    else:
        # first key position attended in any batch row (non-padding segments)
        real = np.diff(seg0.cu_k) > 0
        pos = seg0.k_begin - (seg0.cu_q[:-1] // max(w.q_len, 1)) * w.seq_len
        kv_lo = int(pos[real].min()) if real.any() else w.row_offset
        kv_begin, kv_end = (kv_lo // 64) * 64, w.row_offset + w.q_len
    k = k[:, kv_begin:kv_end].contiguous()
    v = v[:, kv_begin:kv_end].contiguous()
    kv_len = kv_end - kv_begin
    pairs = useful_pairs(seg0)
    D, Hq = w.head_dim, w.h_q
    flops_fwd = 4 * D * Hq * pairs
    flops_bwd = 10 * D * Hq * pairs
    # Algorithmic HBM bytes (every tensor touched once): K and V are read
    # over the keys the chunk attends (W, the table's total key length over
    # the batch rows); dK and dV, outputs over the whole K/V buffer, are
    # written once (zeros at keys no row attends).
    e_sz = 4 if w.dtype == "f32" else 2
    rows = w.batch * w.q_len
    win = int(seg0.cu_k[seg0.n_seg])
    kv_keys = w.batch * kv_len
    bytes_fwd = 2 * e_sz * D * Hq * rows + 2 * e_sz * D * w.h_kv * win + 4 * Hq * rows
    bytes_bwd = 4 * e_sz * D * Hq * rows + 2 * e_sz * D * w.h_kv * (win + kv_keys) + 8 * Hq * rows
    exps = 2 * Hq * pairs  # one exp per allowed pair and query head, forward and backward
    ev = HipEvents()
    stream = torch.cuda.current_stream(dev)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * (1 << 20) // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Inside the timed steps only the dominant kernel (dK/dV) is bracketed by
    # events, and only in every k-th step (ten samples spread over the timed
    # region): every event recorded between two kernels adds a few
    # microseconds of stream idle time to its step.  The forward kernel is
    # timed in a separate loop below.
    def step(marks=None):
        seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device=dev)
        o, lse = bd.attn_fwd(q, k, v, seg, w.scale, kv_begin=kv_begin)
        if marks is not None:
            bd.mark_main_kernel(marks[0], marks[1])
        dq, dk, dv = bd.attn_bwd(q, k, v, o, lse, do, seg, w.scale, kv_begin=kv_begin)
        return o, dq

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    mark_every = max(1, args.steps // 10)
    marks = [[ev.create() for _ in range(2)] if i % mark_every == 0 else None for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(marks[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    marks = [m for m in marks if m is not None]
    bwd_ms = [ev.elapsed_ms(m[0], m[1]) for m in marks]
    for m in marks:
        for e in m:
            ev.destroy(e)
    bwd_avg = sum(bwd_ms) / len(bwd_ms)

    # kernel-only fwd+bwd entry-point times (events around each call), for the
    # fwd+bwd figure that excludes once-per-step metadata work
    # (plus the forward kernel alone, marked like the dK/dV kernel above)
    e = [ev.create() for _ in range(5)]
    seg = bd.segment(w.doc_lens, w.seq_len, w.row_offset, w.q_len, device=dev)
    times_f, times_b, fwd_ms = [], [], []
    for _ in range(max(5, args.steps // 2)):
        ev.record(e[0], stream)
        bd.mark_main_kernel(e[3], e[4])
        o, lse = bd.attn_fwd(q, k, v, seg, w.scale, kv_begin=kv_begin)
        ev.record(e[1], stream)
        bd.attn_bwd(q, k, v, o, lse, do, seg, w.scale, kv_begin=kv_begin)
        ev.record(e[2], stream)
        torch.cuda.synchronize()
        times_f.append(ev.elapsed_ms(e[0], e[1]))
        times_b.append(ev.elapsed_ms(e[1], e[2]))
        fwd_ms.append(ev.elapsed_ms(e[3], e[4]))
    for x in e:
        ev.destroy(x)
    tf = float(np.median(times_f))
    tb = float(np.median(times_b))
    fwd_avg = sum(fwd_ms) / len(fwd_ms)

    flushed = None
    if args.flush_mib > 0:
        buf = torch.empty(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        ef = [ev.create() for _ in range(2)]
        times = []
        for i in range(max(5, args.steps // 2)):
            buf.fill_(float(i))
            ev.record(ef[0], stream)
            step()
            ev.record(ef[1], stream)
            torch.cuda.synchronize()
            times.append(ev.elapsed_ms(ef[0], ef[1]))
        for x in ef:
            ev.destroy(x)
        del buf
        tfl = float(np.median(times))
        flushed = {"flush_mib": args.flush_mib, "ms_per_step": round(tfl, 4),
                   "tflops": round((flops_fwd + flops_bwd) / (tfl * 1e-3) / 1e12, 3),
                   "hbm_gbs": round((bytes_fwd + bytes_bwd) / (tfl * 1e-3) / 1e9, 1)}

    value = (flops_fwd + flops_bwd) / (ms_per_step * 1e-3) / 1e12
    # The kernel the events bracketed (the backward's main kernel): for
    # packings of short documents (bf16, head_dim 64 / 128, no segment of
    # more than 128 keys, at most 2047 segments) the short-document kernel,
    # which computes dQ, dK and dV in one pass; else a matrix-core dK/dV
    # kernel (bf16, head_dim 64 / 128 / 256, any GQA ratio); else the generic
    # vector-ALU kernel, priced against the fp32 vector peak.
    short_path = (w.dtype == "bf16" and D in (64, 128) and 0 <= seg0.max_k <= 128 and seg0.n_seg <= 2047)
    on_mfma = w.dtype == "bf16" and D in (64, 128, 256)
    if short_path:
        # all five products, each pair once: 10 * d FLOP per pair and head
        main_kernel, main_src, main_tag, bound, peak = "bwd_short_kernel", "bwd_short.hip", "bwd_short", "mfma", \
            PEAK_BF16_TFLOPS
        flops_main = 10 * D * Hq * pairs
        # Q, dO, O read and dQ written once, lse read; K, V read over the
        # attended keys; dK, dV written over the whole K/V buffer
        bytes_main = 4 * e_sz * D * Hq * rows + 2 * e_sz * D * w.h_kv * (win + kv_keys) + 4 * Hq * rows
    else:
        # the four products S, dP, dV, dK at 2 * d FLOP per pair and query
        # head each (the backward's fifth, dQ, is credited to the dQ kernel
        # and its recomputation of S and dP is not counted)
        if on_mfma:
            main_kernel, bound, peak = ("bwd_dkdv256_kernel" if D == 256 else "bwd_dkdv_kernel"), "mfma", \
                PEAK_BF16_TFLOPS
        else:
            main_kernel, bound, peak = "dkv_generic_kernel", "alu", PEAK_FP32_VALU_TFLOPS
        main_src, main_tag = "bwd_dkdv.h", "bwd_dkdv"
        flops_main = 8 * D * Hq * pairs
        # Q, dO and the row statistics read once, K, V read and dK, dV
        # written once over the windows
        bytes_main = 2 * e_sz * D * Hq * rows + 2 * e_sz * D * w.h_kv * (win + kv_keys) + 8 * Hq * rows
    achieved = flops_main / (bwd_avg * 1e-3) / 1e12
    # Below the machine balance (peak FLOP/s over 8 TB/s) the kernel is
    # priced against HBM instead (short documents: few pairs per byte).
    unit = "TFLOP/s"
    if flops_main / bytes_main < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        achieved = bytes_main / (bwd_avg * 1e-3) / 1e9
    base_w = synthetic.workload(args.workload)
    named = ((args.head_dim is None or args.head_dim == base_w.head_dim)
             and (args.h_kv is None or args.h_kv == base_w.h_kv))
    traffic = (traffic_from_profile(main_tag, main_src, f"w{args.workload}")
               if on_mfma and D != 256 and named else None)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "row_offset": w.row_offset,
                   "q_len": w.q_len, "kv_window": [kv_begin, kv_end], "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.head_dim,
                   "n_docs": w.n_docs, "useful_pairs_per_head": pairs, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_bwd_entry_ms": {"fwd": round(tf, 4), "bwd": round(tb, 4)},
        "tflops_fwd_plus_bwd_calls": round((flops_fwd + flops_bwd) / ((tf + tb) * 1e-3) / 1e12, 3),
        "main_kernel_ms": {"fwd": round(fwd_avg, 4), "bwd_main": round(bwd_avg, 4)},
        "fwd_kernel_tflops": round(flops_fwd / (fwd_avg * 1e-3) / 1e12, 3),
        # Algorithmic HBM bytes of each entry point and the rate they imply at
        # the entry points' event times, against the 8 TB/s HBM peak.
        "hbm": {"bytes_fwd": bytes_fwd, "bytes_bwd": bytes_bwd,
                "gbs_fwd": round(bytes_fwd / (tf * 1e-3) / 1e9, 1),
                "gbs_bwd": round(bytes_bwd / (tb * 1e-3) / 1e9, 1),
                "frac_fwd": round(bytes_fwd / (tf * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "frac_bwd": round(bytes_bwd / (tb * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        # Lower bounds on one step's time from each roof (us): useful FLOP at
        # the bf16 matrix-core peak, algorithmic bytes at 8 TB/s, one exp per
        # allowed pair and head per direction at the exp rate.
        "roofs_us": {"mfma": round((flops_fwd + flops_bwd) / (PEAK_BF16_TFLOPS * 1e12) * 1e6, 2),
                     "hbm": round((bytes_fwd + bytes_bwd) / (PEAK_HBM_GBS * 1e9) * 1e6, 2),
                     "exp": round(exps / PEAK_EXP_PER_S * 1e6, 2),
                     "step": round(ms_per_step * 1e3, 2)},
        "roofline": {"bound": bound, "kernel": main_kernel, "achieved": round(achieved, 3),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "algorithmic_flop": flops_main, "algorithmic_bytes": bytes_main,
                     "traffic": traffic, "launches_timed": len(bwd_ms)},
    }
    if flushed is not None:
        out["flushed"] = flushed
    if not args.no_clock:
        out["gpu_clock"] = observed_clock(bd, step, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, t, 14 * D)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
