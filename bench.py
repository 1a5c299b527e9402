"""Benchmark of the fused SDPA forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM:
  1. packed THD ragged causal prefill, bf16: 8 sequences with lengths uniform
     in [128, 4096], 32 Q heads / 8 KV heads, D = 128, packed FP32 LSE
     (sdpa_prefill_thd: one kernel);
  2. paged-KV decode, bf16: batch 64, one query token, 32 / 8 heads, D = 128,
     page size 64, KV lengths uniform in [512, 32768], independent randomly
     permuted K and V page tables, 8 KV splits merged by LSE
     (sdpa_decode_paged: the split kernel, then the combine kernel).

Reported: prefill attention TFLOP/s (visible (row, key) pairs x 2 (Dqk + Dv))
against the bf16 dense MFMA peak, and paged-decode KV GB/s against the HBM
peak, each from HIP events recorded on the launch stream around every call
of the timed steps.  Every timed region starts with at least 100 ms of the
same work, untimed, before its W warm-up steps, so the engine clock has left
its idle state (the CPU-baseline legs leave the GPU idle for seconds).  Beside them, the fp64 CPU oracle timed on a bounded
sample of the same workloads (``cpu_baseline``).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
Prints ONE JSON line on stdout.

``roofline.traffic`` (HBM bytes per launch of the kernel) comes from the
committed counter summary profiles/prefill_thd_d128_traffic.md (decode:
profiles/paged_decode_d128_traffic.md): rocprofv3
FETCH_SIZE and WRITE_SIZE of the kernel, each scaled by what the same counter
reads for a plain device copy of known size (``--calibrate-copy`` runs that
copy).  It is null when the kernel sources differ from the ones the counters
were taken on (SHA-1 of the sources recorded in the summary).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
# FP8 prefill runs S = K Q^T (half the flops) on the FP8 MFMA and P V on the
# bf16 MFMA: the time-weighted peak of that mix
PEAK_FP8_PREFILL_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_flops(lengths_q, lengths_kv, hq, dqk, dv, causal=True):
    """Visible (row, key) pairs x 2 (Dqk + Dv) x Hq (bottom-right causal)."""
    pairs = 0
    for lq, lk in zip(lengths_q, lengths_kv):
        for_rows = 0
        if causal:
            # row i sees min(lk, max(0, i + lk - lq + 1)) keys
            for_rows = sum(min(lk, max(0, i + lk - lq + 1)) for i in range(lq))
        else:
            for_rows = lq * lk
        pairs += for_rows
    return pairs * hq * 2 * (dqk + dv)


def decode_bytes(pc):
    """Compulsory HBM bytes of one paged decode call and its K/V share (FP8 cases: one
    byte per Q/K/V element, O still bf16)."""
    eb = 1 if pc.descale is not None else 2
    lens = [int(x) for x in pc.seq_lens.tolist()]
    dqk, dv = int(pc.q.shape[3]), int(pc.v_pool.shape[3])
    kv = sum(lens) * pc.hkv * (dqk + dv) * eb
    rows = pc.batch * pc.sq * pc.hq
    q = rows * dqk * eb
    o = rows * dv * 2
    lse = rows * 4
    pages = sum((L + pc.page_size - 1) // pc.page_size for L in lens)
    tables = 2 * pages * 4 + pc.batch * 4
    return kv, kv + q + o + lse + tables


PREFILL_SOURCES = ["scaled_dot_product_19_amd/csrc/prefill_bf16.hip",
                   "scaled_dot_product_19_amd/csrc/tile_ops.h",
                   "scaled_dot_product_19_amd/csrc/sdpa_device.h"]
DECODE_SOURCES = ["scaled_dot_product_19_amd/csrc/decode_small.hip",
                  "scaled_dot_product_19_amd/csrc/combine.hip",
                  "scaled_dot_product_19_amd/csrc/decode_paged.hip",
                  "scaled_dot_product_19_amd/csrc/sdpa_device.h"]
WIDE_SOURCES = ["scaled_dot_product_19_amd/csrc/decode_wide.hip",
                "scaled_dot_product_19_amd/csrc/combine.hip",
                "scaled_dot_product_19_amd/csrc/tile_ops.h",
                "scaled_dot_product_19_amd/csrc/sdpa_device.h"]
PREFILL_TRAFFIC = os.path.join(ROOT, "profiles", "prefill_thd_d128_traffic.md")
DECODE_TRAFFIC = os.path.join(ROOT, "profiles", "paged_decode_d128_traffic.md")
D256_TRAFFIC = os.path.join(ROOT, "profiles", "prefill_d256_traffic.md")
WIDE_TRAFFIC = os.path.join(ROOT, "profiles", "mla_decode_wide_traffic.md")


def sources_sha1(paths):
    import hashlib
    h = hashlib.sha1()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(summary, sources):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is missing or was taken on other kernel sources."""
    try:
        with open(summary) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line and line.split(":", 1)[0] in ("sources_sha1", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            vals[k] = v.strip().split()[0].strip("`")
    if vals.get("sources_sha1") != sources_sha1(sources):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def calibrate_copy(nbytes):
    """One plain device-to-device copy of nbytes (the FETCH_SIZE / WRITE_SIZE
    reference under rocprofv3 --pmc)."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes}), flush=True)


def host_threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline_prefill(case, target_s, threads):
    """The oracle on a random sample of (token, head) rows; TFLOP/s of the sample."""
    import numpy as np
    import oracle
    from scaled_dot_product_19_amd import inputs
    cu = case.cu_q.numpy()
    T = int(cu[-1])
    rng = np.random.default_rng(7)
    qa, ka, va = inputs.host_array(case.q), inputs.host_array(case.k), inputs.host_array(case.v)

    def run(n):
        toks = rng.integers(0, T, size=n).astype(np.int64)
        heads = rng.integers(0, case.hq, size=n).astype(np.int32)
        b = np.searchsorted(cu, toks, side="right") - 1
        i = toks - cu[b]
        vis = (i + 1).astype(np.float64)  # causal, Lq == Lk
        flops = float(vis.sum()) * 2 * (case.q.shape[2] + case.v.shape[2])
        t0 = time.perf_counter()
        oracle.prefill_thd(qa, ka, va, case.cu_q.numpy(), case.cu_kv.numpy(), case.scale, True,
                           sel_tok=toks, sel_head=heads, nthreads=threads)
        return flops, time.perf_counter() - t0

    f, dt = run(8 * threads)
    n = int(max(8 * threads, min(200000, 8 * threads * target_s / max(dt, 1e-3))))
    f, dt = run(n)
    return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d random (token, head) rows of the %s workload, fp64, %.1f s"
                      % (n, case.name, dt)}


def cpu_baseline_decode(pc, target_s, threads):
    """The oracle on random (sequence, KV head) units, all their query rows; KV GB/s."""
    import numpy as np
    import oracle
    from scaled_dot_product_19_amd import inputs
    rng = np.random.default_rng(11)
    G = pc.hq // pc.hkv
    lens = pc.seq_lens.numpy()
    dqk, dv = int(pc.q.shape[3]), int(pc.v_pool.shape[3])
    qa, ka, va = (inputs.host_array(pc.q), inputs.host_array(pc.k_pool),
                  inputs.host_array(pc.v_pool))

    def run(n_units):
        bs = rng.integers(0, pc.batch, size=n_units)
        kvs = rng.integers(0, pc.hkv, size=n_units)
        rows = []
        for b, kvh in zip(bs, kvs):
            for t in range(pc.sq):
                for h in range(kvh * G, (kvh + 1) * G):
                    rows.append((int(b) * pc.sq + t) * pc.hq + h)
        kv_bytes = float(sum(int(lens[b]) for b in bs)) * (dqk + dv) * 2
        t0 = time.perf_counter()
        oracle.decode_paged(qa, ka, va, pc.pt_k.numpy(), pc.pt_v.numpy(), lens, pc.page_size,
                            pc.scale, pc.causal, num_splits=pc.num_splits,
                            sel_rows=np.array(rows, dtype=np.int64), nthreads=threads)
        return kv_bytes, time.perf_counter() - t0, len(rows)

    by, dt, _ = run(max(2, threads // G))
    n = int(max(2, min(pc.batch * pc.hkv * 4, max(2, threads // G) * target_s / max(dt, 1e-3))))
    by, dt, nrows = run(n)
    return {"value": by / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d random (sequence, KV head) units (%d query rows) of the %s workload, "
                      "%d-way split + LSE merge, fp64, %.1f s"
                      % (n, nrows, pc.name, pc.num_splits, dt)}


def window_prefill_flops(lengths_q, lengths_kv, hq, dqk, dv, causal, window):
    """Visible (row, key) pairs x 2 (Dqk + Dv) x Hq with a left window W: row i of a
    sequence (Lq, Lk) sees keys max(0, d - W + 1) .. min(Lk, d + 1) - 1 (causal) or
    .. Lk - 1, d = i + Lk - Lq."""
    import numpy as np
    pairs = 0
    for lq, lk in zip(lengths_q, lengths_kv):
        d = np.arange(lq, dtype=np.int64) + (lk - lq)
        j1 = np.minimum(lk, d + 1) if causal else np.full(lq, lk, dtype=np.int64)
        j0 = np.maximum(0, d - window + 1) if window > 0 else np.zeros(lq, dtype=np.int64)
        pairs += int(np.maximum(0, j1 - j0).sum())
    return pairs * hq * 2 * (dqk + dv)


def run_window_prefill(args, torch, inputs, sdpa, dev):
    """Sliding-window prefill with sinks, base-2 head-major Stats: one sdpa_prefill_thd_ex
    call per step, on the D=128 prefill workload (W = 1024) and on a 64/8-head D=64 one
    (W = 128).  One JSON line each."""
    for case, window, dk in ((inputs.thd_prefill_d128(), 1024, 128),
                             (inputs.window_prefill_d64(), 128, 64)):
        q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
        cu_q, cu_kv = case.cu_q.to(dev), case.cu_kv.to(dev)
        sinks = inputs.sink_logits(inputs.SEED_BASE + 9, case.hq, special=False).to(dev)
        T = int(case.cu_q[-1])
        o = torch.empty((T, case.hq, dk), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((case.hq, T), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()

        def step():
            sdpa.prefill_thd_ex(q, k, v, cu_q, cu_kv, case.max_q, case.max_kv, case.scale, True,
                                window_left=window, sinks=sinks, out=o, lse=lse,
                                lse_layout=sdpa.LSE_HEAD_MAJOR, lse_s_max=T, stats_log2=True,
                                stream=stream)

        prewarm(torch, step)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        flops = window_prefill_flops(case.lengths_q, case.lengths_kv, case.hq, dk, dk, True,
                                     window)
        tflops = flops / (ms * 1e-3) / 1e12
        kern = "prefill_bf16_kernel<%d, %d, 4, 8, true, false, false>" % (dk, 64 if dk == 128
                                                                           else 128)
        line = {"metric": "sliding-window prefill attn TFLOP/s (% MFMA peak)",
                "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded N(0,1) bf16; lengths and sinks per seed)",
                "config": {"workload": case.name + "_w%d_sinks_log2_headmajor" % window,
                           "window": window, "lengths": case.lengths_q, "flop": flops},
                "roofline": {"kernel": kern, "bound": "mfma", "achieved": round(tflops, 2),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None}}
        print(json.dumps(line), flush=True)


def chunked_prefill_flops(pc):
    """Visible (row, key) pairs x 2 (D_qk + D_v): token i of a chunk of s_q tokens at the end of
    a cache of L tokens sees keys 0 .. L - s_q + i."""
    pairs = 0
    for L in pc.seq_lens.tolist():
        first = L - pc.sq + 1  # keys seen by token 0
        for i in range(pc.sq):
            pairs += max(0, min(L, first + i))
    return 2.0 * (128 + 128) * pairs * pc.hq


def run_chunked_prefill(args, torch, inputs, sdpa, dev):
    """Chunked prefill over the paged cache: one sdpa_decode_paged call per step (the
    prefill kernel over the page tables, plus the LSE combine when splits > 1)."""
    pc = inputs.chunked_prefill_paged(num_splits=args.splits)
    q, kp, vp = pc.q.to(dev), pc.k_pool.to(dev), pc.v_pool.to(dev)
    ptk, ptv, sl = pc.pt_k.to(dev), pc.pt_v.to(dev), pc.seq_lens.to(dev)
    o = torch.empty((pc.batch, pc.sq, pc.hq, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((pc.batch, pc.sq, pc.hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq, 128,
                                                        pc.num_splits)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        sdpa.decode_paged(q, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, pc.causal,
                          num_splits=pc.num_splits, workspace=ws, out=o, lse=lse, stream=stream)

    prewarm(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    flops = chunked_prefill_flops(pc)
    tflops = flops / (ms * 1e-3) / 1e12
    line = {"metric": "chunked prefill attn TFLOP/s (% MFMA peak)", "value": round(tflops, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16; cache lengths, page permutations per seed)",
            "config": {"workload": pc.name, "chunk": pc.sq, "cache_lengths": pc.seq_lens.tolist(),
                       "splits": pc.num_splits, "flop": flops},
            "roofline": {"kernel": "prefill_bf16_kernel<128, 64, 4, 8, true, false, true, false>"
                                   + (" + combine_kernel<false>" if pc.num_splits > 1 else ""),
                         "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": None}}
    print(json.dumps(line), flush=True)


def context_leg(args, torch, inputs, sdpa, dev, stream):
    """The context phase of serving: chunked prefill of 512- and 1024-token chunks against
    64k and 128k caches (batch 2, bottom-right causal), one sdpa_decode_paged call each (the
    prefill kernel over the page tables plus the LSE combine)."""
    res = []
    for chunk, cache in ((512, 65536), (1024, 65536), (512, 131072), (1024, 131072)):
        pc = inputs.context_chunk(chunk, cache)
        q, kp, vp = pc.q.to(dev), pc.k_pool.to(dev), pc.v_pool.to(dev)
        ptk, ptv, sl = pc.pt_k.to(dev), pc.pt_v.to(dev), pc.seq_lens.to(dev)
        o = torch.empty((pc.batch, pc.sq, pc.hq, 128), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((pc.batch, pc.sq, pc.hq), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq, 128,
                                                            pc.num_splits)),
                         dtype=torch.uint8, device=dev)

        def call():
            sdpa.decode_paged(q, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, pc.causal,
                              num_splits=pc.num_splits, workspace=ws, out=o, lse=lse,
                              stream=stream)

        st = ms_stats(per_call_ms(torch, stream, call, args.steps, args.warmup))
        flops = chunked_prefill_flops(pc)
        tf = flops / (st["mean"] * 1e-3) / 1e12
        log("%s: %.4f ms mean (median %.4f, min %.4f) -> %.1f TFLOP/s (%.1f%% of bf16 peak)"
            % (pc.name, st["mean"], st["median"], st["min"], tf, 100 * tf / PEAK_BF16_TFLOPS))
        res.append({"workload": pc.name, "chunk": chunk, "cache": cache,
                    "splits": pc.num_splits, "flop": flops, "ms": st, "value": round(tf, 2),
                    "unit": "TFLOP/s",
                    "roofline": {"kernel": "prefill_bf16_kernel<128, 64, 4, 8, true, false, "
                                           "true, false> + combine_kernel<false>",
                                 "bound": "mfma", "achieved": round(tf, 2),
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None}})
        del q, kp, vp, ws
        torch.cuda.empty_cache()
    return res


def per_call_ms(torch, stream, call, steps, warmup, between=None):
    """Milliseconds of each of `steps` calls, from HIP events recorded on `stream` right
    before and after the call (after `warmup` untimed calls).  `between()` runs before
    every call, outside its events (e.g. a cache flush)."""
    if between is None:
        prewarm(torch, call)
    else:
        prewarm(torch, lambda: (between(), call()))
    for _ in range(warmup):
        if between is not None:
            between()
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        if between is not None:
            between()
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def ms_stats(ms):
    """mean / median / min of per-call milliseconds."""
    srt = sorted(ms)
    n = len(srt)
    med = srt[n // 2] if n % 2 else 0.5 * (srt[n // 2 - 1] + srt[n // 2])
    return {"mean": round(sum(ms) / n, 4), "median": round(med, 4), "min": round(srt[0], 4)}


MALL_FLUSH_BYTES = 512 << 20  # twice the 256 MiB MALL

PREWARM_MS = 100.0  # untimed back-to-back work before every timed region
PREWARM_CALLS = []  # calls each pre-warm made, in the order of the timed regions


def prewarm(torch, call, min_ms=PREWARM_MS):
    """Run `call` back to back, untimed, for at least `min_ms` of wall time before the
    warm-up steps.  After an idle gap (the CPU-baseline legs leave the GPU idle for seconds)
    the engine clock takes tens of milliseconds of load to settle: on an MI355X the MLA
    decode call ran 0.32 ms over its first 15 ms of back-to-back calls after 2 s idle and
    0.274 ms from about 30 ms on."""
    t0 = time.perf_counter()
    n = 0
    while True:
        call()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= min_ms:
                PREWARM_CALLS.append(n)  # lets a kernel trace find the timed launches
                return


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_decode(torch, sdpa, pc, dev, steps, warmup, q=None, kp=None, vp=None):
    """Average ms of one sdpa_decode_paged call (split kernel + combine) over `steps`."""
    q = pc.q.to(dev) if q is None else q
    kp = pc.k_pool.to(dev) if kp is None else kp
    vp = pc.v_pool.to(dev) if vp is None else vp
    ptk, ptv, sl = pc.pt_k.to(dev), pc.pt_v.to(dev), pc.seq_lens.to(dev)
    dv = int(vp.shape[3])
    o = torch.empty((pc.batch, int(q.shape[1]), pc.hq, dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((pc.batch, int(q.shape[1]), pc.hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, sdpa.decode_workspace_bytes(pc.batch, int(q.shape[1]), pc.hq, dv,
                                                        pc.num_splits)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        sdpa.decode_paged(q, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, pc.causal,
                          num_splits=pc.num_splits, workspace=ws, out=o, lse=lse, stream=stream)

    prewarm(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_decode_fp8(torch, sdpa, pc, dev, steps, warmup):
    """Average ms of one sdpa_decode_paged_fp8 call (split kernel + combine) over `steps`."""
    q, kp, vp = pc.q.to(dev), pc.k_pool.to(dev), pc.v_pool.to(dev)
    ptk, ptv, sl = pc.pt_k.to(dev), pc.pt_v.to(dev), pc.seq_lens.to(dev)
    dq, dk, dv = (torch.tensor([x], dtype=torch.float32, device=dev) for x in pc.descale)
    d = int(vp.shape[3])
    o = torch.empty((pc.batch, pc.sq, pc.hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((pc.batch, pc.sq, pc.hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq, d,
                                                        pc.num_splits)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        sdpa.decode_paged_fp8(q, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, dq, dk, dv,
                              causal=pc.causal, num_splits=pc.num_splits, workspace=ws, out=o,
                              lse=lse, stream=stream)

    prewarm(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def run_decode_variant(args, torch, inputs, sdpa, dev):
    """--mtp-sweep: q_tokens 1..4 over the same 128k caches; --mla-aliased: the MLA-shaped
    decode with V aliased into the K rows.  K/V bytes count each live cache row once (for the
    aliased cache: the 576-wide K row, which holds V)."""
    peak = PEAK_HBM_GBS
    if args.fp8_decode:
        # the paged decode workload in per-tensor FP8, and in bf16 on the same GPU
        pc = inputs.paged_decode_d128_fp8()
        ms = time_decode_fp8(torch, sdpa, pc, dev, args.steps, args.warmup)
        kv, _ = decode_bytes(pc)
        name = pc.name
        del pc
        pcb = inputs.paged_decode_d128()
        ms_bf16 = time_decode(torch, sdpa, pcb, dev, args.steps, args.warmup)
        gbs = kv / ms / 1e6
        tokens = int(pcb.seq_lens.sum())
        line = {"metric": "FP8 paged decode KV GB/s (% HBM peak)", "value": round(gbs, 1),
                "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "fp8_e4m3",
                "data": "synthetic (seeded N(0,1) fp32 quantized per tensor to E4M3)",
                "config": {"workload": name, "kv_bytes": kv, "splits": 8,
                           "cached_tokens": tokens,
                           "bf16_ms_same_gpu": round(ms_bf16, 4),
                           "speedup_vs_bf16": round(ms_bf16 / ms, 3)},
                "roofline": {"kernel": "decode_small_kernel<128, true, 128> + combine_kernel<false>",
                             "bound": "hbm", "achieved": round(gbs, 1), "peak": peak,
                             "unit": "GB/s", "frac": round(gbs / peak, 4), "traffic": None}}
    elif args.fp8_mla:
        # the MLA-shaped decode in per-tensor FP8, and in bf16 on the same GPU
        pc = inputs.mla_decode_fp8()
        ms = time_decode_fp8(torch, sdpa, pc, dev, args.steps, args.warmup)
        kv, _ = decode_bytes(pc)
        name = pc.name
        del pc
        pcb = inputs.mla_decode()
        ms_bf16 = time_decode(torch, sdpa, pcb, dev, args.steps, args.warmup)
        gbs = kv / ms / 1e6
        line = {"metric": "FP8 MLA-shaped decode KV GB/s (% HBM peak)", "value": round(gbs, 1),
                "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "fp8_e4m3",
                "data": "synthetic (seeded N(0,1) fp32 quantized per tensor to E4M3)",
                "config": {"workload": name, "kv_bytes": kv, "splits": 16,
                           "bf16_ms_same_gpu": round(ms_bf16, 4),
                           "speedup_vs_bf16": round(ms_bf16 / ms, 3)},
                "roofline": {"kernel": "decode_wide_kernel<576, 512, false, true, 4> + combine_kernel<false>",
                             "bound": "hbm", "achieved": round(gbs, 1), "peak": peak,
                             "unit": "GB/s", "frac": round(gbs / peak, 4), "traffic": None}}
    elif args.mtp_sweep or args.gqa_mtp_sweep:
        # q_tokens 1..4 (4..16 rows per KV head: the few-row kernel), or 8 / 16 / 32 (32 / 64
        # / 128 rows: the prefill kernel with folded rows)
        wide = args.gqa_mtp_sweep
        pc = inputs.mtp_decode_d128(q_tokens=32 if wide else 4)
        kp, vp, q4 = pc.k_pool.to(dev), pc.v_pool.to(dev), pc.q.to(dev)
        kv, _ = decode_bytes(pc)
        res = []
        for qt in ((8, 16, 32) if wide else (1, 2, 3, 4)):
            ms = time_decode(torch, sdpa, pc, dev, args.steps, args.warmup,
                             q=q4[:, :qt].contiguous(), kp=kp, vp=vp)
            res.append({"q_tokens": qt, "ms": round(ms, 4), "kv_gbs": round(kv / ms / 1e6, 1),
                        "frac_hbm": round(kv / ms / 1e6 / peak, 4)})
        line = {"metric": "multi-token decode KV GB/s (% HBM peak), q_tokens "
                          + ("8, 16, 32" if wide else "1..4"),
                "value": res[0]["kv_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16)",
                "config": {"workload": pc.name.replace("_q32_", "_q8-32_").replace("_q4_", "_q1-4_"),
                           "kv_bytes": kv, "splits": pc.num_splits},
                "sweep": res}
    else:
        pc = inputs.mla_decode_aliased()
        kp = pc.k_pool.to(dev)
        lens = [int(x) for x in pc.seq_lens.tolist()]
        kv = sum(lens) * pc.hkv * 576 * 2  # one 576-wide row per live token holds K and V
        ms = time_decode(torch, sdpa, pc, dev, args.steps, args.warmup, kp=kp, vp=kp[..., :512])
        gbs = kv / ms / 1e6
        line = {"metric": "aliased-MLA decode KV GB/s (% HBM peak)", "value": round(gbs, 1),
                "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16)",
                "config": {"workload": pc.name, "kv_bytes": kv, "splits": pc.num_splits},
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": peak,
                             "unit": "GB/s", "frac": round(gbs / peak, 4), "traffic": None}}
    print(json.dumps(line), flush=True)


def time_prefill(torch, steps, warmup, call):
    """Average ms of `call` (one prefill launch) over `steps` back-to-back launches."""
    prewarm(torch, call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def run_fp8_prefill(args, torch, inputs, sdpa, dev):
    """--fp8-prefill: the THD prefill workload (same seed, lengths and fp32 draws) in
    per-tensor FP8 E4M3, and the bf16 workload on the same GPU."""
    case = inputs.thd_prefill_d128()
    c8 = inputs.fp8_thd_case(inputs.SEED_BASE + 2, hq=32, hkv=8, d=128, batch=8, lo=128,
                             hi=4096, name=case.name.replace("bf16", "fp8"))
    assert c8.lengths_q == case.lengths_q
    stream = torch.cuda.current_stream()
    T = int(case.cu_q[-1])
    cu_q, cu_kv = case.cu_q.to(dev), case.cu_kv.to(dev)
    o = torch.empty((T, case.hq, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, case.hq), dtype=torch.float32, device=dev)
    q8, k8, v8 = c8.q.to(dev), c8.k.to(dev), c8.v.to(dev)
    dq, dk, dv = (torch.tensor([x], dtype=torch.float32, device=dev) for x in c8.descale)
    ms8 = time_prefill(torch, args.steps, args.warmup, lambda: sdpa.prefill_thd_fp8(
        q8, k8, v8, cu_q, cu_kv, case.max_q, case.max_kv, case.scale, dq, dk, dv, True,
        out=o, lse=lse, lse_layout=sdpa.LSE_PACKED, stream=stream))
    del q8, k8, v8
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    ms16 = time_prefill(torch, args.steps, args.warmup, lambda: sdpa.prefill_thd(
        q, k, v, cu_q, cu_kv, case.max_q, case.max_kv, case.scale, True, out=o, lse=lse,
        lse_layout=sdpa.LSE_PACKED, stream=stream))
    flops = prefill_flops(case.lengths_q, case.lengths_kv, case.hq, 128, 128)
    tf = flops / (ms8 * 1e-3) / 1e12
    line = {"metric": "FP8 prefill attn TFLOP/s (% of the FP8-QK / bf16-PV MFMA peak)",
            "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms8, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
            "data": "synthetic (seeded N(0,1) fp32 quantized per tensor to E4M3)",
            "config": {"workload": c8.name, "prefill_lengths": case.lengths_q, "flop": flops,
                       "bf16_ms_same_gpu": round(ms16, 4),
                       "speedup_vs_bf16": round(ms16 / ms8, 3)},
            "roofline": {"kernel": "prefill_bf16_kernel<128, 64, 4, 8, true, false, false, true>",
                         "bound": "mfma", "achieved": round(tf, 2),
                         "peak": round(PEAK_FP8_PREFILL_TFLOPS, 1), "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_PREFILL_TFLOPS, 4),
                         "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None}}
    print(json.dumps(line), flush=True)


def decode_visible_pairs(lens, sq, causal):
    """(token, key) pairs a paged decode computes per query head: token t of a sequence of
    length L sits at key position L - sq + t and sees keys 0 .. L - sq + t (causal) or all
    L keys."""
    pairs = 0
    for L in lens:
        for t in range(sq):
            pairs += max(0, min(L, L - sq + t + 1)) if causal else L
    return pairs


def d256_leg(args, torch, inputs, sdpa, dev, stream, threads, ragged):
    """The D = 256 prefill workload (dense 2 x 8192 or ragged {8192, 3000}, 24/2 heads,
    padded [2, 8192, 24] LSE seeded -inf by the call): per-call HIP events around
    sdpa_prefill_thd (the -inf fill and the prefill kernel)."""
    case = inputs.ragged_prefill_d256() if ragged else inputs.dense_prefill_d256()
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    cu_q, cu_kv = case.cu_q.to(dev), case.cu_kv.to(dev)
    T = int(case.cu_q[-1])
    o = torch.empty((T, case.hq, 256), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((2, 8192, case.hq), dtype=torch.float32, device=dev)

    def call():
        sdpa.prefill_thd(q, k, v, cu_q, cu_kv, case.max_q, case.max_kv, case.scale, True, out=o,
                         lse=lse, lse_layout=sdpa.LSE_PADDED, lse_s_max=8192, stream=stream)

    ms = per_call_ms(torch, stream, call, args.steps, args.warmup)
    st = ms_stats(ms)
    flops = prefill_flops(case.lengths_q, case.lengths_kv, case.hq, 256, 256)
    tf = flops / (st["mean"] * 1e-3) / 1e12
    log("%s: %.4f ms mean (median %.4f, min %.4f) -> %.1f TFLOP/s (%.1f%% of bf16 peak)"
        % (case.name, st["mean"], st["median"], st["min"], tf, 100 * tf / PEAK_BF16_TFLOPS))
    leg = {"workload": case.name, "lengths": case.lengths_q, "flop": flops, "ms": st,
           "value": round(tf, 2), "unit": "TFLOP/s",
           "roofline": {"kernel": "prefill_bf16_kernel<256, 32, 4, 4, false, false, false, false>",
                        "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        # counters were taken on the dense workload
                        "traffic": None if ragged else recorded_traffic(D256_TRAFFIC,
                                                                        PREFILL_SOURCES)}}
    del q, k, v, o
    if not args.no_cpu_baseline:
        leg["cpu_baseline"] = cpu_baseline_prefill(case, args.cpu_seconds / 2, threads)
        log("  oracle: %.3g TFLOP/s (%s)" % (leg["cpu_baseline"]["value"],
                                            leg["cpu_baseline"]["sample"]))
    return leg


def mla_leg(args, torch, inputs, sdpa, dev, stream, threads):
    """The absorbed-MLA-shaped decode (576/512, 128/1 heads, 2 tokens, B = 32, 16 splits):
    per-call HIP events around sdpa_decode_paged (the wide split kernel and the combine)."""
    pc = inputs.mla_decode()
    q, kp, vp = pc.q.to(dev), pc.k_pool.to(dev), pc.v_pool.to(dev)
    ptk, ptv, sl = pc.pt_k.to(dev), pc.pt_v.to(dev), pc.seq_lens.to(dev)
    o = torch.empty((pc.batch, pc.sq, pc.hq, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((pc.batch, pc.sq, pc.hq), dtype=torch.float32, device=dev)
    ws = torch.empty(sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq, 512, pc.num_splits),
                     dtype=torch.uint8, device=dev)

    def call():
        sdpa.decode_paged(q, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, pc.causal,
                          num_splits=pc.num_splits, workspace=ws, out=o, lse=lse, stream=stream)

    ms = per_call_ms(torch, stream, call, args.steps, args.warmup)
    st = ms_stats(ms)
    kv, comp = decode_bytes(pc)
    lens = [int(x) for x in pc.seq_lens.tolist()]
    flops = decode_visible_pairs(lens, pc.sq, pc.causal) * pc.hq * 2 * (576 + 512)
    gbs = comp / (st["mean"] * 1e-3) / 1e9
    tf = flops / (st["mean"] * 1e-3) / 1e12
    rows = pc.batch * pc.sq * pc.hq
    # the library gives `merge` adjacent chunks to one work-group when the chunks would
    # make more than two work-groups per CU; the other slots of a group hold an empty
    # partial (its LSE only).  fp32 partials written + read back:
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    n_rb = (pc.sq * (pc.hq // pc.hkv) + 127) // 128
    merge = max(1, min(pc.num_splits, pc.batch * pc.hkv * pc.num_splits * n_rb // (2 * n_cu)))
    slots = (pc.num_splits + merge - 1) // merge
    part_bytes = 2 * rows * (slots * 512 + pc.num_splits) * 4
    log("%s: %.4f ms mean (median %.4f, min %.4f) -> %.1f GB/s compulsory (%.1f%% of HBM), "
        "%.1f TFLOP/s (%.1f%% of bf16 MFMA)" % (pc.name, st["mean"], st["median"], st["min"], gbs,
                                                 100 * gbs / PEAK_HBM_GBS, tf,
                                                 100 * tf / PEAK_BF16_TFLOPS))
    leg = {"workload": pc.name, "kv_bytes": kv, "compulsory_bytes": comp,
           "split_partial_bytes": part_bytes, "chunks_per_work_group": merge, "flop": flops, "ms": st,
           "value": round(kv / (st["mean"] * 1e-3) / 1e9, 1), "unit": "GB/s",
           "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
           "roofline": {"kernel": "decode_wide_kernel<576, 512, false, false, 4> + combine_kernel<false>",
                        "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": recorded_traffic(WIDE_TRAFFIC, WIDE_SOURCES)}}
    del q, kp, vp
    if not args.no_cpu_baseline:
        leg["cpu_baseline"] = cpu_baseline_decode(pc, args.cpu_seconds / 2, threads)
        log("  oracle: %.3g GB/s (%s)" % (leg["cpu_baseline"]["value"],
                                         leg["cpu_baseline"]["sample"]))
    return leg


def tiny_leg(args, torch, inputs, sdpa, dev, stream, threads):
    """The tiny fp32 THD workload ({5, 17}, 2/1 heads, D = 64): the oracle's CPU seconds on
    one thread and on `threads`, and the GPU call for context."""
    import oracle
    case = inputs.tiny_fp32()
    qa, ka, va = (inputs.host_array(case.q), inputs.host_array(case.k),
                  inputs.host_array(case.v))
    res = {"workload": case.name, "flop": prefill_flops(case.lengths_q, case.lengths_kv,
                                                        case.hq, 64, 64)}
    for key, n in (("oracle_s_1_thread", 1), ("oracle_s_all_threads", threads)):
        oracle.prefill_thd(qa, ka, va, case.cu_q.numpy(), case.cu_kv.numpy(), case.scale, True,
                           nthreads=n)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            oracle.prefill_thd(qa, ka, va, case.cu_q.numpy(), case.cu_kv.numpy(), case.scale,
                               True, nthreads=n)
            reps += 1
        res[key] = (time.perf_counter() - t0) / reps
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    cu_q, cu_kv = case.cu_q.to(dev), case.cu_kv.to(dev)
    o = torch.empty((22, 2, 64), dtype=torch.float32, device=dev)
    lse = torch.empty((22, 2), dtype=torch.float32, device=dev)

    def call():
        sdpa.prefill_thd(q, k, v, cu_q, cu_kv, case.max_q, case.max_kv, case.scale, True, out=o,
                         lse=lse, stream=stream)

    res["gpu_ms"] = ms_stats(per_call_ms(torch, stream, call, args.steps, args.warmup))
    res["cores"] = threads
    log("%s: oracle %.3g s (1 thread), %.3g s (%d threads); GPU %.4f ms"
        % (case.name, res["oracle_s_1_thread"], res["oracle_s_all_threads"], threads,
           res["gpu_ms"]["median"]))
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU seconds of each oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one device copy of BYTES (counter calibration)")
    ap.add_argument("--chunked-prefill", action="store_true",
                    help="time only chunked prefill over the paged cache (2 x 1024-token chunks, "
                         "caches U[32768, 65536], 32/8 heads, D=128, page 64) and print its line")
    ap.add_argument("--splits", type=int, default=4, help="num_splits of --chunked-prefill")
    ap.add_argument("--mtp-sweep", action="store_true",
                    help="time only multi-token decode, q_tokens 1..4 against 128k caches "
                         "(batch 4, 32/8 heads, D=128, page 64, 32 splits)")
    ap.add_argument("--window-prefill", action="store_true",
                    help="time only sliding-window prefill with sinks and base-2 head-major "
                         "Stats (D=128 workload with W=1024; 64/8 heads D=64 with W=128)")
    ap.add_argument("--fp8-decode", action="store_true",
                    help="time only the paged decode workload in per-tensor FP8 E4M3 (and in "
                         "bf16 on the same GPU for the ratio)")
    ap.add_argument("--fp8-mla", action="store_true",
                    help="the MLA-shaped decode in per-tensor FP8 (wide kernel), bf16 beside it")
    ap.add_argument("--gqa-mtp-sweep", action="store_true",
                    help="multi-token decode with 8 / 16 / 32 tokens (32-128 rows per KV head)")
    ap.add_argument("--fp8-prefill", action="store_true",
                    help="time only the THD prefill workload in per-tensor FP8 E4M3 (and in "
                         "bf16 on the same GPU)")
    ap.add_argument("--legs", default="c4,c5,c1,ctx",
                    help="extra workloads timed after the step, comma-separated from c4 (D=256 "
                         "dense and ragged prefill), c5 (absorbed-MLA-shaped decode), c1 (tiny "
                         "fp32: oracle CPU seconds), ctx (context phase: 512/1024-token chunks "
                         "against 64k/128k caches); empty for none")
    ap.add_argument("--mla-aliased", action="store_true",
                    help="time only the MLA-shaped decode over an absorbed-MLA cache (V = the "
                         "first 512 columns of the 576-wide K rows, one page table)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the kernels here run on a single MI355X and "
              "no multi-GPU path is built (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from scaled_dot_product_19_amd import inputs, sdpa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    sdpa.load()  # raises if the HIP library is missing; there is no fallback
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.chunked_prefill:
        run_chunked_prefill(args, torch, inputs, sdpa, dev)
        return
    if args.window_prefill:
        run_window_prefill(args, torch, inputs, sdpa, dev)
        return
    if args.fp8_prefill:
        run_fp8_prefill(args, torch, inputs, sdpa, dev)
        return
    if args.mtp_sweep or args.mla_aliased or args.fp8_decode or args.fp8_mla or args.gqa_mtp_sweep:
        run_decode_variant(args, torch, inputs, sdpa, dev)
        return

    t0 = time.time()
    case = inputs.thd_prefill_d128()
    pc = inputs.paged_decode_d128()
    log("inputs drawn in %.1f s: prefill T=%d lengths=%s; decode pages=%d lens sum=%d"
        % (time.time() - t0, int(case.cu_q[-1]), case.lengths_q, pc.k_pool.shape[0],
           int(pc.seq_lens.sum())))

    # --- device-resident inputs and caller-owned outputs -------------------
    q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
    cu_q, cu_kv = case.cu_q.to(dev), case.cu_kv.to(dev)
    T = int(case.cu_q[-1])
    o_p = torch.empty((T, case.hq, 128), dtype=torch.bfloat16, device=dev)
    lse_p = torch.empty((T, case.hq), dtype=torch.float32, device=dev)

    dq, kp, vp = pc.q.to(dev), pc.k_pool.to(dev), pc.v_pool.to(dev)
    ptk, ptv, sl = pc.pt_k.to(dev), pc.pt_v.to(dev), pc.seq_lens.to(dev)
    o_d = torch.empty((pc.batch, pc.sq, pc.hq, 128), dtype=torch.bfloat16, device=dev)
    lse_d = torch.empty((pc.batch, pc.sq, pc.hq), dtype=torch.float32, device=dev)
    ws = torch.empty(sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq, 128, pc.num_splits),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        sdpa.prefill_thd(q, k, v, cu_q, cu_kv, case.max_q, case.max_kv, case.scale, True,
                         out=o_p, lse=lse_p, lse_layout=sdpa.LSE_PACKED, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        sdpa.decode_paged(dq, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, pc.causal,
                          num_splits=pc.num_splits, workspace=ws, out=o_d, lse=lse_d,
                          stream=stream)
        if ev is not None:
            ev[2].record(stream)

    prewarm(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0

    total_ms = start.elapsed_time(end)
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    ms_per_step = total_ms / args.steps

    # the decode call alone, with a 512 MiB write between calls that evicts the MALL
    flush = torch.empty(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    dec_flushed = ms_stats(per_call_ms(
        torch, stream,
        lambda: sdpa.decode_paged(dq, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, pc.causal,
                                  num_splits=pc.num_splits, workspace=ws, out=o_d, lse=lse_d,
                                  stream=stream),
        args.steps, args.warmup, between=lambda: flush.fill_(1.0)))
    del flush

    flops = prefill_flops(case.lengths_q, case.lengths_kv, case.hq, 128, 128)
    kv_bytes, comp_bytes = decode_bytes(pc)
    pre_tflops = flops / (pre_avg * 1e-3) / 1e12
    dec_kv_gbs = kv_bytes / (dec_avg * 1e-3) / 1e9
    dec_comp_gbs = comp_bytes / (dec_avg * 1e-3) / 1e9
    log("prefill: %.4f ms avg (min %.4f) -> %.1f TFLOP/s (%.1f%% of bf16 peak)"
        % (pre_avg, min(pre_ms), pre_tflops, 100 * pre_tflops / PEAK_BF16_TFLOPS))
    log("decode : %.4f ms avg (min %.4f) -> %.1f GB/s K/V, %.1f GB/s compulsory (%.1f%% of HBM)"
        % (dec_avg, min(dec_ms), dec_kv_gbs, dec_comp_gbs, 100 * dec_comp_gbs / PEAK_HBM_GBS))
    log("step   : %.4f ms (wall %.4f ms)" % (ms_per_step, 1e3 * wall / args.steps))
    log("decode alone, MALL flushed before each call: %.4f ms median (min %.4f)"
        % (dec_flushed["median"], dec_flushed["min"]))

    cpu_pre = cpu_dec = None
    if not args.no_cpu_baseline:
        threads = host_threads()
        log("cpu baseline: oracle on %d threads, ~%.0f s per sample" % (threads,
                                                                      args.cpu_seconds))
        cpu_pre = cpu_baseline_prefill(case, args.cpu_seconds, threads)
        log("  prefill oracle: %.3g TFLOP/s (%s)" % (cpu_pre["value"], cpu_pre["sample"]))
        cpu_dec = cpu_baseline_decode(pc, args.cpu_seconds, threads)
        log("  decode oracle: %.3g GB/s (%s)" % (cpu_dec["value"], cpu_dec["sample"]))

    legs = [x for x in args.legs.split(",") if x]
    extra = {}
    threads = host_threads()
    del q, k, v, dq, kp, vp
    torch.cuda.empty_cache()
    if "c4" in legs:
        extra["c4_dense"] = d256_leg(args, torch, inputs, sdpa, dev, stream, threads, False)
        extra["c4_ragged"] = d256_leg(args, torch, inputs, sdpa, dev, stream, threads, True)
        torch.cuda.empty_cache()
    if "c5" in legs:
        extra["c5_mla_decode"] = mla_leg(args, torch, inputs, sdpa, dev, stream, threads)
        torch.cuda.empty_cache()
    if "c1" in legs:
        extra["c1_tiny_fp32"] = tiny_leg(args, torch, inputs, sdpa, dev, stream, threads)
    if "ctx" in legs:
        extra["context_phase"] = context_leg(args, torch, inputs, sdpa, dev, stream)

    line = {
        "metric": "prefill attn TFLOP/s (% MFMA peak); paged decode KV GB/s (% HBM peak)",
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16; lengths, page permutations drawn per seed)",
        "config": {
            "workload": "THD ragged causal prefill bf16 (8 seqs U[128,4096], 32/8 heads, D=128)"
                        " + paged decode bf16 (B=64, 32/8 heads, D=128, page 64, "
                        "L U[512,32768], 8 splits + LSE combine)",
            "prefill_tokens": T,
            "prefill_lengths": case.lengths_q,
            "prefill_flop": flops,
            "prefill_ms": round(pre_avg, 4),
            "prefill_ms_stats": ms_stats(pre_ms),
            "decode_batch": pc.batch,
            "decode_kv_bytes": kv_bytes,
            "decode_compulsory_bytes": comp_bytes,
            "decode_ms": round(dec_avg, 4),
            "decode_ms_stats": ms_stats(dec_ms),
            "decode_ms_mall_flushed": dec_flushed,
            "seeds": [inputs.SEED_BASE + 2, inputs.SEED_BASE + 3],
        },
        "decode": {
            "value": round(dec_kv_gbs, 1),
            "unit": "GB/s",
            "what": "K/V bytes of live tokens / (split kernel + combine kernel) time",
        },
        "roofline": {
            "kernel": "prefill_bf16_kernel<128, 64, 4, 8, true, false, false, false>",
            "bound": "mfma",
            "achieved": round(pre_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_traffic(PREFILL_TRAFFIC, PREFILL_SOURCES),
        },
        "roofline_decode": {
            "kernel": "decode_small_kernel<128, false, 128> + combine_kernel<false>",
            "bound": "hbm",
            "achieved": round(dec_comp_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_comp_gbs / PEAK_HBM_GBS, 4),
            "traffic": recorded_traffic(DECODE_TRAFFIC, DECODE_SOURCES),
        },
        "cpu_baseline": cpu_pre,
        "cpu_baseline_decode": cpu_dec,
        "host_cpu": {"model": host_cpu_model(), "threads_used": threads},
    }
    line.update(extra)
    line["prewarm_calls"] = PREWARM_CALLS
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
