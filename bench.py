#!/usr/bin/env python3
"""Benchmark of the shared-KV cross-decoder hot path on one MI355X.

One *step* is one generation step of the cross-decoder over the shared cache
at N = 131072 rows (YOCO-3B shapes: H_q=24, H_kv=8, d_h=128, 13 cross layers,
d_model=3072, bf16 storage, fp32 accumulation):

  1. append: RMSNorm of the new self-decoder row and its K^/V^ projection,
     written once into cache row 131071 (``yoco_kv_append``);
  2. for each of the 13 cross layers, one split-N decode call over all
     131072 rows with that layer's own query (``yoco_cross_attn_decode``).

The cache length is set back to 131071 before each step (a host-side
truncation), so every step decodes exactly 131072 rows.  Inputs are resident
in HBM before timing starts.  ``value`` is the whole step's time divided by
13 (microseconds per token per layer).

The same run also times causal prefill on the 32768-token workload (bf16
MFMA) and reports its TFLOP/s, and times the fp64 CPU oracle on the host
cores for the same decode step (``cpu_baseline``).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-prefill] [--prefill-reps R] [--cold-steps C]
                       [--workload decode128k|ragged16|decode1m]
       python bench.py --copy-calibration   (a plain 512 MiB device copy, three
                       times: the known-size reference for scaling the
                       FETCH_SIZE / WRITE_SIZE hardware counters)

The default workload is the 128K decode; ragged16 (16 sequences of 8192..131072
rows) and decode1m (2^20 rows) run the same step and report the same fields.
The cold figure repeats C steps with a 512 MiB copy before every decode launch,
so no cache level holds any of the shared K^/V^; it is reported apart from
``value``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, AMD published
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="decode128k")
    p.add_argument("--cold-steps", type=int, default=3,
                   help="extra steps with a 512 MiB copy before every decode launch (reported apart)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--prefill-reps", type=int, default=20)
    p.add_argument("--prefill-warmup", type=int, default=6)
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--dense-rows", action="store_true",
                   help="decode cache with dense rows instead of the library's padded row stride (for comparison)")
    p.add_argument("--no-graph-step", action="store_true",
                   help="skip the step replayed from a HIP graph (reported beside the headline)")
    p.add_argument("--no-extra-decodes", action="store_true",
                   help="skip the ragged-16 and 2^20-row decode workloads reported beside the headline")
    p.add_argument("--extra-steps", type=int, default=10, help="timed steps of each extra decode workload")
    return p.parse_args()


COPY_BYTES = 512 * 1024 * 1024
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "decode_128k_counters.md")
# The decode kernel's own sources: the FETCH/WRITE counters recorded in the
# summary hold only while these files hash to the digest stored beside them.
DECODE_SOURCES = (
    "yoco_shared_kv_amd/csrc/decode_kernel.h",
    "yoco_shared_kv_amd/csrc/decode.hip",
    "yoco_shared_kv_amd/csrc/device_common.h",
    "yoco_shared_kv_amd/csrc/decode_args.h",
)


PREFILL_COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "prefill_32k_counters.md")
PREFILL_SOURCES = (
    "yoco_shared_kv_amd/csrc/prefill.hip",
    "yoco_shared_kv_amd/csrc/attn_tiles.h",
    "yoco_shared_kv_amd/csrc/device_common.h",
)


def _digest(sources):
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def decode_source_digest():
    return _digest(DECODE_SOURCES)


def prefill_source_digest():
    return _digest(PREFILL_SOURCES)


def _summary_json(path):
    try:
        text = open(path).read()
    except OSError:
        return None, "no counter summary"
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if m is None:
        return None, "counter summary has no json block"
    return json.loads(m.group(1)), None


def prefill_mfma_busy():
    """Fraction of the prefill kernel's cycles its matrix cores were busy, from
    the committed counter summary: SQ_VALU_MFMA_BUSY_CYCLES (summed over the
    SIMDs) over SIMDs x GRBM_GUI_ACTIVE per XCD; or (None, reason)."""
    rec, why = _summary_json(PREFILL_COUNTER_SUMMARY)
    if rec is None:
        return None, why
    if rec["prefill_source_sha256"] != prefill_source_digest():
        return None, "prefill kernel sources changed since the counters were taken"
    return rec["mfma_busy_cycles"] / (rec["simds"] * rec["gui_active_cycles"] / rec["xcds"]), None


def counter_traffic():
    """HBM bytes per decode launch from the committed counter summary, or
    (None, reason).  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each
    scaled by COPY_BYTES over what the same counter read for the plain copy."""
    rec, why = _summary_json(COUNTER_SUMMARY)
    if rec is None:
        return None, why
    if rec["decode_source_sha256"] != decode_source_digest():
        return None, "decode kernel sources changed since the counters were taken"
    fetch_scale = rec["copy_bytes"] / (rec["copy_fetch_kib"] * 1024)
    write_scale = rec["copy_bytes"] / (rec["copy_write_kib"] * 1024)
    return (rec["decode_fetch_kib"] * 1024 * fetch_scale
            + rec["decode_write_kib"] * 1024 * write_scale), None


def copy_calibration(torch):
    """Copy 512 MiB device-to-device three times (torch's copy kernel): each
    dispatch reads and writes exactly COPY_BYTES of algorithmic traffic."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": COPY_BYTES, "dispatches": 3}), flush=True)


def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


WORKLOADS = {
    # name: (generator, size dict, description)
    "decode128k": ("make_decode", "DECODE_128K",
                   "decode, shared cache N=131072, H_q=24, H_kv=8, d_h=128, bf16, batch 1, 13 cross layers, "
                   "plus one appended row (d_model=3072)"),
    "ragged16": ("make_ragged_decode", "RAGGED_16",
                 "ragged decode, 16 sequences of 8192..131072 rows (sum 1,122,749), H_q=24, H_kv=8, "
                 "d_h=128, bf16, 13 cross layers, plus one appended row per sequence (d_model=3072)"),
    "decode1m": ("make_needle_decode", "NEEDLE_1M",
                 "decode, shared cache N=1048576 with a planted needle per KV head, H_q=24, H_kv=8, "
                 "d_h=128, bf16, batch 1, 13 cross layers, plus one appended row (d_model=3072)"),
}


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def bench_decode(args, torch, y, W):
    gen, size_name, _ = WORKLOADS[args.workload]
    cfg = getattr(W, size_name)
    log(f"generating {args.workload} workload")
    case = getattr(W, gen)(**cfg)
    n_seq = len(case.lens)
    lens = np.asarray(case.lens, dtype=np.int64)
    hq, hkv, dh, layers = case.n_q_heads, case.n_kv_heads, case.head_dim, case.layers
    cap = int(lens.max())
    d_model = 3072
    proj = W.make_project(n=(args.warmup + args.steps + args.cold_steps) * n_seq, d_model=d_model,
                          n_kv_heads=hkv, head_dim=dh, seed=1)

    cache = y.KVCache(n_seq, cap, hkv, dh, torch.bfloat16, padded=not args.dense_rows)
    log(f"cache rows: {cache.row_stride} elements ({'dense' if cache.row_stride == hkv * dh else 'padded'})")
    for b in range(n_seq):
        cache.k[b, :lens[b]] = to_dev(case.k[b], torch)
        cache.v[b, :lens[b]] = to_dev(case.v[b], torch)
    q_layers = [to_dev(case.q[l], torch) for l in range(layers)]          # each [n_seq, 24, 128]
    m_rows = to_dev(proj.m, torch)                                        # [steps * n_seq, 3072]
    w_k, w_v = to_dev(proj.w_k, torch), to_dev(proj.w_v, torch)
    gain = torch.ones(d_model, dtype=torch.float32, device="cuda")
    ws = y.decode_workspace(cache, hq)
    pws = torch.zeros(max(1, y.project_workspace_bytes(n_seq, d_model, hkv * dh, 2)), dtype=torch.uint8,
                      device="cuda")
    outs = [torch.empty((n_seq, hq, dh), dtype=torch.float32, device="cuda") for _ in range(layers)]
    stream = torch.cuda.current_stream()
    # Cold variant: a 512 MiB copy between layer calls evicts every cache level
    # (the MALL is 256 MB) before each decode launch.
    flush_src = flush_dst = None
    if args.cold_steps > 0:
        flush_src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        flush_dst = torch.empty_like(flush_src)
    torch.cuda.synchronize()

    # Three passes over the same step, each of args.steps steps:
    #   plain:     no event inside the steps; the wall clock and one event pair
    #              around the whole pass give ms_per_step (the headline);
    #   per step:  one event pair around each step (its spread);
    #   decode run: one event pair around the step's 13 back-to-back decode
    #              launches (after the append), so elapsed / 13 is the decode
    #              kernel's average launch duration for the roofline.
    # Every recorded event sits between two kernels on the stream and widens
    # that gap, so the instrumented passes are not used for the headline.
    ev_start = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    cold_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(layers * args.cold_steps)]

    def step(i, record_step=None, record_launch=None, cold=None):
        cache.len[:] = lens - 1
        if record_step is not None:
            step_ev[record_step][0].record(stream)
        y.kv_append(cache, m_rows[i * n_seq:(i + 1) * n_seq], w_k, w_v, gain, 1e-6, stream=stream, workspace=pws)
        for l in range(layers):
            if cold is not None:
                flush_dst.copy_(flush_src)
                cold_ev[cold * layers + l][0].record(stream)
            if record_launch is not None and l == 0:
                ev_start[record_launch].record(stream)
            y.cross_attn_decode(q_layers[l], cache, workspace=ws, out=outs[l], stream=stream)
            if record_launch is not None and l == layers - 1:
                ev_end[record_launch].record(stream)
            if cold is not None:
                cold_ev[cold * layers + l][1].record(stream)
        if record_step is not None:
            step_ev[record_step][1].record(stream)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    pass_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    pass_ev[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    pass_ev[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_per_step = pass_ev[0].elapsed_time(pass_ev[1]) / args.steps
    log(f"per-step and decode-run passes, {args.steps} steps each")
    for i in range(args.steps):
        step(args.warmup + i, record_step=i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + i, record_launch=i)
    torch.cuda.synchronize()
    kern_ms = [s_.elapsed_time(e_) / layers for s_, e_ in zip(ev_start, ev_end)]
    step_ms = [s_.elapsed_time(e_) for s_, e_ in step_ev]
    kern_avg_ms = float(np.mean(kern_ms))
    bytes_per_launch = int(2 * lens.sum() * hkv * dh * 2)   # K^ + V^ read once per layer call
    achieved_gbps = bytes_per_launch / (kern_avg_ms * 1e-3) / 1e9
    us_per_token_layer = ms_per_step * 1e3 / layers
    step_bytes = layers * bytes_per_launch + n_seq * 2 * d_model * hkv * dh * 2
    log(f"decode step {ms_per_step:.3f} ms (events: {gpu_ms_per_step:.3f}); {us_per_token_layer:.2f} "
        f"us/token/layer; decode kernel avg {kern_avg_ms * 1e3:.2f} us -> {achieved_gbps:.0f} GB/s")
    cold = None
    if args.cold_steps > 0:
        for i in range(args.cold_steps):
            step(args.warmup + args.steps + i, cold=i)
        torch.cuda.synchronize()
        cold_ms = [s_.elapsed_time(e_) for s_, e_ in cold_ev]
        cold = dict(avg_launch_us=float(np.mean(cold_ms)) * 1e3, p50_launch_us=pct(cold_ms, 50) * 1e3,
                    GBps=bytes_per_launch / (float(np.mean(cold_ms)) * 1e-3) / 1e9, launches=len(cold_ms))
        log(f"cold decode (512 MiB flush before each launch): avg {cold['avg_launch_us']:.2f} us "
            f"-> {cold['GBps']:.0f} GB/s")
    # The same step captured once in a HIP graph and replayed (how a serving
    # loop removes host work between launches): every replay appends the
    # captured row and decodes at the captured lengths, the same work as a
    # step.  Reported beside the headline, never as it.
    graph_ms = None
    if not args.no_graph_step:
        def graph_step():
            cache.len[:] = lens - 1
            i0 = args.warmup * n_seq
            y.kv_append(cache, m_rows[i0:i0 + n_seq], w_k, w_v, gain, 1e-6, workspace=pws)
            for l in range(layers):
                y.cross_attn_decode(q_layers[l], cache, workspace=ws, out=outs[l])
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            graph_step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        g_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        g_ev[0].record(stream)
        for _ in range(args.steps):
            graph.replay()
        g_ev[1].record(stream)
        torch.cuda.synchronize()
        graph_ms = g_ev[0].elapsed_time(g_ev[1]) / args.steps
        del graph
        log(f"decode step as a HIP graph replay: {graph_ms:.3f} ms ({graph_ms * 1e3 / layers:.2f} us/token/layer)")
    return dict(case=case, cache=cache, q_layers=q_layers, outs=outs, ms_per_step=ms_per_step,
                gpu_ms_per_step=gpu_ms_per_step, graph_ms_per_step=graph_ms,
                graph_us_per_token_layer=None if graph_ms is None else graph_ms * 1e3 / layers,
                us_per_token_layer=us_per_token_layer, kern_avg_us=kern_avg_ms * 1e3,
                kern_p10_us=pct(kern_ms, 10) * 1e3, kern_p50_us=pct(kern_ms, 50) * 1e3,
                kern_p90_us=pct(kern_ms, 90) * 1e3,
                step_p10_ms=pct(step_ms, 10), step_p50_ms=pct(step_ms, 50), step_p90_ms=pct(step_ms, 90),
                achieved_gbps=achieved_gbps, bytes_per_launch=bytes_per_launch,
                step_gbps=step_bytes / (ms_per_step * 1e-3) / 1e9, cold=cold, n_seq=n_seq, lens=lens,
                row_stride=cache.row_stride)


def bench_prefill(args, torch, y, W):
    cfg = W.PREFILL_32K
    n, hq, hkv, dh = cfg["n"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    log(f"generating prefill workload N={n}")
    c = W.make_prefill(**cfg)
    cache = y.KVCache(1, n, hkv, dh, torch.bfloat16)
    cache.k[0] = to_dev(c.k, torch)
    cache.v[0] = to_dev(c.v, torch)
    cache.len[0] = n
    q = to_dev(c.q, torch)
    o = torch.empty((n, hq, dh), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    # Untimed launches until the clocks have settled: the first few launches
    # after the decode phase run up to 20% slower.
    for _ in range(args.prefill_warmup):
        y.cross_attn_prefill(q, cache, out=o, stream=stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.prefill_reps)]
    for s, e in evs:
        s.record(stream)
        y.cross_attn_prefill(q, cache, out=o, stream=stream)
        e.record(stream)
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in evs]
    flops = 2.0 * dh * hq * n * (n + 1)                # causal QK^T and PV, diagonal included
    avg = float(np.mean(ms))
    tflops = flops / (avg * 1e-3) / 1e12
    log(f"prefill {avg:.3f} ms (p50 {pct(ms, 50):.3f}) -> {tflops:.1f} TFLOP/s")
    return dict(ms=avg, ms_p10=pct(ms, 10), ms_p50=pct(ms, 50), ms_p90=pct(ms, 90), tflops=tflops, flops=flops,
                frac=tflops / BF16_DENSE_PEAK_TFLOPS, case=c)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def stratified_rows(n, per_decile, seed=0):
    """Rows 0, 1 and n-1 plus `per_decile` distinct seeded rows in each tenth
    of the positions [0, n)."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, n - 1}
    for d in range(10):
        lo, hi = d * n // 10, (d + 1) * n // 10
        rows.update(int(r) for r in rng.choice(np.arange(lo, hi), min(per_decile, hi - lo), replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def causal_cpu_baseline(name, run_rows, n, per_decile):
    """Time an oracle call on a stratified sample of query rows of a causal
    workload of n rows and extrapolate to all n rows: the work of row r is
    proportional to its r + 1 visible keys."""
    import oracle
    rows = stratified_rows(n, per_decile)
    t0 = time.perf_counter()
    run_rows(rows)
    dt = time.perf_counter() - t0
    frac = float(np.sum(rows + 1)) / (n * (n + 1) / 2.0)
    full_ms = dt / frac * 1e3
    log(f"cpu baseline ({name}): {rows.size} sampled rows in {dt:.2f} s -> {full_ms / 1e3:.1f} s extrapolated")
    return {"value": round(full_ms, 1), "unit": "ms", "cores": oracle.num_threads(), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"rows 0, 1, {n - 1} and {per_decile} seeded rows per position decile ({rows.size} query rows "
                      f"of {n}), every head, timed ({dt:.2f} s wall, {frac * 100:.3f}% of the causal work) and "
                      f"extrapolated to all rows"}


def bench_backward(args, torch, y, W):
    """Backward of one cross layer's causal prefill at N=32768 (bf16 MFMA):
    dQ written, dK/dV added into fp32 buffers shared by the layers."""
    cfg = W.PREFILL_32K
    n, hq, hkv, dh = cfg["n"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    log(f"generating backward workload N={n}")
    c = W.make_prefill(**cfg)
    cache = y.KVCache(1, n, hkv, dh, torch.bfloat16)
    cache.k[0] = to_dev(c.k, torch)
    cache.v[0] = to_dev(c.v, torch)
    cache.len[0] = n
    q = to_dev(c.q, torch)
    d_o = to_dev(W.make_grad(n, hq, dh, seed=0)[0], torch)
    stream = torch.cuda.current_stream()
    o, lse = y.cross_attn_prefill(q, cache, want_lse=True, stream=stream)
    d_q = torch.empty((n, hq, dh), dtype=torch.float32, device="cuda")
    d_k = torch.zeros((n, hkv, dh), dtype=torch.float32, device="cuda")
    d_v = torch.zeros_like(d_k)
    ws = torch.empty(y.prefill_bwd_workspace_bytes(n, hq), dtype=torch.uint8, device="cuda")

    def bwd():
        y.cross_attn_prefill_bwd(q, o, d_o, lse, cache, d_q=d_q, d_k=d_k, d_v=d_v, workspace=ws, stream=stream)

    for _ in range(3):
        bwd()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.prefill_reps)]
    for s_ev, e_ev in evs:
        s_ev.record(stream)
        bwd()
        e_ev.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    # Five products per visible (row, key) pair: S (recomputed), dP, dV, dK
    # and dQ, 2 * d_h flops each; 2.5 times the forward.
    flops = 5.0 * dh * hq * n * (n + 1)
    tflops = flops / (avg * 1e-3) / 1e12
    log(f"prefill backward {avg:.3f} ms (p50 {pct(ms, 50):.3f}) -> {tflops:.1f} TFLOP/s")
    return dict(ms=avg, ms_p10=pct(ms, 10), ms_p50=pct(ms, 50), ms_p90=pct(ms, 90), tflops=tflops, flops=flops)


def bench_project(args, torch, y, W):
    """K^/V^ projection of a 32768-row prompt at 3B-like widths (3072 -> 2 x
    1024, bf16, matrix cores), with unit gain, with an fp32 gain, and with an
    fp32 gain plus RoPE on K^."""
    cfg = W.PROJECT_3B
    log(f"generating projection workload N={cfg['n']}")
    pc = W.make_project(**cfg, unit_gain=False)
    n, d = pc.m.shape
    m, w_k, w_v = to_dev(pc.m, torch), to_dev(pc.w_k, torch), to_dev(pc.w_v, torch)
    gain = torch.from_numpy(pc.gain).cuda()
    cache = y.KVCache(1, n, pc.n_kv_heads, pc.head_dim, torch.bfloat16)
    stream = torch.cuda.current_stream()
    flops = 2.0 * n * d * 2 * pc.n_kv_heads * pc.head_dim
    res = {}
    # rope: K^ rotated at its row positions in the epilogue (base 640K)
    for name, g, theta in (("unit_gain", None, None), ("fp32_gain", gain, None), ("fp32_gain_rope", gain, 640e3)):
        for _ in range(3):  # untimed: the first calls of a variant run slower
            y.kv_project(cache, m, w_k, w_v, g, pc.eps, stream=stream, rope_theta=theta)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.prefill_reps)]
        for s_ev, e_ev in evs:
            s_ev.record(stream)
            y.kv_project(cache, m, w_k, w_v, g, pc.eps, stream=stream, rope_theta=theta)
            e_ev.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        res[name] = dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)
        log(f"kv_project ({name}) {ms:.3f} ms -> {res[name]['tflops']:.1f} TFLOP/s")
    res["flops"] = flops

    # The cross-decoder's share of prefill with early exit: history rows only
    # write the cache (chunked projection), the last prompt token is appended
    # and runs the 13 cross layers (query projection + one decode each).
    layers, hq, dh = 13, 24, pc.head_dim
    rng = np.random.default_rng(5)
    x_last = [to_dev(W.store(rng.standard_normal((1, d)).astype(np.float32), W.BF16), torch) for _ in range(layers)]
    w_q = [to_dev(W.store((rng.standard_normal((d, hq * dh)) / math.sqrt(d)).astype(np.float32), W.BF16), torch)
           for _ in range(layers)]
    ws = y.decode_workspace(cache, hq)
    ncols = pc.n_kv_heads * pc.head_dim
    pws = torch.zeros(max(y.project_workspace_bytes(1, d, ncols, 2), y.project_workspace_bytes(1, d, hq * dh, 1)),
                      dtype=torch.uint8, device="cuda")
    outs = [torch.empty((1, hq, dh), dtype=torch.float32, device="cuda") for _ in range(layers)]
    qs = [torch.empty((1, hq, dh), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    chunk = 4096

    # The same pipeline with the RMSNorm gain folded into W_K and W_V once
    # (W' = diag(g) W in bf16, a weight preparation outside the timed region):
    # the chunks then run the unit-gain matrix-core path.
    w_k_f, w_v_f = y.fold_norm_gain(w_k, gain, stream=stream), y.fold_norm_gain(w_v, gain, stream=stream)
    f_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    f_ev[0].record(stream)
    y.fold_norm_gain(w_k, gain, out=w_k_f, stream=stream)
    y.fold_norm_gain(w_v, gain, out=w_v_f, stream=stream)
    f_ev[1].record(stream)
    torch.cuda.synchronize()
    log(f"gain folded into W_K and W_V (2 x {d} x {ncols} bf16, once per model; second call): "
        f"{f_ev[0].elapsed_time(f_ev[1]) * 1e3:.1f} us")

    def pipeline(folded=False):
        wk_, wv_, g_ = (w_k_f, w_v_f, None) if folded else (w_k, w_v, gain)
        cache.len[0] = 0
        for s0 in range(0, n - 1, chunk):
            e0 = min(s0 + chunk, n - 1)
            y.kv_project(cache, m[s0:e0], wk_, wv_, g_, pc.eps, row_start=s0, stream=stream)
        y.kv_append(cache, m[n - 1:n], wk_, wv_, g_, pc.eps, stream=stream, workspace=pws)
        for l in range(layers):
            q = y.q_project(x_last[l], w_q[l], hq, dh, out=qs[l], stream=stream, workspace=pws)
            y.cross_attn_decode(q, cache, workspace=ws, out=outs[l], stream=stream)

    for folded, key in ((False, "early_exit"), (True, "early_exit_folded")):
        pipeline(folded)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.prefill_reps)]
        for s_ev, e_ev in evs:
            s_ev.record(stream)
            pipeline(folded)
            e_ev.record(stream)
        torch.cuda.synchronize()
        ee = [a.elapsed_time(b) for a, b in evs]
        res[f"{key}_ms"] = float(np.mean(ee))
        res[f"{key}_p50_ms"] = pct(ee, 50)
        log(f"early-exit prefill at N={n} (chunked projection + append + 13 x (q_project + decode))"
            f"{', gain folded into W_K/W_V' if folded else ', fp32 gain'}: {res[f'{key}_ms']:.3f} ms")

    # The one-row projections of generation: the append of one K^/V^ row
    # (W_K and W_V read once) and one layer's query row (W_Q read once).  A
    # call through the Python binding costs more host time than the kernel
    # takes, so 50 launches are captured into a HIP graph and the graph is
    # replayed between one event pair (the kernels' back-to-back time).
    reps, replays = 50, 4
    one = {}
    for name, wbytes in (("append", 2 * d * ncols * 2), ("query", d * hq * dh * 2)):
        def launch(s_):
            if name == "append":
                cache.len[0] = n - 1
                y.kv_append(cache, m[n - 1:n], w_k, w_v, gain, pc.eps, stream=s_, workspace=pws)
            else:
                y.q_project(x_last[0], w_q[0], hq, dh, gain=gain, out=qs[0], stream=s_, workspace=pws)
        for _ in range(5):
            launch(stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                launch(None)          # the capturing stream
        graph.replay()
        torch.cuda.synchronize()
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        for _ in range(replays):
            graph.replay()
        b_ev.record(stream)
        torch.cuda.synchronize()
        us = a_ev.elapsed_time(b_ev) * 1e3 / (reps * replays)
        del graph
        one[name] = dict(us=us, bytes=wbytes, GBps=wbytes / (us * 1e-6) / 1e9)
        log(f"one-row {name} projection: {us:.2f} us per launch -> {one[name]['GBps']:.0f} GB/s of weights")
    res["one_row"] = one
    return res


def bench_project_bwd(args, torch, y, W):
    """Backward of the shared K^/V^ projection of a 32768-row prompt at 3B
    widths (bf16 M and weights, fp32 gain, fp32 upstream gradients as the
    attention backward leaves them): d_M written, d_W_K, d_W_V, d_gain added."""
    cfg = W.PROJECT_3B
    log(f"generating projection backward workload N={cfg['n']}")
    pc = W.make_project(**cfg, unit_gain=False)
    n, d = pc.m.shape
    ncols = pc.n_kv_heads * pc.head_dim
    dz_k, dz_v = W.make_proj_grad(n, ncols, 2, dtype=W.F32, seed=0)
    m, w_k, w_v = to_dev(pc.m, torch), to_dev(pc.w_k, torch), to_dev(pc.w_v, torch)
    dzk, dzv = to_dev(dz_k, torch), to_dev(dz_v, torch)
    gain = torch.from_numpy(pc.gain).cuda()
    d_m = torch.empty((n, d), dtype=torch.float32, device="cuda")
    d_wk = torch.zeros((d, ncols), dtype=torch.float32, device="cuda")
    d_wv = torch.zeros_like(d_wk)
    d_g = torch.zeros(d, dtype=torch.float32, device="cuda")
    ws = torch.empty(y.project_bwd_workspace_bytes(n, d, ncols, 2), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def bwd():
        y.kv_project_bwd(m, w_k, w_v, dzk, dzv, pc.n_kv_heads, pc.head_dim, gain=gain, eps=pc.eps, d_m=d_m,
                         d_w_k=d_wk, d_w_v=d_wv, d_gain=d_g, workspace=ws, stream=stream)

    for _ in range(3):
        bwd()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.prefill_reps)]
    for s_ev, e_ev in evs:
        s_ev.record(stream)
        bwd()
        e_ev.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    # Two products of 2 * n * d * (2 * ncols) flops each: dy = dZ W^T and dW = y^T dZ.
    flops = 2.0 * 2.0 * n * d * 2 * ncols
    tflops = flops / (avg * 1e-3) / 1e12
    log(f"kv_project backward {avg:.3f} ms (p50 {pct(ms, 50):.3f}) -> {tflops:.1f} TFLOP/s")
    return dict(ms=avg, ms_p10=pct(ms, 10), ms_p50=pct(ms, 50), ms_p90=pct(ms, 90), tflops=tflops, flops=flops)


def bench_gret(args, torch, y, W):
    """Gated retention (the self-decoder's token mixer) at the 3B shapes:
    the chunkwise prefill of 32768 positions x 24 heads of 128 (bf16), and
    one generation step of 13 self layers (recurrent, fp32 states of
    [24, 128, 128]) for batch 1."""
    cfg = W.GRET_32K
    log(f"generating gated-retention workload N={cfg['n']}")
    c = W.make_gret(**cfg, dtype=W.BF16, seed=0)
    n, heads, dh = cfg["n"], cfg["n_heads"], cfg["head_dim"]
    q, k, v = to_dev(c.q, torch), to_dev(c.k, torch), to_dev(c.v, torch)
    g = torch.from_numpy(c.gate).cuda()
    o = torch.empty((n, heads, dh), dtype=torch.float32, device="cuda")
    s_out = torch.empty((heads, dh, dh), dtype=torch.float32, device="cuda")
    ws = torch.empty(y.gret_prefill_workspace_bytes(n, heads, dh, torch.bfloat16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def pre():
        if y.lib().yoco_gret_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), 1, g.data_ptr(), c.tau, n, heads, dh,
                                     None, o.data_ptr(), s_out.data_ptr(), ws.data_ptr(), ws.numel(),
                                     stream.cuda_stream) != 0:
            raise RuntimeError(y.lib().yoco_last_error().decode())

    pre()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.prefill_reps)]
    for s_ev, e_ev in evs:
        s_ev.record(stream)
        pre()
        e_ev.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    # Algorithmic bytes: q, k, v (bf16) and the gate logits read once, o (fp32) written once.
    alg = n * heads * (3 * dh * 2 + 4 + dh * 4)
    gbps = alg / (avg * 1e-3) / 1e9
    log(f"gret prefill {avg:.3f} ms -> {gbps:.0f} GB/s algorithmic")
    # One generation step of 13 self layers, batch 1.
    layers = 13
    cd = W.make_gret(n=layers, n_heads=heads, head_dim=dh, dtype=W.BF16, seed=1)
    qd, kd, vd = to_dev(cd.q, torch), to_dev(cd.k, torch), to_dev(cd.v, torch)
    gd = torch.from_numpy(cd.gate).cuda()
    states = torch.zeros((layers, 1, heads, dh, dh), dtype=torch.float32, device="cuda")
    od = torch.empty((layers, 1, heads, dh), dtype=torch.float32, device="cuda")

    # Pointers marshalled once: the step is 13 calls of the C entry point.
    lib = y.lib()
    es = 2  # bf16 element size
    call_args = [(qd.data_ptr() + l * heads * dh * es, kd.data_ptr() + l * heads * dh * es,
                  vd.data_ptr() + l * heads * dh * es, gd.data_ptr() + l * heads * 4, states[l].data_ptr(),
                  od[l].data_ptr()) for l in range(layers)]

    def dec():
        for qp, kp, vp, gp, sp, op in call_args:
            if lib.yoco_gret_decode(qp, kp, vp, 1, gp, cd.tau, 1, heads, dh, sp, op, stream.cuda_stream) != 0:
                raise RuntimeError(lib.yoco_last_error().decode())

    for _ in range(3):
        dec()
    torch.cuda.synchronize()
    d_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.prefill_reps)]
    for s_ev, e_ev in d_evs:
        s_ev.record(stream)
        dec()
        e_ev.record(stream)
    torch.cuda.synchronize()
    dms = [a.elapsed_time(b) for a, b in d_evs]
    davg = float(np.mean(dms))
    log(f"gret decode step (13 layers) {davg * 1e3:.1f} us")
    return dict(ms=avg, ms_p10=pct(ms, 10), ms_p50=pct(ms, 50), ms_p90=pct(ms, 90), gbps=gbps, bytes=alg,
                decode_us=davg * 1e3, decode_p50_us=pct(dms, 50) * 1e3, case=c)


def needle_cosines(torch, dec):
    """cos(o, V^ row of the needle) for every layer and query head of the last
    timed step of the 2^20-row workload (the needle reading of the pages'
    long-context test: the output points along the needle's value row)."""
    case, cache, outs = dec["case"], dec["cache"], dec["outs"]
    g_size = case.n_q_heads // case.n_kv_heads
    cos = []
    for h in range(case.n_q_heads):
        g = h // g_size
        v = cache.v[0, int(case.needle_pos[0, g]), g].float()
        for o in outs:
            oh = o[0, h]
            cos.append(float((oh @ v) / (oh.norm() * v.norm())))
    return cos


def bench_extra_decodes(args, torch, y, W):
    """The ragged 16-sequence and the 2^20-row (planted needle) decode
    workloads through the same step as the headline (one append per sequence
    and 13 decode calls), fewer steps each."""
    res = {}
    for wl in ("ragged16", "decode1m"):
        sub = argparse.Namespace(**vars(args))
        sub.workload, sub.steps, sub.warmup, sub.cold_steps = wl, args.extra_steps, 2, 0
        sub.no_graph_step = True
        d = bench_decode(sub, torch, y, W)
        entry = {
            "workload": WORKLOADS[wl][2],
            "us_per_token_layer": round(d["us_per_token_layer"], 2),
            "ms_per_step": round(d["ms_per_step"], 4),
            "steps": args.extra_steps,
            "roofline": {"bound": "hbm", "achieved": round(d["achieved_gbps"], 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(d["achieved_gbps"] / HBM_PEAK_GBPS, 4),
                         "avg_launch_us": round(d["kern_avg_us"], 2), "bytes_per_launch": d["bytes_per_launch"]},
        }
        if wl == "decode1m":
            cos = needle_cosines(torch, d)
            entry["needle_cos_min"] = round(min(cos), 5)
            entry["needle_check"] = "min over 13 layers x 24 heads of cos(o, V^ needle row) >= 0.99"
            log(f"decode1m needle: min cos {min(cos):.5f} over {len(cos)} (layer, head) outputs")
        res[wl] = entry
        del d
        torch.cuda.empty_cache()
    return res


def cpu_baseline(dec, W):
    import oracle
    case = dec["case"]
    threads = oracle.num_threads()
    rows = int(np.sum(case.lens))
    log(f"cpu baseline: fp64 oracle decode, 13 layers x 24 heads over {rows} rows, {threads} threads")
    t0 = time.perf_counter()
    for b, n in enumerate(case.lens):
        oracle.decode(case.q[:, b], int(n), case.k[b], case.v[b], case.softmax_scale)
    dt = time.perf_counter() - t0
    return {"value": dt * 1e6 / case.layers, "unit": "us/token/layer", "cores": threads, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"one full decode step: 13 layers x 24 query heads over all {rows} cache rows of "
                      f"{len(case.lens)} sequence(s) (fp64, {dt:.2f} s wall)"}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              f"(each box has a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import workloads as W
    import yoco_shared_kv_amd as y

    dec = bench_decode(args, torch, y, W)
    pre = None if args.no_prefill else bench_prefill(args, torch, y, W)
    proj = None if args.no_prefill else bench_project(args, torch, y, W)
    bwd = None if args.no_prefill else bench_backward(args, torch, y, W)
    pbwd = None if args.no_prefill else bench_project_bwd(args, torch, y, W)
    gret = None if args.no_prefill else bench_gret(args, torch, y, W)
    extra = None if (args.no_extra_decodes or args.workload != "decode128k") else bench_extra_decodes(args, torch, y, W)
    cpu = None if args.no_cpu_baseline else cpu_baseline(dec, W)
    pre_cpu = gret_cpu = None
    if not args.no_cpu_baseline and pre is not None:
        import oracle
        c = pre["case"]
        pre_cpu = causal_cpu_baseline(
            "prefill", lambda rows: oracle.prefill(c.q, 0, c.k, c.v, c.softmax_scale, rows=rows), c.k.shape[0], 128)
    if not args.no_cpu_baseline and gret is not None:
        import oracle
        gc = gret["case"]
        gamma = oracle.gret_gate(gc.gate, gc.tau)
        gret_cpu = causal_cpu_baseline(
            "gated retention", lambda rows: oracle.gret(gc.q, gc.k, gc.v, gamma, rows=rows), gc.q.shape[0], 8)
    # The committed counters were taken on the 128K workload.
    traffic, why = counter_traffic() if args.workload == "decode128k" else (None, "counters cover decode128k only")
    if args.dense_rows and why is None:
        traffic, why = None, "counters were taken on padded cache rows"
    if why:
        log(f"roofline.traffic is null: {why}")
    metric = "cross-attn decode us/token/layer at N=128K (shared bf16 K^/V^, 13 layers)"
    if args.workload != "decode128k":
        metric = f"cross-attn decode us/token/layer, {args.workload} (shared bf16 K^/V^, 13 layers)"

    result = {
        "metric": metric,
        "value": round(dec["us_per_token_layer"], 3),
        "unit": "us/token/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), no weights)",
        "config": {
            "workload": WORKLOADS[args.workload][2],
            "n_rows": int(dec["lens"].sum()), "layers": 13, "n_q_heads": 24, "n_kv_heads": 8, "head_dim": 128,
            "d_model": 3072, "batch": dec["n_seq"], "cache_row_stride": dec["row_stride"],
        },
        "gpu_ms_per_step": round(dec["gpu_ms_per_step"], 4),
        "step_ms_p10_p50_p90": [round(dec["step_p10_ms"], 4), round(dec["step_p50_ms"], 4),
                                round(dec["step_p90_ms"], 4)],
        "decode_hbm_GBps": round(dec["achieved_gbps"], 1),
        "step_GBps": round(dec["step_gbps"], 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel<bf16, d_h=128, G=3>",
            "achieved": round(dec["achieved_gbps"], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec["achieved_gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else round(traffic),
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "traffic_over_algorithmic": None if traffic is None else round(traffic / dec["bytes_per_launch"], 4),
            "avg_launch_us": round(dec["kern_avg_us"], 2),
            "launch_us_p10_p50_p90": [round(dec["kern_p10_us"], 2), round(dec["kern_p50_us"], 2),
                                      round(dec["kern_p90_us"], 2)],
            "launch_timing": "HIP events on the launch stream around each step's 13 back-to-back decode launches; "
                             "avg over steps of elapsed / 13 (percentiles over steps)",
            "bytes_per_launch": dec["bytes_per_launch"],
        },
        "decode_graph": None if dec["graph_ms_per_step"] is None else {
            "what": "the same step (append + 13 decodes) captured once in a HIP graph and replayed "
                    "--steps times between two events; each replay appends the captured row and decodes at "
                    "the captured lengths",
            "ms_per_step": round(dec["graph_ms_per_step"], 4),
            "us_per_token_layer": round(dec["graph_us_per_token_layer"], 3)},
        "decode_cold": None if dec["cold"] is None else {
            "what": "a 512 MiB device copy before every decode launch (evicts L2 and the 256 MB MALL)",
            "avg_launch_us": round(dec["cold"]["avg_launch_us"], 2),
            "p50_launch_us": round(dec["cold"]["p50_launch_us"], 2),
            "GBps": round(dec["cold"]["GBps"], 1), "launches": dec["cold"]["launches"]},
        "cpu_baseline": cpu,
    }
    if extra is not None:
        result.update(extra)
    if pre is not None:
        busy, busy_why = prefill_mfma_busy()
        if busy_why:
            log(f"prefill.roofline.mfma_busy is null: {busy_why}")
        result["prefill"] = {
            "workload": "causal prefill N=32768, H_q=24, H_kv=8, d_h=128, bf16 MFMA, fp32 out",
            "ms": round(pre["ms"], 3), "tflops": round(pre["tflops"], 1),
            "ms_p10_p50_p90": [round(pre["ms_p10"], 3), round(pre["ms_p50"], 3), round(pre["ms_p90"], 3)],
            "roofline": {"bound": "mfma", "achieved": round(pre["tflops"], 1),
                         "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pre["frac"], 4), "flops_per_launch": pre["flops"],
                         "mfma_busy": None if busy is None else round(busy, 4),
                         "mfma_busy_unit": "fraction of the kernel's cycles the matrix cores were busy "
                                           "(SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE per "
                                           "XCD, committed counters)"},
            "cpu_baseline": pre_cpu,
        }
    if proj is not None:
        u = proj["unit_gain"]
        result["kv_project"] = {
            "workload": "K^/V^ projection of 32768 rows, 3072 -> 2 x 1024 (8 KV heads x 128), bf16 MFMA, "
                        "RMSNorm fused, written into the cache",
            "ms": round(u["ms"], 4), "tflops": round(u["tflops"], 1),
            "ms_fp32_gain": round(proj["fp32_gain"]["ms"], 4),
            "ms_fp32_gain_rope": round(proj["fp32_gain_rope"]["ms"], 4),
            "roofline": {"bound": "mfma", "achieved": round(u["tflops"], 1), "peak": BF16_DENSE_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(u["tflops"] / BF16_DENSE_PEAK_TFLOPS, 4),
                         "flops_per_launch": proj["flops"]},
            # Same algorithmic flops with an fp32 gain: x*g enters the bf16
            # products as hi + lo halves, so the matrix cores do twice the work.
            "roofline_fp32_gain": {"bound": "mfma", "achieved": round(proj["fp32_gain"]["tflops"], 1),
                                   "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(proj["fp32_gain"]["tflops"] / BF16_DENSE_PEAK_TFLOPS, 4),
                                   "flops_per_launch": proj["flops"], "mfma_flops_per_launch": 2 * proj["flops"]},
        }
        result["early_exit_prefill"] = {
            "workload": "cross-decoder share of a 32768-token prompt with early exit: K^/V^ of rows 0..N-2 "
                        "projected in 4096-row chunks, the last token appended, then 13 x (Q projection of "
                        "one row + one decode over all 32768 rows)",
            "ms": round(proj["early_exit_ms"], 4), "p50_ms": round(proj["early_exit_p50_ms"], 4),
            "ms_folded_gain": round(proj["early_exit_folded_ms"], 4),
            "p50_ms_folded_gain": round(proj["early_exit_folded_p50_ms"], 4),
            "folded_gain": "the RMSNorm gain folded into W_K and W_V once (W' = diag(g) W rounded to bf16 per "
                           "element), so the chunks run the unit-gain matrix-core path; `ms` applies the fp32 "
                           "gain to the activations (x*g as a bf16 hi + lo pair, two products per fragment)",
            "without_early_exit_ms": None if pre is None else round(13 * pre["ms"], 3),
            "without_early_exit": "13 causal prefill launches over the whole prompt (the cross layers "
                                  "run for every position)",
        }
        one = proj["one_row"]
        result["one_row_projection"] = {
            "workload": "generation-time projections of one row at 3B widths (bf16 weights, fp32 gain, RMSNorm "
                        "fused): the K^/V^ append (3072 -> 2 x 1024) and one layer's query (3072 -> 24 x 128); "
                        "weights split over their d_model rows across the chip",
            "timing": "50 launches captured in a HIP graph, HIP events around 4 replays (no host time "
                      "between launches)",
        }
        for name in ("append", "query"):
            e = one[name]
            result["one_row_projection"][name] = {
                "us": round(e["us"], 2), "weight_bytes": e["bytes"],
                "roofline": {"bound": "hbm", "achieved": round(e["GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(e["GBps"] / HBM_PEAK_GBPS, 4)},
            }
    if bwd is not None:
        result["prefill_backward"] = {
            "workload": "backward of one cross layer's causal prefill N=32768, H_q=24, H_kv=8, d_h=128, bf16 "
                        "MFMA: dQ written, dK/dV added (fp32)",
            "ms": round(bwd["ms"], 3),
            "ms_p10_p50_p90": [round(bwd["ms_p10"], 3), round(bwd["ms_p50"], 3), round(bwd["ms_p90"], 3)],
            "roofline": {"bound": "mfma", "achieved": round(bwd["tflops"], 1), "peak": BF16_DENSE_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(bwd["tflops"] / BF16_DENSE_PEAK_TFLOPS, 4),
                         "flops_per_launch": bwd["flops"],
                         "flops_convention": "5 products x 2 d_h per visible (row, key) pair"},
        }
    if pbwd is not None:
        result["kv_project_backward"] = {
            "workload": "backward of the K^/V^ projection of 32768 rows, 3072 -> 2 x 1024, bf16 MFMA (y and dz "
                        "rounded to bf16), fp32 gain: d_M written, d_W_K, d_W_V, d_gain added (fp32)",
            "ms": round(pbwd["ms"], 4),
            "ms_p10_p50_p90": [round(pbwd["ms_p10"], 4), round(pbwd["ms_p50"], 4), round(pbwd["ms_p90"], 4)],
            "roofline": {"bound": "mfma", "achieved": round(pbwd["tflops"], 1), "peak": BF16_DENSE_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(pbwd["tflops"] / BF16_DENSE_PEAK_TFLOPS, 4),
                         "flops_per_launch": pbwd["flops"],
                         "flops_convention": "dy = dZ W^T and dW = y^T dZ, 2 n d (2 ncols) flops each"},
        }
    if gret is not None:
        result["gret_self_decoder"] = {
            "workload": "gated retention at the 3B self-decoder shapes: chunkwise prefill of 32768 positions x 24 "
                        "heads of 128 (bf16 q/k/v, fp32 gates, o and states; tau 16), and one generation step of "
                        "13 self layers at batch 1 (recurrent, fp32 [24,128,128] states)",
            "prefill_ms": round(gret["ms"], 4),
            "prefill_ms_p10_p50_p90": [round(gret["ms_p10"], 4), round(gret["ms_p50"], 4), round(gret["ms_p90"], 4)],
            "prefill_roofline": {"bound": "hbm", "achieved": round(gret["gbps"], 1), "peak": HBM_PEAK_GBPS,
                                 "unit": "GB/s", "frac": round(gret["gbps"] / HBM_PEAK_GBPS, 4),
                                 "bytes_per_launch": gret["bytes"],
                                 "bytes_convention": "q, k, v (bf16) and gate logits read once, o (fp32) written "
                                                     "once; chunk states are implementation traffic"},
            "prefill_cpu_baseline": gret_cpu,
            "decode_step_us": round(gret["decode_us"], 2),
            "decode_step_p50_us": round(gret["decode_p50_us"], 2),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
