#!/usr/bin/env python3
"""Benchmark of paged decode attention on one MI355X.

One step is one decode step of the 64-request Qwen3-235B-shaped workload
(one GPU's share under TP8: 8 query heads on 1 KV head, head_dim 128,
block_size 16, contexts U[1000,2000]):
  1. cache write of each request's new token into the shuffled KV cache,
  2. paged GQA decode attention over every request's whole context
     (split-KV partitions + log-sum-exp merge),
both in one launch (pa_paged_decode_attn_write; --separate-cache-write runs
them as two launches).  Steps rotate over several independent KV pools
(like the layers of a model), together larger than the 256 MB Infinity
Cache, so every step reads its KV from HBM.  The timed region launches the
steps eagerly (--graph-timing replays captured HIP graphs instead; a replay
is also checked against the eager result); the decode kernel's own duration
is measured with HIP events on the stream it is launched on.

The decode lines also carry hbm_read_ceiling: the time of a plain
streaming read (pa_stream_read) of the same number of bytes on the same GPU,
i.e. what the memory system delivers at this transfer size; the GQA lines
over the preshuffled cache also carry hbm_gather_ceiling: the time of
reading exactly the blocks the decode reads, through its block table over
the same rotating pools, with no arithmetic (pa_gather_read).

Prints one JSON line.  Other workloads: --config long_context | mla | extend.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: achieved HBM GB/s (% of peak) and decode tok/s, 64 reqs"

# HBM traffic per launch of each workload's dominant kernel from rocprofv3 FETCH_SIZE +
# WRITE_SIZE, scaled by a plain copy of known size (summaries and commands in profiles/),
# valid only for the kernel sources it was measured on:
# workload -> (sources, sha256 prefix of those sources, bytes per launch).
_CSRC = "paged_attention_decode_reshape_amd/csrc/"
# The sources of each workload's kernels, for the tag the JSON line carries.
KERNEL_SOURCES = {
    "gqa": (_CSRC + "decode_gqa.hip", _CSRC + "decode_common.h", _CSRC + "fp8.h"),
    "mla": (_CSRC + "mla_decode.hip", _CSRC + "decode_common.h", _CSRC + "fp8.h"),
    "extend": (_CSRC + "extend.hip", _CSRC + "decode_common.h"),
    "merge": (_CSRC + "merge.hip",),
    "cache_write": (_CSRC + "cache_write.hip", _CSRC + "fp8.h"),
}

# HBM bytes per launch of the line's dominant kernel from rocprofv3 FETCH_SIZE
# and WRITE_SIZE runs (one counter per run, each scaled by what it reads for a
# plain 64 MiB device copy in the same process), for the workload's default
# launch: key -> (source group, sha256 prefix of that group when measured,
# bytes).  Keys name the variant: workload, then _fp8 (FP8 cache) and _mfma
# (matrix-core MLA engine).
MEASURED_TRAFFIC = {
    "qwen3": ("gqa", "9809f6225010d674", 52.32e6),
    "qwen3_fp8": ("gqa", "9809f6225010d674", 28.37e6),
    "long_context": ("gqa", "9809f6225010d674", 1147.95e6),
    "mla": ("mla", "30dd7bded0e5261d", 237.16e6),
    "mla_mfma": ("mla", "30dd7bded0e5261d", 216.84e6),
    "mla_fp8": ("mla", "30dd7bded0e5261d", 139.27e6),
    "mla_fp8_mfma": ("mla", "30dd7bded0e5261d", 145.69e6),
    "extend": ("extend", "f06b1df214d4f57b", 1295.37e6),
    "merge": ("merge", "5767d743027acd19", 340.74e6),
    "cache_write": ("cache_write", "a6f4db786c645612", 107.92e6),
}


def sources_sha(sources) -> str:
    """sha256 prefix of the concatenated source files (tags measurements)."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def default_launch(args) -> bool:
    """Whether the line times the launch the counters were taken on: the
    workload's own split, the fused cache write and the shuffled layout."""
    return (args.partition_tokens is None and not args.separate_cache_write
            and args.kv_layout == "shuffled")


def measured_traffic(key, default_launch=True):
    """The counter-measured bytes per launch, or None for a launch other than
    the measured one (another split or layout) or once the kernel changed."""
    if not default_launch or key not in MEASURED_TRAFFIC:
        return None
    group, sha, nbytes = MEASURED_TRAFFIC[key]
    return nbytes if sources_sha(KERNEL_SOURCES[group]) == sha else None


def trace_summary(path, top=12):
    """Per-kernel duration statistics (count, mean, median, p10, p90, min,
    max in microseconds) from a rocprofv3 kernel-trace CSV, as a markdown
    table, longest total time first."""
    import csv
    durs = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or row.get("KernelName")
            t0 = int(row.get("Start_Timestamp") or row.get("Start-Timestamp"))
            t1 = int(row.get("End_Timestamp") or row.get("End-Timestamp"))
            durs.setdefault(name, []).append((t1 - t0) / 1000.0)
    lines = ["| kernel | launches | mean us | median us | p10 us | p90 us | min us | max us |",
             "|---|---|---|---|---|---|---|---|"]
    for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1]))[:top]:
        a = np.array(d)
        short = name if len(name) <= 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {a.size} | {a.mean():.2f} | {np.median(a):.2f} | "
                     f"{np.percentile(a, 10):.2f} | {np.percentile(a, 90):.2f} | {a.min():.2f} | "
                     f"{a.max():.2f} |")
    return "\n".join(lines)


HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="qwen3",
                    choices=["qwen3", "qwen3_10k", "long_context", "mla", "mla_bs1", "extend",
                             "mixed", "merge", "cache_write"])
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="GQA decode cache element type: bf16, or FP8 E4M3 codes with "
                         "per-tensor scales (amax / 448), shuffled layout with x = 16")
    ap.add_argument("--mla-engine", default="valu", choices=["valu", "mfma"],
                    help="MLA decode: the VALU kernels (pa_mla_decode_attn*) or the matrix-core "
                         "ones (pa_mla_decode_attn_mfma, pa_mla_decode_attn_fp8_mfma)")
    ap.add_argument("--kv-layout", default="shuffled", choices=["shuffled", "standard"],
                    help="GQA decode cache layout: the pages' shuffled one, or the standard "
                         "[num_blocks, block_size, kv_heads, head_dim] it replaces (same "
                         "kernel, V transposed through LDS) to measure the difference")
    ap.add_argument("--pools", type=int, default=0, help="KV pool copies (0: enough to exceed the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle CPU-baseline budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph capture check")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip timing a plain streaming read of the decode's algorithmic bytes")
    ap.add_argument("--graph-timing", action="store_true",
                    help="time GQA steps as HIP-graph replays instead of eager launches")
    ap.add_argument("--separate-cache-write", action="store_true",
                    help="GQA step as two launches (cache write, then decode) instead of the "
                         "fused pa_paged_decode_attn_write")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="decode split (GQA and MLA): 0 auto, -2 balanced, > 0 fixed "
                         "partitions, -1 unsplit (default: the workload's own)")
    ap.add_argument("--trace-summary", default=None, metavar="CSV",
                    help="print per-kernel duration statistics of a rocprofv3 kernel-trace CSV "
                         "and exit (no GPU needed)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after the bench, run plain device copies of this many MiB (a known "
                         "byte count for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# GQA decode workloads
# ---------------------------------------------------------------------------

def gqa_algorithmic_bytes(case, with_write=False, kv_bytes=2) -> int:
    """Bytes the method must move per decode launch: every context token's K
    and V once (kv_bytes per element: 2 bf16, 1 FP8), q, out, lse, the used
    block-table entries and lengths (and, with the fused cache write, each
    new token's bf16 K and V read and its cache elements written, plus its
    slot)."""
    S, Hq, Hkv, D, B = case.S, case.Hq, case.Hkv, case.D, case.B
    n = case.context_lens.astype(np.int64)
    kv = int(n.sum()) * Hkv * D * 2 * kv_bytes
    blocks = int(((n + B - 1) // B).sum())
    write = S * Hkv * D * 2 * (2 + kv_bytes) + S * 8 if with_write else 0
    return kv + S * Hq * D * 2 * 2 + S * Hq * 4 + blocks * 4 + S * 4 + write


def gqa_algorithmic_flops(case) -> int:
    return int(case.context_lens.astype(np.int64).sum()) * case.Hq * case.D * 4


def time_launches(launch, n):
    """Average per-launch time (ms) of n back-to-back launches, measured with
    HIP events recorded on the stream the launches use."""
    import torch
    cur = torch.cuda.current_stream()
    for i in range(5):
        launch(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for i in range(n):
        launch(i)
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


_SLEEP_CYCLES_PER_MS = None


def _gate(ms):
    """Hold the current stream for about `ms` with torch's bounded spin
    kernel, so that launches enqueued meanwhile then run back to back."""
    import torch
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 2_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def launch_stats(launch, n=240, batch=20):
    """Device time per launch (ms) of n launches run back to back: the
    stream is held by a short spin while they are enqueued.  mean_ms comes
    from one pair of HIP events around all n on the launch stream; a second
    pass records an event after every `batch` launches and reports the
    spread of the per-batch means (an event after every single launch would
    add its own few microseconds to each).  The median of the batch means
    (`avg_ms`) is the figure the lines use: one slow host enqueue that lets
    the GPU idle inflates the single-pair mean but only one batch.
    Per-launch percentiles come from rocprofv3 kernel traces."""
    import torch
    cur = torch.cuda.current_stream()
    for i in range(5):
        launch(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _gate(max(2.0, 0.05 * n))
    e0.record(cur)
    for i in range(n):
        launch(i)
    e1.record(cur)
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / n
    nb = max(1, n // batch)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    _gate(max(2.0, 0.05 * n))
    ev[0].record(cur)
    for b in range(nb):
        for j in range(batch):
            launch(b * batch + j)
        ev[b + 1].record(cur)
    torch.cuda.synchronize()
    d = np.array([ev[b].elapsed_time(ev[b + 1]) / batch for b in range(nb)])
    return {"launches": n, "avg_ms": float(np.median(d)), "mean_ms": mean, "batch": batch,
            "batch_mean_median_ms": float(np.median(d)),
            "batch_mean_p10_ms": float(np.percentile(d, 10)),
            "batch_mean_p90_ms": float(np.percentile(d, 90)),
            "method": "HIP events on the launch stream around back-to-back launches"}


def read_ceiling(nbytes, grids=(1024, 2048, 4096, 8192), n=200):
    """What a plain streaming read of `nbytes` achieves on this GPU: the
    library's pa_stream_read over enough rotated copies to defeat the
    Infinity Cache, best workgroup count, HIP events around n back-to-back
    launches."""
    import torch
    import paged_attention_decode_reshape_amd as pa

    nbytes = max(16, nbytes // 16 * 16)
    copies = max(2, math.ceil(2 * MALL_BYTES / nbytes))
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.empty(max(grids), dtype=torch.int32, device="cuda")
    best = None
    for g in grids:
        ms = time_launches(lambda i: pa.stream_read(bufs[i % copies], g, sink, verify=False), n)
        if best is None or ms < best[1]:
            best = (g, ms)
    del bufs
    torch.cuda.empty_cache()
    gbps = nbytes / (best[1] * 1e-3) / 1e9
    return {"kernel": "stream_read_kernel (pa_stream_read)", "bytes": nbytes,
            "workgroups": best[0], "avg_launch_ms": best[1], "gbps": gbps,
            "frac_of_peak": gbps / HBM_PEAK_GBPS}


def bench_gqa(args, case, label):
    import torch
    import paged_attention_decode_reshape_amd as pa

    dev = torch.device("cuda:0")
    pg = case.paging
    std = args.kv_layout == "standard"
    f8 = args.kv_dtype == "fp8"
    if std and f8:
        raise SystemExit("--kv-dtype fp8 uses the shuffled layout only")
    layout = pa.LAYOUT_STANDARD_KV if std else pa.LAYOUT_SHUFFLED_KV
    kv_bytes = 1 if f8 else 2
    pool_bytes = pg.num_blocks * case.Hkv * case.D * case.B * 2 * kv_bytes
    if f8:  # per-tensor scales from the data's largest magnitude
        k_scale = float(case.key.abs().max()) / 448.0
        v_scale = float(case.value.abs().max()) / 448.0
    pools = args.pools or max(1, math.ceil(2 * MALL_BYTES / pool_bytes))
    log(f"[bench] {label}: S={case.S} Hq={case.Hq} Hkv={case.Hkv} D={case.D} B={case.B} "
        f"tokens={pg.total_tokens} pool={pool_bytes / 1e6:.1f} MB x {pools} copies")
    key = case.key.to(dev)
    value = case.value.to(dev)
    slots_all = torch.from_numpy(pg.slot_mapping).to(dev)
    caches = []
    for _ in range(pools):
        if f8:
            kc = torch.zeros((pg.num_blocks, case.Hkv, case.D // 16, case.B, 16),
                             dtype=torch.uint8, device=dev)
            vc = torch.zeros((pg.num_blocks, case.Hkv, case.B // 16, case.D, 16),
                             dtype=torch.uint8, device=dev)
            pa.reshape_and_cache_fp8(key, value, kc, vc, slots_all, k_scale, v_scale)
            caches.append((kc, vc))
            continue
        if std:
            kc = torch.zeros((pg.num_blocks, case.B, case.Hkv, case.D), dtype=torch.bfloat16,
                             device=dev)
            vc = torch.zeros_like(kc)
        else:
            kc = torch.zeros((pg.num_blocks, case.Hkv, case.D // 8, case.B, 8),
                             dtype=torch.bfloat16, device=dev)
            vc = torch.zeros((pg.num_blocks, case.Hkv, case.B // 8, case.D, 8),
                             dtype=torch.bfloat16, device=dev)
        pa.reshape_and_cache(key, value, kc, vc, slots_all, layout=layout)
        caches.append((kc, vc))
    rows = torch.from_numpy(case.new_token_rows()).to(dev)
    new_k = key[rows].contiguous()
    new_v = value[rows].contiguous()
    new_slots = slots_all[rows].contiguous()
    del key, value
    q = case.query.to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(pg.lens).to(dev)
    max_ctx = int(pg.lens.max())
    P = case.partition_tokens if args.partition_tokens is None else args.partition_tokens
    ws = torch.zeros(max(1, pa.decode_workspace_size(case.S, case.Hq, case.Hkv, case.D, max_ctx, P)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((case.S, case.Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    fused = not args.separate_cache_write

    def decode_call(i):
        kc, vc = caches[i % pools]
        if f8:
            pa.paged_decode_attn_fp8(q, kc, vc, bt, cl, case.scale, max_ctx, k_scale, v_scale,
                                     partition_tokens=P, new_key=new_k if fused else None,
                                     new_value=new_v if fused else None,
                                     slot_mapping=new_slots if fused else None, out=out, lse=lse,
                                     workspace=ws)
        elif std:  # same kernel over the standard layout
            pa.paged_decode_attn_layout(layout, q, kc, vc, bt, cl, case.scale, max_ctx,
                                        partition_tokens=P, new_key=new_k if fused else None,
                                        new_value=new_v if fused else None,
                                        slot_mapping=new_slots if fused else None, out=out,
                                        lse=lse, workspace=ws)
        elif fused:  # the new tokens' cache write inside the decode launch
            pa.paged_decode_attn_write(q, new_k, new_v, new_slots, kc, vc, bt, cl, case.scale,
                                       max_ctx, partition_tokens=P, out=out, lse=lse, workspace=ws)
        else:
            pa.paged_decode_attn(q, kc, vc, bt, cl, case.scale, max_ctx, partition_tokens=P,
                                 out=out, lse=lse, workspace=ws)

    # each pool's call checked and marshalled once (pa.prepare); a launch is
    # then one C call, so the host enqueues faster than the GPU runs them
    prepared = [pa.prepare(decode_call, i) for i in range(pools)]

    def decode(i):
        prepared[i % pools]()

    def step(i):
        if not fused:
            kc, vc = caches[i % pools]
            if f8:
                pa.reshape_and_cache_fp8(new_k, new_v, kc, vc, new_slots, k_scale, v_scale)
            else:
                pa.reshape_and_cache(new_k, new_v, kc, vc, new_slots, layout=layout)
        decode(i)

    # eager reference for the graph check
    step(0)
    torch.cuda.synchronize()
    ref_out = out.clone()

    stream = torch.cuda.Stream()
    graphs = []
    if not args.no_graph:
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for i in range(pools):  # warm the capture stream
                step(i)
        torch.cuda.synchronize()
        for i in range(pools):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()

    # A step is timed as eager launches unless asked otherwise: with the
    # fused cache write the step is one launch, and a graph replay costs
    # ~5 us more per step on this stack (25.0 vs 20.3 us measured).
    replay = bool(graphs) and args.graph_timing

    def run(i):
        if replay:
            graphs[i % pools].replay()
        else:
            step(i)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # a graph replay recomputes pool 0's step output bit for bit
    graph_ok = None
    if graphs:
        graphs[0].replay()
        torch.cuda.synchronize()
        graph_ok = bool(torch.equal(out.view(torch.int16), ref_out.view(torch.int16)))

    # the decode kernel's own duration: HIP events on the launch stream between
    # back-to-back launches (rotating pools)
    stats = launch_stats(decode, 240)
    dec_ms = stats["avg_ms"]

    algo = gqa_algorithmic_bytes(case, with_write=fused, kv_bytes=kv_bytes)
    achieved = algo / (dec_ms * 1e-3) / 1e9
    tok_s = case.S / (ms_per_step * 1e-3)
    # the same blocks read through the same block table over the same
    # rotating pools, with no arithmetic (preshuffled layouts only)
    gather = None
    if not args.no_read_ceiling and not std:
        gsink = torch.empty(case.S * case.Hkv * ((bt.shape[1] + 3) // 4), dtype=torch.int32,
                            device=dev)
        gstats = launch_stats(lambda i: pa.gather_read(caches[i % pools][0], caches[i % pools][1],
                                                       bt, cl, gsink, verify=False), 240)
        gather = {"kernel": "gather_read_kernel (pa_gather_read)",
                  "avg_launch_ms": gstats["avg_ms"],
                  "gbps": algo / (gstats["avg_ms"] * 1e-3) / 1e9,
                  "decode_frac_of_gather": gstats["avg_ms"] / dec_ms,
                  "note": "K and V of every block a decode reads, one wave per block, "
                          "no arithmetic; gbps counts the decode's algorithmic bytes"}
    return {
        "gather_ceiling": gather,
        "value": tok_s,
        "ms_per_step": ms_per_step,
        "graph_replay_matches_eager": graph_ok,
        "decode_ms": dec_ms,
        "launch_stats": stats,
        "hbm_gbps": achieved,
        "pct_hbm_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "algo_bytes": algo,
        "algo_flops": gqa_algorithmic_flops(case),
        "pools": pools,
        "cache_write": "fused" if fused else "separate launch",
        "kv_layout": args.kv_layout,
        "kv_dtype": args.kv_dtype,
        "kv_scales": (k_scale, v_scale) if f8 else None,
        "step_launch": "graph replay" if replay else "eager",
        "partition_tokens": ("balanced" if pa.decode_uses_balanced_split(case.S, case.Hkv, max_ctx, P)
                             else pa.decode_partition_tokens(case.S, case.Hkv, max_ctx, P)),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def time_oracle(step, units, unit, seconds, sample, omp=True):
    """The oracle's throughput on this host: one untimed warm-up step, then
    three runs of about seconds/4 each (the median is the value), then a run
    of about seconds/4 on one thread.  `units` counted per step.  omp: the
    step is the C oracle (OpenMP threads); otherwise numpy on one BLAS
    thread throughout."""
    import oracle
    from threadpoolctl import threadpool_limits
    orc = oracle.get()

    def run(budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            step()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return units * reps / el, reps, el

    cores = orc.max_threads() if omp else 1
    with threadpool_limits(1, user_api="blas"):
        step()
        runs = [run(seconds / 4) for _ in range(3)]
        if omp:
            orc.set_threads(1)
            try:
                one = run(seconds / 4)
            finally:
                orc.set_threads(cores)
        else:
            one = sorted(runs)[1]
    vals = sorted(r[0] for r in runs)
    return {"value": vals[1], "unit": unit, "cores": cores, "kind": "oracle",
            "runs": [r[0] for r in runs], "one_thread_value": one[0],
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"{sample}; median of 3 runs ({sum(r[1] for r in runs)} steps in "
                      f"{sum(r[2] for r in runs):.1f} s) after a warm-up step, then "
                      f"{one[1]} step(s) on one thread, fp64"}


def cpu_baseline_gqa(case, seconds, kv_layout="shuffled", kv_scales=None):
    """The oracle as it stands on this host: decode steps (cache write of the
    new tokens + exact attention through the block table), repeated for
    about `seconds`.  The oracle of the step's own cache: the shuffled bf16
    cache (C, fp64), the standard-layout one (shuffled on the fly, then the
    same C decode) or the FP8 one (numpy, fp64 over the dequantised values;
    every step covers a sample of the requests)."""
    import oracle
    from oracle import fp8 as OF
    from paged_attention_decode_reshape_amd import workloads as W

    orc = oracle.get()
    pg = case.paging
    rows = case.new_token_rows()
    kb, vb = W.bf16_bits(case.key), W.bf16_bits(case.value)
    nk, nv, ns = kb[rows], vb[rows], pg.slot_mapping[rows]
    qb = W.bf16_bits(case.query)
    seqs = list(range(case.S))
    if kv_scales is not None:
        ks, vs = kv_scales
        kc, vc = OF.empty_cache(pg.num_blocks, case.Hkv, case.D, case.B)
        OF.cache_write(kb, vb, pg.slot_mapping, kc, vc, ks, vs)
        seqs = seqs[::8]  # the numpy decode takes ~20 ms per request

        def step():
            OF.cache_write(nk, nv, ns, kc, vc, ks, vs)
            OF.paged_decode_gqa(qb, kc, vc, pg.block_table, case.context_lens, case.scale, ks,
                                vs, seqs=seqs)
    elif kv_layout == "standard":
        kc, vc = orc.empty_standard_cache(pg.num_blocks, case.B, case.Hkv, case.D)
        orc.cache_write_standard(kb, vb, pg.slot_mapping, kc, vc)

        def step():
            orc.cache_write_standard(nk, nv, ns, kc, vc)
            orc.paged_decode_gqa_standard(qb, kc, vc, pg.block_table, case.context_lens,
                                          case.scale)
    else:
        kc, vc = orc.empty_shuffled_cache(pg.num_blocks, case.Hkv, case.D, case.B)
        orc.cache_write_shuffled(kb, vb, pg.slot_mapping, kc, vc, case.B)

        def step():
            orc.cache_write_shuffled(nk, nv, ns, kc, vc, case.B)
            orc.paged_decode_gqa(qb, kc, vc, pg.block_table, case.context_lens, case.B,
                                 case.scale)
    what = ("FP8 numpy oracle, every 8th request" if kv_scales is not None else
            "standard-layout cache, shuffled on the fly" if kv_layout == "standard" else
            "shuffled bf16 cache")
    return time_oracle(step, len(seqs), "tok/s", seconds,
                       f"decode steps of the same workload ({len(seqs)} of {case.S} requests "
                       f"per step, {what})", omp=kv_scales is None)


def cpu_baseline_mixed(case, seconds):
    """The oracle's extend definition over the whole mixed batch (decode,
    extend and prefill requests alike), repeated for about `seconds`."""
    import oracle
    from paged_attention_decode_reshape_amd import workloads as W

    orc = oracle.get()
    pg = case.paging
    kb, vb = W.bf16_bits(case.key), W.bf16_bits(case.value)
    kc, vc = orc.empty_shuffled_cache(pg.num_blocks, case.Hkv, case.D, case.B)
    orc.cache_write_shuffled(kb, vb, pg.slot_mapping, kc, vc, case.B)
    rows = case.new_rows()
    kn, vn = kb[rows], vb[rows]
    qb = W.bf16_bits(case.query)
    def step():
        orc.extend(qb, kn, vn, case.query_start_loc, kc, vc, case.paging.block_table,
                   case.ctx_lens, case.B, case.scale)
    tokens = int(case.query_start_loc[-1])
    return time_oracle(step, tokens, "new tok/s", seconds,
                       f"passes over the whole mixed batch ({tokens} new tokens)")


# ---------------------------------------------------------------------------
# MLA decode
# ---------------------------------------------------------------------------

VALU_PEAK_TFLOPS = 157.3  # fp32 vector (bf16 dot2 issues at the same rate)
MFMA_BF16_PEAK_TFLOPS = 2500.0


def mla_algorithmic_bytes(case, with_write=False, kv_bytes=2) -> int:
    """Every context latent row once (kv_bytes per value: 2 bf16, 1 FP8),
    q, out, lse, used table entries and lengths (and, with the fused cache
    write, each new bf16 latent read and its cache row written, plus its
    slot)."""
    n = case.context_lens.astype(np.int64)
    lat = int(n.sum()) * case.Dl * kv_bytes
    blocks = int(((n + case.B - 1) // case.B).sum())
    write = case.S * case.Dl * (2 + kv_bytes) + case.S * 8 if with_write else 0
    return (lat + case.S * case.Hq * (case.Dl + case.Dv) * 2 + case.S * case.Hq * 4 + blocks * 4 +
            case.S * 4 + write)


def mla_algorithmic_flops(case) -> int:
    return int(case.context_lens.astype(np.int64).sum()) * case.Hq * (case.Dl + case.Dv) * 2


def bench_mla(args, case, label):
    import torch
    import paged_attention_decode_reshape_amd as pa

    dev = torch.device("cuda:0")
    pg = case.paging
    f8 = args.kv_dtype == "fp8"
    kv_bytes = 1 if f8 else 2
    pool_bytes = pg.num_blocks * case.B * case.Dl * kv_bytes
    pools = args.pools or max(1, math.ceil(2 * MALL_BYTES / pool_bytes))
    log(f"[bench] {label}: S={case.S} Hq={case.Hq} B={case.B} tokens={pg.total_tokens} "
        f"pool={pool_bytes / 1e6:.1f} MB x {pools} copies, {args.kv_dtype} cache")
    lat = case.latent.to(dev)
    # FP8: one scale for the cache, the latents' amax over the largest code
    kvs = float(np.float32(lat.float().abs().max().item() / 448.0)) if f8 else 1.0
    slots_all = torch.from_numpy(pg.slot_mapping).to(dev)
    caches = []
    for _ in range(pools):
        if f8:
            kv = torch.zeros((pg.num_blocks, case.B, case.Dl), dtype=torch.uint8, device=dev)
            pa.reshape_and_cache_mla_fp8(lat, kv, slots_all, kvs)
        else:
            kv = torch.zeros((pg.num_blocks, case.B, case.Dl), dtype=torch.bfloat16, device=dev)
            pa.reshape_and_cache(lat, None, kv, None, slots_all, layout=pa.LAYOUT_MLA_LATENT)
        caches.append(kv)
    rows = torch.from_numpy(case.new_token_rows()).to(dev)
    new_lat = lat[rows].contiguous()
    new_slots = slots_all[rows].contiguous()
    del lat
    q = case.query.to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(pg.lens).to(dev)
    max_ctx = int(pg.lens.max())
    P = 0 if args.partition_tokens is None else args.partition_tokens
    ws = torch.zeros(max(1, pa.mla_workspace_size(case.S, case.Hq, case.Dv, max_ctx, P)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((case.S, case.Hq, case.Dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.S, case.Hq), dtype=torch.float32, device=dev)

    fused = not args.separate_cache_write
    mfma = args.mla_engine == "mfma"

    def decode_call(i):
        if mfma and f8:
            pa.mla_decode_attn_fp8_mfma(q, caches[i % pools], bt, cl, case.scale, max_ctx, kvs,
                                        v_dim=case.Dv, partition_tokens=P,
                                        new_latent=new_lat if fused else None,
                                        slot_mapping=new_slots if fused else None, out=out,
                                        lse=lse, workspace=ws)
        elif mfma:
            pa.mla_decode_attn_mfma(q, caches[i % pools], bt, cl, case.scale, max_ctx,
                                    v_dim=case.Dv, partition_tokens=P,
                                    new_latent=new_lat if fused else None,
                                    slot_mapping=new_slots if fused else None, out=out, lse=lse,
                                    workspace=ws)
        elif f8:
            pa.mla_decode_attn_fp8(q, caches[i % pools], bt, cl, case.scale, max_ctx, kvs,
                                   v_dim=case.Dv, partition_tokens=P,
                                   new_latent=new_lat if fused else None,
                                   slot_mapping=new_slots if fused else None, out=out, lse=lse,
                                   workspace=ws)
        elif fused:  # the new latents' cache write inside the decode launch
            pa.mla_decode_attn_write(q, new_lat, new_slots, caches[i % pools], bt, cl, case.scale,
                                     max_ctx, v_dim=case.Dv, partition_tokens=P, out=out, lse=lse,
                                     workspace=ws)
        else:
            pa.mla_decode_attn(q, caches[i % pools], bt, cl, case.scale, max_ctx, v_dim=case.Dv,
                               partition_tokens=P, out=out, lse=lse, workspace=ws)

    prepared = [pa.prepare(decode_call, i) for i in range(pools)]

    def decode(i):
        prepared[i % pools]()

    def step(i):
        if not fused and f8:
            pa.reshape_and_cache_mla_fp8(new_lat, caches[i % pools], new_slots, kvs)
        elif not fused:
            pa.reshape_and_cache(new_lat, None, caches[i % pools], None, new_slots,
                                 layout=pa.LAYOUT_MLA_LATENT)
        decode(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    stats = launch_stats(decode, 240)
    dec_ms = stats["avg_ms"]
    algo = mla_algorithmic_bytes(case, with_write=fused, kv_bytes=kv_bytes)
    flops = mla_algorithmic_flops(case)
    # MLA picks its split like GQA decode with one unit per sequence
    balanced = pa.decode_uses_balanced_split(case.S, 1, max_ctx, P)
    return {"value": case.S / (ms_per_step * 1e-3), "ms_per_step": ms_per_step,
            "decode_ms": dec_ms, "launch_stats": stats, "algo_bytes": algo, "algo_flops": flops,
            "hbm_gbps": algo / (dec_ms * 1e-3) / 1e9, "tflops": flops / (dec_ms * 1e-3) / 1e12,
            "pools": pools, "cache_write": "fused" if fused else "separate launch",
            "kv_scale": kvs if f8 else None,
            "kernel": ("mla_decode_balanced_kernel" if balanced else "mla_decode_kernel")
                      + (f"<{'fp8' if f8 else 'bf16'}, matrix cores>" if mfma else "")}


def cpu_baseline_mla(case, seconds, kv_scale=None):
    """The oracle's MLA decode over the whole batch, repeated for about
    `seconds`; with kv_scale, the FP8 numpy oracle on one BLAS thread."""
    import oracle
    from oracle import fp8 as OF
    from paged_attention_decode_reshape_amd import workloads as W

    orc = oracle.get()
    qb = W.bf16_bits(case.query)
    if kv_scale is None:
        kv = np.zeros((case.paging.num_blocks, case.B, case.Dl), dtype=np.uint16)
        orc.cache_write_latent(W.bf16_bits(case.latent), case.paging.slot_mapping, kv, case.B)

        def step():
            orc.paged_decode_mla(qb, kv, case.paging.block_table, case.context_lens, case.B,
                                 case.Dv, case.scale)
    else:
        kv = np.zeros((case.paging.num_blocks, case.B, case.Dl), dtype=np.uint8)
        OF.cache_write_latent(W.bf16_bits(case.latent), case.paging.slot_mapping, kv, kv_scale)

        def step():
            OF.paged_decode_mla(qb, kv, case.paging.block_table, case.context_lens, case.Dv,
                                case.scale, kv_scale)
    return time_oracle(step, case.S, "tok/s", seconds,
                       f"full MLA decode steps of the same workload ({case.S} requests"
                       f"{', FP8 numpy oracle' if kv_scale is not None else ''})",
                       omp=kv_scale is None)


# ---------------------------------------------------------------------------
# chunked extend
# ---------------------------------------------------------------------------

def extend_algorithmic_flops(case) -> int:
    n = case.new_lens.astype(np.int64)
    c = case.ctx_lens.astype(np.int64)
    pairs = int((n * c).sum() + (n * (n + 1) // 2).sum())
    return pairs * case.Hq * case.D * 4


def mixed_case():
    """One serving-shaped mixed batch: 60 decode requests (contexts
    U[1000,2000]), 3 extend requests (256 new tokens over ~4000 cached) and
    1 prefill of 512 tokens, interleaved; 8 q heads on 1 kv head."""
    from paged_attention_decode_reshape_amd import workloads as W
    rng = np.random.default_rng(1006)
    ctx = list(rng.integers(1000, 2001, size=60)) + [4000, 4100, 3900, 0]
    new = [1] * 60 + [256, 256, 256, 512]
    perm = rng.permutation(len(ctx))
    return W.extend_case("mixed_batch", 1006, ctx_lens=[ctx[i] for i in perm],
                         new_tokens=[new[i] for i in perm], Hq=8, Hkv=1, D=128, block_size=16)


def bench_mixed(args):
    """The routed call (pa_mixed_batch_attn: cache write, decode, extend and
    prefill paths) on one reordered mixed batch, eager launches."""
    import torch
    import paged_attention_decode_reshape_amd as pa

    dev = torch.device("cuda:0")
    case = mixed_case()
    pg = case.paging
    new_rows = case.new_rows()
    is_new = np.zeros(pg.total_tokens, dtype=bool)
    is_new[new_rows] = True
    cached = np.nonzero(~is_new)[0]
    kc = torch.zeros((pg.num_blocks, case.Hkv, case.D // 8, case.B, 8), dtype=torch.bfloat16,
                     device=dev)
    vc = torch.zeros((pg.num_blocks, case.Hkv, case.B // 8, case.D, 8), dtype=torch.bfloat16,
                     device=dev)
    pa.reshape_and_cache(case.key[cached].to(dev), case.value[cached].to(dev), kc, vc,
                         torch.from_numpy(pg.slot_mapping[cached]).to(dev))
    qsl = case.query_start_loc
    order, counts = pa.mixed_batch_plan(qsl, case.ctx_lens)
    starts = np.cumsum(np.concatenate([[0], case.new_lens]))
    q_rows = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in order])
    n_rows = np.concatenate([new_rows[starts[r]:starts[r + 1]] for r in order])
    new_qsl = np.concatenate([[0], np.cumsum(case.new_lens[order])]).astype(np.int32)
    ctx = case.ctx_lens[order].astype(np.int32)
    q = case.query[torch.from_numpy(q_rows)].to(dev).contiguous()
    k = case.key[torch.from_numpy(n_rows)].to(dev).contiguous()
    v = case.value[torch.from_numpy(n_rows)].to(dev).contiguous()
    slots = torch.from_numpy(pg.slot_mapping[n_rows]).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(pg.block_table[order])).to(dev)
    qsl_d = torch.from_numpy(new_qsl).to(dev)
    ctx_d = torch.from_numpy(ctx).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], case.Hq), dtype=torch.float32, device=dev)
    nbytes = int(pa.library().pa_mixed_batch_workspace_size(
        len(ctx), new_qsl.ctypes.data, ctx.ctypes.data, case.Hq, case.Hkv, case.D, case.B,
        case.chunk_budget_tokens))
    ws = torch.zeros(max(1, nbytes), dtype=torch.uint8, device=dev)

    def step(i):
        pa.mixed_batch_attn(q, k, v, slots, qsl_d, ctx_d, kc, vc, bt, case.scale, new_qsl, ctx,
                            chunk_budget_tokens=case.chunk_budget_tokens, out=out, lse=lse,
                            workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    tokens = int(new_qsl[-1])
    return {"value": tokens / (ms * 1e-3), "ms_per_step": ms, "counts": [int(c) for c in counts],
            "new_tokens": tokens, "cached_tokens": int(ctx.sum())}


def bench_cache_write(args):
    """Bulk reshape_and_cache: every token of the 64-request workload (93.5 K
    tokens, one kv head, head_dim 128) written into the shuffled cache in one
    launch, over rotated pools larger than the Infinity Cache."""
    import torch
    import paged_attention_decode_reshape_amd as pa
    from paged_attention_decode_reshape_amd import workloads as W

    dev = torch.device("cuda:0")
    case = W.qwen3_decode()
    pg = case.paging
    pool_bytes = pg.num_blocks * case.Hkv * case.D * case.B * 2 * 2
    pools = max(2, math.ceil(2 * MALL_BYTES / pool_bytes))
    key, value = case.key.to(dev), case.value.to(dev)
    slots = torch.from_numpy(pg.slot_mapping).to(dev)
    caches = [(torch.zeros((pg.num_blocks, 1, 16, 16, 8), dtype=torch.bfloat16, device=dev),
               torch.zeros((pg.num_blocks, 1, 2, 128, 8), dtype=torch.bfloat16, device=dev))
              for _ in range(pools)]
    srcs = [(key.clone(), value.clone()) for _ in range(pools)]

    def launch(i):
        kc, vc = caches[i % pools]
        k, v = srcs[i % pools]
        pa.reshape_and_cache(k, v, kc, vc, slots)

    stats = launch_stats(launch, 240)
    ms = stats["avg_ms"]
    T = pg.total_tokens
    nbytes = T * case.Hkv * case.D * 2 * 2 * 2 + T * 8
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"value": T / (ms * 1e-3), "ms_per_step": ms, "algo_bytes": nbytes, "gbps": gbps,
            "tokens": T, "pools": pools, "launch_stats": stats}


def bench_merge(args):
    """The standalone merge_attn_states at the chunked-extend shape: two fp32
    partial results [4096, 64, 128] with their LSEs -> bf16 output and LSE
    (one context-chunk merge of the pages' extend loop), over rotated copies
    larger than the Infinity Cache; HIP events over back-to-back launches."""
    import torch
    import paged_attention_decode_reshape_amd as pa

    T, H, D = 4096, 64, 128
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(1007)
    per = 2 * T * H * D * 4 + 2 * T * H * 4
    copies = max(2, math.ceil(2 * MALL_BYTES / per))
    sets = []
    for _ in range(copies):
        po = torch.randn((T, H, D), generator=g).to(dev)
        so = torch.randn((T, H, D), generator=g).to(dev)
        pl = (torch.randn((T, H), generator=g) * 3).to(dev)
        sl = (torch.randn((T, H), generator=g) * 3).to(dev)
        sets.append((po, pl, so, sl))
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)

    def launch(i):
        po, pl, so, sl = sets[i % copies]
        pa.merge_attn_states(po, pl, so, sl, out=out, out_lse=lse)

    stats = launch_stats(launch, 240)
    ms = stats["avg_ms"]
    nbytes = per + T * H * D * 2 + T * H * 4
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"value": T / (ms * 1e-3), "ms_per_step": ms, "algo_bytes": nbytes, "gbps": gbps,
            "copies": copies, "launch_stats": stats}


def bench_extend(args, case, label):
    import torch
    import paged_attention_decode_reshape_amd as pa

    dev = torch.device("cuda:0")
    pg = case.paging
    log(f"[bench] {label}: S={case.S} new={int(case.new_lens.sum())} "
        f"context={int(case.ctx_lens.sum())} tokens, budget {case.chunk_budget_tokens}")
    kc = torch.zeros((pg.num_blocks, case.Hkv, case.D // 8, case.B, 8), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((pg.num_blocks, case.Hkv, case.B // 8, case.D, 8), dtype=torch.bfloat16, device=dev)
    pa.reshape_and_cache(case.key.to(dev), case.value.to(dev), kc, vc,
                         torch.from_numpy(pg.slot_mapping).to(dev))
    rows = torch.from_numpy(case.new_rows())
    k_new = case.key[rows].to(dev).contiguous()
    v_new = case.value[rows].to(dev).contiguous()
    q = case.query.to(dev)
    qsl = torch.from_numpy(case.query_start_loc).to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(case.ctx_lens).to(dev)
    Tn = int(case.query_start_loc[-1])
    ws = torch.zeros(pa.extend_workspace_size(case.S, Tn, case.Hq, case.Hkv, case.D, case.B,
                                              case.chunk_budget_tokens), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((Tn, case.Hq), dtype=torch.float32, device=dev)

    def call(i):
        pa.chunked_extend_attn(q, k_new, v_new, qsl, kc, vc, bt, cl, case.scale,
                               case.query_start_loc, case.ctx_lens,
                               chunk_budget_tokens=case.chunk_budget_tokens, out=out, lse=lse,
                               workspace=ws)

    for i in range(max(1, args.warmup)):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stats = launch_stats(call, 200)
    ev_ms = stats["avg_ms"]
    flops = extend_algorithmic_flops(case)

    # The context gather on its own (pa_gather_cache_chunk, the pages'
    # cp_mha_gather_cache): one pass = every iteration of the chunk plan,
    # each request's context copied out once (bytes read + written).
    c = pa.extend_chunk_tokens(case.S, case.B, case.chunk_budget_tokens)
    iters = -(-int(case.ctx_lens.max()) // c)
    ko = torch.empty((case.S * c, case.Hkv, case.D), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)

    def gather_pass(i):
        for it in range(iters):
            pa.gather_cache_chunk(kc, vc, bt, cl, it, c, k_out=ko, v_out=vo)

    g_ms = time_launches(gather_pass, max(3, args.steps // 20))
    g_bytes = int(case.ctx_lens.astype(np.int64).sum()) * case.Hkv * case.D * 2 * 2 * 2
    return {"value": Tn / (ms * 1e-3), "ms_per_step": ms, "call_ms": ev_ms, "launch_stats": stats,
            "algo_flops": flops,
            "tflops": flops / (ev_ms * 1e-3) / 1e12,
            "gather": {"kernel": "gather_chunk_kernel", "chunk_tokens": c, "iterations": iters,
                       "ms_per_pass": g_ms, "algo_bytes_per_pass": g_bytes,
                       "gbps": g_bytes / (g_ms * 1e-3) / 1e9}}


def cpu_baseline_extend(case, seconds):
    """The oracle's extend (the definition, fp64) on a bounded sample: two
    new tokens (all 64 q heads) over the first request's context."""
    import oracle
    from paged_attention_decode_reshape_amd import workloads as W

    orc = oracle.get()
    sub = W.extend_case("extend_sample", 1005, ctx_lens=[int(case.ctx_lens[0])], new_tokens=[2],
                        Hq=case.Hq, Hkv=case.Hkv, D=case.D, block_size=case.B)
    rows = sub.new_rows()
    kc, vc = orc.empty_shuffled_cache(sub.paging.num_blocks, sub.Hkv, sub.D, sub.B)
    orc.cache_write_shuffled(W.bf16_bits(sub.key), W.bf16_bits(sub.value), sub.paging.slot_mapping,
                             kc, vc, sub.B)
    kn, vn, qb = W.bf16_bits(sub.key)[rows], W.bf16_bits(sub.value)[rows], W.bf16_bits(sub.query)
    def step():
        orc.extend(qb, kn, vn, sub.query_start_loc, kc, vc, sub.paging.block_table, sub.ctx_lens,
                   sub.B, sub.scale)
    return time_oracle(step, 2, "new tok/s", seconds,
                       f"runs of 2 new tokens over a {int(case.ctx_lens[0])}-token context "
                       f"(64 q heads)")


def copy_calibration(mb):
    """Plain device-to-device copies of a known size: rocprofv3 memory counters
    read on them give the scale between counter units and bytes."""
    import torch
    n = mb << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 5 copies of {mb} MiB")


def main():
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library's "
              "path has no multi-GPU leg", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    from paged_attention_decode_reshape_amd import workloads as W
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb)

    if args.config == "qwen3":
        case = W.qwen3_decode()
        r = bench_gqa(args, case, "qwen3_decode_64req")
        workload = {"workload": "qwen3_235b_tp8_decode_64req", "requests": 64, "q_heads": 8,
                    "kv_heads": 1, "head_dim": 128, "block_size": 16,
                    "context_lens": "U[1000,2000]", "kv_layout": r["kv_layout"], "kv_dtype": r["kv_dtype"],
                    "kv_pool_copies": r["pools"], "partition_tokens": r["partition_tokens"],
                    "cache_write": r["cache_write"], "step_launch": r["step_launch"]}
    elif args.config == "qwen3_10k":
        case = W.qwen3_decode(lens_range=(10000, 11000))
        r = bench_gqa(args, case, "qwen3_decode_64req_10k")
        workload = {"workload": "qwen3_235b_tp8_decode_64req_10k", "requests": 64, "q_heads": 8,
                    "kv_heads": 1, "head_dim": 128, "block_size": 16,
                    "context_lens": "U[10000,11000]", "kv_layout": r["kv_layout"], "kv_dtype": r["kv_dtype"],
                    "kv_pool_copies": r["pools"], "partition_tokens": r["partition_tokens"],
                    "cache_write": r["cache_write"], "step_launch": r["step_launch"]}
    elif args.config == "long_context":
        case = W.long_context_decode()
        r = bench_gqa(args, case, "long_context_decode")
        workload = {"workload": "long_context_gqa_decode_8req", "requests": 8, "q_heads": 64,
                    "kv_heads": 4, "head_dim": 128, "block_size": 16,
                    "context_lens": "U[32768,131072]", "kv_layout": r["kv_layout"], "kv_dtype": r["kv_dtype"],
                    "kv_pool_copies": r["pools"],
                    "partition_tokens": r["partition_tokens"], "cache_write": r["cache_write"]}
    elif args.config in ("mla", "mla_bs1"):
        B = 1 if args.config == "mla_bs1" else 64
        case = W.deepseek_mla_decode(block_sizes=(B,))[B]
        r = bench_mla(args, case, f"deepseek_mla_decode_bs{B}")
        workload = {"workload": f"deepseek_r1_tp8_mla_decode_64req_bs{B}", "requests": 64,
                    "q_heads": 16, "latent_dim": 576, "v_dim": 512, "block_size": B,
                    "context_lens": "U[1024,4096]", "kv_pool_copies": r["pools"],
                    "cache_write": r["cache_write"], "kv_dtype": args.kv_dtype}
        if r["kv_scale"] is not None:
            workload["kv_scale"] = r["kv_scale"]
        line = base_line(args, r, workload)
        line["hbm_gbps"] = r["hbm_gbps"]
        line["pct_hbm_peak"] = 100.0 * r["hbm_gbps"] / HBM_PEAK_GBPS
        if not args.no_read_ceiling:
            rc = read_ceiling(r["algo_bytes"])
            rc["decode_frac_of_ceiling"] = r["hbm_gbps"] / rc["gbps"]
            line["hbm_read_ceiling"] = rc
        if args.mla_engine == "mfma":
            # matrix cores: the latent read bounds it; the bf16 MFMA fraction
            # (algorithmic flops; P.V runs twice, hi and lo parts) is reported beside
            line["config"]["engine"] = "matrix cores"
            line["roofline"] = {"bound": "hbm", "kernel": r["kernel"], "achieved": r["hbm_gbps"],
                                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": r["hbm_gbps"] / HBM_PEAK_GBPS,
                                "traffic": measured_traffic(
                                    args.config + ("_fp8" if args.kv_dtype == "fp8" else "")
                                    + "_mfma", default_launch(args)),
                                "algo_bytes_per_launch": r["algo_bytes"],
                                "avg_launch_ms": r["decode_ms"],
                                "launch_stats": r["launch_stats"],
                                "mfma_tflops": r["tflops"],
                                "mfma_frac_of_bf16_peak": r["tflops"] / MFMA_BF16_PEAK_TFLOPS}
        else:
            line["roofline"] = {"bound": "alu", "kernel": r["kernel"], "achieved": r["tflops"],
                                "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": r["tflops"] / VALU_PEAK_TFLOPS,
                                "traffic": measured_traffic(
                                    args.config + ("_fp8" if args.kv_dtype == "fp8" else ""),
                                    default_launch(args)),
                                "algo_flops_per_launch": r["algo_flops"],
                                "algo_bytes_per_launch": r["algo_bytes"],
                                "avg_launch_ms": r["decode_ms"],
                                "launch_stats": r["launch_stats"]}
        if not args.no_cpu_baseline:
            log("[bench] timing the oracle on the host cores")
            line["cpu_baseline"] = cpu_baseline_mla(case, args.cpu_seconds, r["kv_scale"])
        emit(line, ("mla",))
        return
    elif args.config == "cache_write":
        r = bench_cache_write(args)
        workload = {"workload": "reshape_and_cache_bulk_93k_tokens", "tokens": r["tokens"],
                    "kv_heads": 1, "head_dim": 128, "block_size": 16, "layout": "shuffled",
                    "pools": r["pools"]}
        line = base_line(args, r, workload, unit="tokens/s")
        line["roofline"] = {"bound": "hbm", "kernel": "cache_write_runs_kernel",
                            "achieved": r["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": r["gbps"] / HBM_PEAK_GBPS,
                            "traffic": measured_traffic(args.config, default_launch(args)),
                            "algo_bytes_per_launch": r["algo_bytes"],
                            "avg_launch_ms": r["ms_per_step"],
                            "launch_stats": r["launch_stats"]}
        emit(line, ("cache_write",))
        return
    elif args.config == "merge":
        r = bench_merge(args)
        workload = {"workload": "merge_attn_states_4096x64x128", "tokens": 4096, "heads": 64,
                    "head_dim": 128, "inputs": "two fp32 partials + LSEs", "output": "bf16 + LSE",
                    "copies": r["copies"]}
        line = base_line(args, r, workload, unit="rows/s")
        line["dtype"] = "f32"
        line["roofline"] = {"bound": "hbm", "kernel": "merge_pair_kernel", "achieved": r["gbps"],
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": r["gbps"] / HBM_PEAK_GBPS,
                            "traffic": measured_traffic(args.config, default_launch(args)),
                            "algo_bytes_per_launch": r["algo_bytes"],
                            "avg_launch_ms": r["ms_per_step"],
                            "launch_stats": r["launch_stats"]}
        if not args.no_read_ceiling:
            rc = read_ceiling(r["algo_bytes"])
            rc["decode_frac_of_ceiling"] = r["gbps"] / rc["gbps"]
            line["hbm_read_ceiling"] = rc
        emit(line, ("merge",))
        return
    elif args.config == "mixed":
        r = bench_mixed(args)
        workload = {"workload": "mixed_batch_60dec_3ext_1pre", "requests": 64,
                    "decode_extend_prefill": r["counts"], "q_heads": 8, "kv_heads": 1,
                    "head_dim": 128, "block_size": 16, "new_tokens": r["new_tokens"],
                    "cached_tokens": r["cached_tokens"],
                    "step": "pa_mixed_batch_attn: cache write + decode + extend + prefill paths"}
        line = base_line(args, r, workload, unit="new tok/s")
        if not args.no_cpu_baseline:
            log("[bench] timing the oracle on the host cores")
            line["cpu_baseline"] = cpu_baseline_mixed(mixed_case(), args.cpu_seconds)
        emit(line, ("gqa", "extend"))
        return
    else:  # extend
        case = W.chunked_extend()
        r = bench_extend(args, case, "chunked_extend")
        workload = {"workload": "chunked_extend_16req_256new", "requests": 16, "new_tokens": 256,
                    "q_heads": 64, "kv_heads": 4, "head_dim": 128, "block_size": 16,
                    "context_lens": "U[8192,40960]", "chunk_budget_tokens": case.chunk_budget_tokens}
        line = base_line(args, r, workload, unit="new tok/s")
        line["roofline"] = {"bound": "mfma", "kernel": "extend_attn_kernel (+ plan, new-V shuffle, merge)",
                            "achieved": r["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": r["tflops"] / MFMA_BF16_PEAK_TFLOPS,
                            "traffic": measured_traffic(args.config, default_launch(args)),
                            "traffic_kernel": "extend_attn_kernel",
                            "algo_flops_per_call": r["algo_flops"],
                            "avg_call_ms": r["call_ms"],
                            "launch_stats": r["launch_stats"]}
        line["gather_pass"] = r["gather"]
        if not args.no_cpu_baseline:
            log("[bench] timing the oracle on the host cores")
            line["cpu_baseline"] = cpu_baseline_extend(case, args.cpu_seconds)
        emit(line, ("extend",))
        return

    line = base_line(args, r, workload)
    line.update({
        "hbm_gbps": r["hbm_gbps"],
        "pct_hbm_peak": r["pct_hbm_peak"],
        "graph_replay_matches_eager": r["graph_replay_matches_eager"],
        "roofline": {
            "bound": "hbm",
            "kernel": (("paged_decode_balanced_kernel (balanced split"
                        if r["partition_tokens"] == "balanced" else
                        "paged_decode_kernel (partitions")
                       + " + fused merge"
                       + (" + fused cache write" if r["cache_write"] == "fused" else "")
                       + (", standard layout" if r["kv_layout"] == "standard" else "")
                       + (", FP8 cache)" if r["kv_dtype"] == "fp8" else ")")),
            "achieved": r["hbm_gbps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": r["hbm_gbps"] / HBM_PEAK_GBPS,
            "traffic": measured_traffic(args.config + ("_fp8" if r["kv_dtype"] == "fp8" else ""),
                                        default_launch(args)),
            "algo_bytes_per_launch": r["algo_bytes"],
            "avg_launch_ms": r["decode_ms"],
            "launch_stats": r["launch_stats"],
        },
    })
    if not args.no_read_ceiling:
        rc = read_ceiling(r["algo_bytes"])
        rc["decode_frac_of_ceiling"] = r["hbm_gbps"] / rc["gbps"]
        line["hbm_read_ceiling"] = rc
        if r["gather_ceiling"] is not None:
            line["hbm_gather_ceiling"] = r["gather_ceiling"]
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores")
        line["cpu_baseline"] = cpu_baseline_gqa(case, args.cpu_seconds, r["kv_layout"],
                                                r["kv_scales"])
    emit(line, ("gqa",))


def emit(line, kinds):
    """Tag the line with the sha of the kernel sources it measured; print it."""
    files = []
    for k in kinds:
        files += [f for f in KERNEL_SOURCES[k] if f not in files]
    line["kernel_sources_sha16"] = sources_sha(files)
    print(json.dumps(line), flush=True)


def base_line(args, r, workload, unit="tok/s"):
    return {
        "metric": METRIC,
        "value": r["value"],
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": workload,
        "cpu_baseline": None,
    }


if __name__ == "__main__":
    main()
