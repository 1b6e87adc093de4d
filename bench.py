#!/usr/bin/env python3
"""Benchmark: one decode step of paged attention on one MI355X.

A step is, for each of the 16 layers, the append of this step's token of every
sequence into its page slot followed by batched paged decode attention over the
shared BF16 page pool, issued as one ``pa_append_decode`` call per layer (the
same work as ``pa_append`` + ``pa_decode``, which is timed too), all on one
stream, with every input already resident in HBM.  The default workload is the full-context batch: 64 sequences
at 2048 tokens, 16 layers, 32 query / 8 KV heads, head dim 64, 16-token pages
(4 GiB of K and V read per step).

Prints one JSON line: effective KV GB/s for the whole step (KV bytes the
attention must read / step time), µs per step, the roofline of the decode kernel
(algorithmic bytes per launch / launch time) and the FP64 CPU oracle timed on a
bounded sample of the same workload.

``--op fill`` measures the prefill page fill instead: every layer's prompt rows
(positions 0..L-2 of each sequence of the workload, packed one sequence after
another) written into the pool with one ``pa_fill`` per layer.

``--op prefill`` measures the causal prefill attention over the same prompts:
one ``pa_prefill`` per layer (each prompt's rows attend its own earlier rows),
reported in TFLOP/s of attention arithmetic (4 D flops per attended
(query, key) pair and query head) against the bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attn: effective KV GB/s (% HBM peak), µs/step at batch 64×2048"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_kernel_full_b64_l2048.md")
FILL_PROFILE = os.path.join(ROOT, "profiles", "fill_kernel_full_b64_l2047.md")
PREFILL_PROFILE = {"bf16x2": os.path.join(ROOT, "profiles", "prefill_kernel_full_b64_l2047.md"),
                   "fp16": os.path.join(ROOT, "profiles", "prefill_kernel_fp16w_full_b64_l2047.md")}
PREFILL_METRIC = ("prefill attention: TFLOP/s (causal GQA, 4*D flops per attended pair and query head), "
                  "µs/step at batch 64×2047")
MFMA_BF16_PEAK_TFLOPS = 2500.0
FILL_METRIC = "prefill page fill: effective GB/s (K/V rows read + written), µs/step at batch 64×2047"
ROPE_METRIC = ("RoPE + KV append: effective GB/s (q, new K/V and the table row read; rotated q and the pool "
               "rows written), µs/step at batch 64×2048")
ROPE_BYTES_PER_SEQ = 4096 + 4096 + 2 * 1024 + 2 * 1024 + 256  # q in/out, K/V in/out, one table row


def cpu_workers():
    """(workers, affinity): one oracle worker per host core this process may run on,
    capped at the CPU share the host grants one GPU job when it states one
    (OMP_NUM_THREADS, read before the workers set it to 1)."""
    aff = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    except ValueError:
        share = 0
    return max(1, min(aff, share) if share > 0 else aff), aff


def measured_traffic(profile=None, sources=("pa_kernels.hip", "pa_kernels.h")):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source (the given csrc files); else None."""
    import hashlib
    import re
    try:
        text = open(profile or TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m_sha = re.search(r"sha256[^`]*`([0-9a-f]{64})`", text)
    m_tr = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not (m_sha and m_tr):
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "paged_kv_cache_205_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return int(m_tr.group(1)) if h.hexdigest() == m_sha.group(1) else None


def decode_profile(sources=("pa_kernels.hip", "pa_kernels.h")):
    """The headline decode kernel's committed rocprofv3 summary: whether it was
    taken on the current kernel source, its calibrated HBM bytes per launch and
    the kernel's average duration under the tracer (None where absent)."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m_avg = re.search(r"kernel_avg_us: ([0-9.]+)", text)
    return {"traffic": measured_traffic(TRAFFIC_PROFILE, sources),
            "kernel_avg_us": float(m_avg.group(1)) if m_avg else None}


# Workloads timed beside the headline; a step of the cache-resident ones reads
# less than the 256 MB Infinity Cache, so each of their steps follows a 1 GiB write.
OTHER_CONFIGS = ("tiny", "small", "fragmented", "skewed", "large")
CACHE_RESIDENT = ("tiny", "small")


def time_workload(name, steps, warmup, stream_gbs, flush):
    """µs per step of one workload (one pa_append_decode per layer, automatic split),
    its sequence-steps/s and effective KV GB/s against the spec peak and the
    measured streaming read."""
    import torch
    from paged_kv_cache_205_amd import ops, synth
    dev = "cuda"
    lay = synth.get(name)
    t_gen = time.perf_counter()
    k_pool, v_pool = synth.make_pools(lay, dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
    inputs = [synth.step_inputs(lay, l, dev) for l in range(lay.n_layers)]
    outs = [torch.empty((lay.B, 32, 64), dtype=torch.float32, device=dev) for _ in range(lay.n_layers)]
    ws = ops.workspace_for(lay.B, lay.max_blocks, 0, dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    plan = torch.empty(ops.pa_decode_plan_bytes(lay.B, lay.max_blocks, 0), dtype=torch.uint8, device=dev)

    def step():
        for l in range(lay.n_layers):
            x = inputs[l]
            ops.pa_append_decode(x["k_new"], x["v_new"], k_pool, v_pool, x["q"], bt[l], seq_lens, lay.scale,
                                 out=outs[l], workspace=ws)

    def step_planned():
        ops.pa_decode_plan(seq_lens, lay.max_blocks, 0, plan=plan)
        for l in range(lay.n_layers):
            x = inputs[l]
            ops.pa_decode_planned(x["q"], k_pool, v_pool, bt[l], plan, lay.scale, k_new=x["k_new"], v_new=x["v_new"],
                                  out=outs[l], workspace=ws)

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(run):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        if name in CACHE_RESIDENT:
            times = []
            for _ in range(steps):
                flush.fill_(1.0)  # evicts the pool from the L2 caches and the Infinity Cache
                e0.record()
                run()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            return float(np.median(times))
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_unplanned = timed(step)
    ms_planned = timed(step_planned)
    ms = min(ms_unplanned, ms_planned)
    timing = ("median of the steps, each timed alone after a 1 GiB write (cold caches)" if name in CACHE_RESIDENT
              else "back-to-back stream launches (a step reads more than the Infinity Cache holds)")
    kv = lay.kv_bytes_per_step
    gbs = kv / (ms * 1e-3) / 1e9
    res = {
        "B": lay.B,
        "layers": lay.n_layers,
        "kv_bytes_per_step": kv,
        "us_per_step": round(ms * 1e3, 2),
        "us_per_launch": round(ms * 1e3 / lay.n_layers, 3),
        "seq_steps_per_s": round(lay.B / (ms * 1e-3), 1),
        "kv_GBps": round(gbs, 2),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "frac_stream_read": None if stream_gbs is None else round(gbs / stream_gbs, 4),
        "timing": timing,
        "step": "pa_decode_plan + planned launches" if ms == ms_planned else "pa_append_decode launches",
        "us_per_step_planned": round(ms_planned * 1e3, 2),
        "us_per_step_unplanned": round(ms_unplanned * 1e3, 2),
    }
    log(f"config {name}: {res['us_per_step']} us/step, {res['kv_GBps']} GB/s (inputs built in {t_gen:.1f} s)")
    del k_pool, v_pool, inputs, outs, ws, plan
    torch.cuda.empty_cache()
    return res


def _oracle_fill(item):
    """fill_ref for one (layer, sequence) of the fill sample; returns the rows written."""
    from oracle import fill_ref
    l, b = item
    d = _CPU[("fill", l)]
    kp, vp, bt = d["pages"][b]
    c0, c1 = int(d["cu"][b]), int(d["cu"][b + 1])
    fill_ref(kp, vp, d["k"][c0:c1], d["v"][c0:c1], bt, None, np.array([0, c1 - c0], np.int32))
    return c1 - c0


def cpu_baseline_fill(lay, n_layers: int, workers: int):
    """Time the oracle's fill on the first n_layers layers (each sequence into its own pages)."""
    import torch
    from paged_kv_cache_205_amd import synth
    torch.set_num_threads(1)
    layers = list(range(min(n_layers, lay.n_layers)))
    for l in layers:
        ks, vs, cu = synth.prefill_inputs(lay, l, "cpu")
        pages = {}
        for b in range(lay.B):
            n = max(synth.nblocks(int(lay.seq_lens[b]) - 1), 1)
            nan = np.full((n, 16, 8, 64), 0x7FC0, np.uint16)
            pages[b] = (nan, nan.copy(), np.arange(n, dtype=np.int32)[None])
        _CPU[("fill", l)] = dict(pages=pages, k=synth.bits(ks), v=synth.bits(vs), cu=cu.numpy())
    items = [(l, b) for l in layers for b in range(lay.B)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        rows = sum(pool.map(_oracle_fill, items, chunksize=1))
    tw = time.perf_counter() - t0
    return {
        "value": round(rows * 4096 / tw / 1e9, 6),  # 2 KiB of K and V read and 2 KiB written per row
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"layers 0..{layers[-1]} of the same prefill, all {lay.B} sequences each ({rows} rows): "
                  f"fill_ref (NumPy) in {workers} worker processes, {tw:.1f} s wall",
        "seconds": round(tw, 2),
    }


def bench_fill(args, lay):
    """One step = one pa_fill per layer of every sequence's prompt rows."""
    cpu = None
    if not args.no_cpu:
        workers, aff = cpu_workers()
        log(f"cpu baseline (fill): oracle on {workers} workers ...")
        cpu = cpu_baseline_fill(lay, args.cpu_layers, workers)
        cpu["affinity_cores"] = aff
    import torch
    from paged_kv_cache_205_amd import ops, synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ops.load()
    dev = "cuda"
    shape = (lay.num_pages, 16, 8, 64)
    k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    src = [synth.prefill_inputs(lay, l, dev) for l in range(lay.n_layers)]
    T = int(src[0][0].shape[0])
    bytes_launch = sum(int(x[0].shape[0]) for x in src) * 4096 // lay.n_layers
    if args.calib_copy_mib:
        a = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        torch.empty_like(a).copy_(a)
        del a
    torch.cuda.synchronize()

    def step():
        for l in range(lay.n_layers):
            ks, vs, cu = src[l]
            ops.pa_fill(ks, vs, k_pool, v_pool, bt[l], cu)

    for _ in range(args.warmup):
        step()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    launch_ms = ms_step / lay.n_layers
    value = bytes_launch * lay.n_layers / (ms_step * 1e-3) / 1e9
    res = {
        "metric": FILL_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"prefill fill of {lay.name}: B={lay.B} prompts of L-1 tokens, {lay.n_layers} layers, "
                        f"8 kv heads, D=64, 16-token BF16 pages",
            "batch": lay.B,
            "rows_per_layer": T,
            "layers": lay.n_layers,
            "bytes_per_step": bytes_launch * lay.n_layers,
            "timing": "stream launches",
            "parallelism": "single GPU",
        },
        "us_per_step": round(ms_step * 1e3, 2),
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": "fill_kernel (one launch per layer)",
            "bound": "hbm",
            "achieved": round(bytes_launch / (launch_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(bytes_launch / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(FILL_PROFILE) if lay.name == "full" else None,
            "bytes_per_launch": bytes_launch,
            "mean_launch_us": round(launch_ms * 1e3, 3),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def _oracle_rope(item):
    """rope_append_ref for one (layer, sequence) of the sample, into a one-page pool."""
    from oracle.rope import rope_append_ref
    l, b = item
    d = _CPU[("rope", l)]
    one = np.zeros((1, 16, 8, 64), np.uint16)
    rope_append_ref(d["q"][b:b + 1], d["k"][b:b + 1], d["v"][b:b + 1], d["table"], one, one.copy(),
                    np.zeros((1, 128), np.int32), d["L"][b:b + 1], np.zeros((1, 32, 64), np.uint16))
    return 1


def cpu_baseline_rope(lay, n_layers: int, workers: int):
    """Time the oracle's RoPE + append on every sequence of the first n_layers layers."""
    import torch
    from paged_kv_cache_205_amd import synth
    torch.set_num_threads(1)
    layers = list(range(min(n_layers, lay.n_layers)))
    table = synth.rope_table(2048).numpy()
    for l in layers:
        x = synth.step_inputs(lay, l, "cpu")
        _CPU[("rope", l)] = dict(q=synth.bits(x["q"]), k=synth.bits(x["k_new"]), v=synth.bits(x["v_new"]),
                                 table=table, L=lay.seq_lens.astype(np.int32))
    items = [(l, b) for l in layers for b in range(lay.B)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        n = sum(pool.map(_oracle_rope, items, chunksize=4))
    tw = time.perf_counter() - t0
    return {
        "value": round(n * ROPE_BYTES_PER_SEQ / tw / 1e9, 6),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"layers 0..{layers[-1]} of the same step, all {lay.B} sequences each ({n} sequence-layers): "
                  f"rope_append_ref (NumPy FP32) in {workers} worker processes, {tw:.2f} s wall",
        "seconds": round(tw, 3),
    }


def bench_rope(args, lay):
    """One step = one pa_rope_append per layer: every sequence's query and new key rotated at
    position L - 1, the key and value appended."""
    cpu = None
    if not args.no_cpu:
        workers, aff = cpu_workers()
        log(f"cpu baseline (rope): oracle on {workers} workers ...")
        cpu = cpu_baseline_rope(lay, lay.n_layers, workers)
        cpu["affinity_cores"] = aff
    import torch
    from paged_kv_cache_205_amd import ops, synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ops.load()
    dev = "cuda"
    k_pool, v_pool = synth.make_pools(lay, dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
    table = synth.rope_table(2048, device=dev)
    inputs = [synth.step_inputs(lay, l, dev) for l in range(lay.n_layers)]
    q_out = [torch.empty_like(x["q"]) for x in inputs]
    live = int((lay.seq_lens > 0).sum())
    bytes_launch = live * ROPE_BYTES_PER_SEQ
    torch.cuda.synchronize()

    def step():
        for l in range(lay.n_layers):
            x = inputs[l]
            ops.pa_rope_append(x["q"], x["k_new"], x["v_new"], table, k_pool, v_pool, bt[l], seq_lens, q_out=q_out[l])

    def timed(run):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            run()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    for _ in range(args.warmup):
        step()
    ms_stream = timed(step)
    # A launch takes a few microseconds, less than the host's cost of issuing
    # it, so the step is timed as a captured graph of its 16 launches (the
    # stream timing is reported beside it).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    ms_step = timed(graph.replay)
    launch_ms = ms_step / lay.n_layers
    value = bytes_launch * lay.n_layers / (ms_step * 1e-3) / 1e9
    res = {
        "metric": ROPE_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"RoPE + append of {lay.name}: B={lay.B} new tokens per layer, {lay.n_layers} layers, "
                        f"32 q / 8 kv heads, D=64, 16-token BF16 pages, FP32 table of 2048 positions",
            "batch": lay.B,
            "layers": lay.n_layers,
            "bytes_per_step": bytes_launch * lay.n_layers,
            "timing": "graph replay of the 16 launches",
            "parallelism": "single GPU",
        },
        "us_per_step": round(ms_step * 1e3, 2),
        "us_per_step_stream": round(ms_stream * 1e3, 2),
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": "rope_append_kernel (one launch per layer, one wave per sequence)",
            "bound": "hbm",
            "achieved": round(bytes_launch / (launch_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(bytes_launch / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
            "bytes_per_launch": bytes_launch,
            "mean_launch_us": round(launch_ms * 1e3, 3),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def _oracle_prefill(item):
    """prefill_ref for one (layer, prompt) of the prefill sample; returns its attention flops."""
    from threadpoolctl import threadpool_limits
    from oracle import prefill_ref
    l, b = item
    d = _CPU[("prefill", l)]
    c0, c1 = int(d["cu"][b]), int(d["cu"][b + 1])
    with threadpool_limits(1):
        prefill_ref(d["q"][c0:c1], d["k"][c0:c1], d["v"][c0:c1], np.array([0, c1 - c0], np.int32), d["scale"])
    n = c1 - c0
    return n * (n + 1) // 2 * 32 * 4 * 64


def prefill_flops(cu: np.ndarray) -> int:
    """Attention flops of one layer: 4 D per attended (query, key) pair, for each of the 32 query heads."""
    n = np.diff(cu.astype(np.int64))
    return int((n * (n + 1) // 2).sum()) * 32 * 4 * 64


def cpu_baseline_prefill(lay, n_prompts: int, workers: int):
    """Time the oracle's prefill attention on the first n_prompts prompts (layer by layer), one prompt per task."""
    import torch
    from paged_kv_cache_205_amd import synth
    torch.set_num_threads(1)
    items = [(l, b) for l in range(lay.n_layers) for b in range(lay.B)][:max(1, n_prompts)]
    for l in sorted({l for l, _ in items}):
        ks, vs, cu = synth.prefill_inputs(lay, l, "cpu")
        q = synth.prefill_queries(lay, l, "cpu")
        _CPU[("prefill", l)] = dict(q=synth.bits(q), k=synth.bits(ks), v=synth.bits(vs), cu=cu.numpy(),
                                    scale=lay.scale)
        del q, ks, vs
    rows = int(_CPU[("prefill", 0)]["cu"][1])
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        flops = sum(pool.map(_oracle_prefill, items, chunksize=1))
    tw = time.perf_counter() - t0
    return {
        "value": round(flops / tw / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"the first {len(items)} prompts ({rows} rows each; layers 0..{items[-1][0]}) of the same "
                  f"prefill: prefill_ref (FP64 NumPy, one BLAS thread each) in {workers} worker processes, "
                  f"{tw:.1f} s wall",
        "seconds": round(tw, 2),
    }


def bench_prefill(args, lay):
    """One step = one pa_prefill per layer over every prompt's rows."""
    cpu = None
    if not args.no_cpu:
        workers, aff = cpu_workers()
        log(f"cpu baseline (prefill): oracle on {workers} workers ...")
        cpu = cpu_baseline_prefill(lay, args.cpu_prompts, workers)
        cpu["affinity_cores"] = aff
        log(f"cpu baseline: {cpu['value']:.6f} TFLOP/s ({cpu['seconds']} s)")
    import torch
    from paged_kv_cache_205_amd import ops, synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ops.load()
    dev = "cuda"
    src = []
    for l in range(lay.n_layers):
        k, v, cu = synth.prefill_inputs(lay, l, dev)
        src.append((synth.prefill_queries(lay, l, dev), k, v, cu))
    T = int(src[0][0].shape[0])
    outs = [torch.empty((T, 32, 64), dtype=torch.float32, device=dev) for _ in range(lay.n_layers)]
    flops_launch = prefill_flops(src[0][3].cpu().numpy())
    bytes_launch = T * (32 * 64 * 2 + 2 * 8 * 64 * 2 + 32 * 64 * 4)  # q, k, v read once, out written once
    if args.calib_copy_mib:
        a = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        torch.empty_like(a).copy_(a)
        del a
    torch.cuda.synchronize()

    def step(weights):
        for l in range(lay.n_layers):
            q, k, v, cu = src[l]
            ops.pa_prefill(q, k, v, cu, lay.scale, out=outs[l], weights=weights)

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def timed(weights):
        for _ in range(args.warmup):
            step(weights)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            step(weights)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    ms_step = timed(args.prefill_weights)
    other = "fp16" if args.prefill_weights == "bf16x2" else "bf16x2"
    ms_other = timed(other)
    launch_ms = ms_step / lay.n_layers
    tflops = flops_launch / (launch_ms * 1e-3) / 1e12
    res = {
        "metric": PREFILL_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"causal prefill attention of {lay.name}: B={lay.B} prompts of L-1 tokens, "
                        f"{lay.n_layers} layers, 32 q / 8 kv heads, D=64, FP32 output",
            "batch": lay.B,
            "rows_per_layer": T,
            "layers": lay.n_layers,
            "flops_per_step": flops_launch * lay.n_layers,
            "weights": args.prefill_weights,
            "timing": "stream launches",
            "parallelism": "single GPU",
        },
        "us_per_step": round(ms_step * 1e3, 2),
        "other_weights": {
            "weights": other,
            "value": round(flops_launch * lay.n_layers / (ms_other * 1e-3) / 1e12, 2),
            "us_per_step": round(ms_other * 1e3, 2),
            "frac_mfma_peak": round(flops_launch * lay.n_layers / (ms_other * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "roofline": {
            "kernel": f"prefill_kernel<{args.prefill_weights} weights> (one launch per layer)",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": (measured_traffic(PREFILL_PROFILE[args.prefill_weights],
                                         ("pa_prefill.hip", "pa_prefill.h", "pa_kernels.h"))
                        if lay.name == "full" else None),
            "flops_per_launch": flops_launch,
            "min_hbm_bytes_per_launch": bytes_launch,
            "mean_launch_us": round(launch_ms * 1e3, 3),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def stream_read_reference(torch, dev, gib: int = 4, reps: int = 5):
    """GB/s of a plain non-temporal streaming read of a 4 GiB buffer (libpa_probe.so), or None."""
    import ctypes
    path = os.path.join(ROOT, "paged_kv_cache_205_amd", "libpa_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.pa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_probe_stream_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    if lib.pa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), st) != 0:
        return None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        lib.pa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), st)
    t1.record()
    torch.cuda.synchronize()
    gbs = reps * nbytes / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del buf
    return gbs


# ----------------------------------------------------------------------------
# CPU baseline: the FP64 oracle as it stands, on a bounded sample (runs before
# the GPU is touched so that worker processes fork from a GPU-free parent).

_CPU = {}


def _oracle_seq(item):
    """append_ref + decode_ref for one (layer, sequence) of the sample; returns its length."""
    from oracle import append_ref, decode_ref
    l, b = item
    d = _CPU[l]
    kp, vp, bt = d["pages"][b]
    L = d["L"][b:b + 1]
    k2, v2 = append_ref(kp, vp, d["k_new"][b:b + 1], d["v_new"][b:b + 1], bt, L)
    decode_ref(d["q"][b:b + 1], k2, v2, bt, L, d["scale"])
    return int(L[0])


def cpu_baseline(lay, n_layers: int, workers: int):
    """Time the FP64 oracle (append + decode) on the first n_layers layers of the workload."""
    import torch
    from paged_kv_cache_205_amd import synth
    torch.set_num_threads(1)
    layers = list(range(min(n_layers, lay.n_layers)))
    for l in layers:
        k, v, bt = synth.layer_pages(lay, l, "cpu")
        k, v = synth.bits(k), synth.bits(v)
        x = synth.step_inputs(lay, l, "cpu")
        pages = {}
        for b in range(lay.B):  # each sequence's own pages, block table renumbered 0..n-1
            n = synth.nblocks(lay.seq_lens[b])
            ids = bt[b, :n]
            pages[b] = (k[ids], v[ids], np.arange(max(n, 1), dtype=np.int32)[None])
        _CPU[l] = dict(pages=pages, L=lay.seq_lens, q=synth.bits(x["q"]), k_new=synth.bits(x["k_new"]),
                       v_new=synth.bits(x["v_new"]), scale=lay.scale)
        del k, v
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    items = [(l, b) for l in layers for b in range(lay.B)]
    # one core, on the first few items
    t0 = time.perf_counter()
    n1 = sum(_oracle_seq(it) for it in items[:max(1, min(8, len(items)))])
    t1 = time.perf_counter() - t0
    # all workers (forked before the GPU is touched)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        ntok = sum(pool.map(_oracle_seq, items, chunksize=1))
    tw = time.perf_counter() - t0
    return {
        "value": round(ntok * 2048 / tw / 1e9, 6),  # 2048 bytes of K and V per token per layer
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"layers 0..{layers[-1]} of the same workload, all {lay.B} sequences each "
                  f"({ntok} tokens, {ntok * 2048 / 1e9:.3f} GB of K+V): append_ref + decode_ref "
                  f"(FP64 NumPy) in {workers} worker processes, {tw:.1f} s wall",
        "single_core_GBps": round(n1 * 2048 / t1 / 1e9, 6),
        "seconds": round(tw, 2),
    }


# ----------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="full", help="workload: full, fragmented, skewed, large, small, tiny")
    ap.add_argument("--partition", type=int, default=0, help="partition_tokens (0 = library default)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-layers", type=int, default=8, help="layers of the workload the oracle runs on")
    ap.add_argument("--no-graph", action="store_true", help="skip the captured-graph timing")
    ap.add_argument("--op", choices=("decode", "fill", "prefill", "rope"), default="decode",
                    help="decode: the decode step (default); fill: the prefill page fill; "
                         "prefill: the causal prefill attention; rope: RoPE at the position + append")
    ap.add_argument("--cpu-prompts", type=int, default=192, help="prompts (layer by layer) the prefill oracle runs on")
    ap.add_argument("--prefill-weights", choices=("bf16x2", "fp16"), default="bf16x2",
                    help="prefill: weights as bf16 pairs (default) or fp16 weights with fp16 V")
    ap.add_argument("--configs", default=",".join(OTHER_CONFIGS),
                    help="decode: other workloads timed after the headline one (comma list, or 'none')")
    ap.add_argument("--pv-valu", action="store_true",
                    help="decode: time libpa_pv_valu.so, the build whose PV product runs in FP32 on the VALU "
                         "instead of MFMA (for the comparison; the default build uses MFMA)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    from paged_kv_cache_205_amd import synth
    lay = synth.get(args.config)
    if args.op == "fill":
        bench_fill(args, lay)
        return
    if args.op == "prefill":
        bench_prefill(args, lay)
        return
    if args.op == "rope":
        bench_rope(args, lay)
        return

    cpu = None
    if not args.no_cpu:
        workers, aff = cpu_workers()
        log(f"cpu baseline: oracle on {workers} workers ...")
        cpu = cpu_baseline(lay, args.cpu_layers, workers)
        cpu["affinity_cores"] = aff
        log(f"cpu baseline: {cpu['value']:.4f} GB/s ({cpu['seconds']} s)")

    import torch
    from paged_kv_cache_205_amd import ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.pv_valu:
        from paged_kv_cache_205_amd import build as _build
        ops.LIB_PATH = _build.LIB_PV_VALU
    ops.load()
    dev = "cuda"
    log(f"workload {lay.name}: B={lay.B} layers={lay.n_layers} pool {lay.pool_bytes / 2**30:.2f} GiB, "
        f"KV/step {lay.kv_bytes_per_step / 1e9:.3f} GB")
    k_pool, v_pool = synth.make_pools(lay, dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
    inputs = [synth.step_inputs(lay, l, dev) for l in range(lay.n_layers)]
    outs = [torch.empty((lay.B, 32, 64), dtype=torch.float32, device=dev) for _ in range(lay.n_layers)]
    part = args.partition
    ws = ops.workspace_for(lay.B, lay.max_blocks, part, dev)
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    def step(ev=None, separate=False):
        for l in range(lay.n_layers):
            x = inputs[l]
            if separate:
                ops.pa_append(x["k_new"], x["v_new"], k_pool, v_pool, bt[l], seq_lens)
            if ev is not None:
                ev[l][0].record()
            if separate:
                ops.pa_decode(x["q"], k_pool, v_pool, bt[l], seq_lens, lay.scale, out=outs[l],
                              partition_tokens=part, workspace=ws)
            else:
                ops.pa_append_decode(x["k_new"], x["v_new"], k_pool, v_pool, x["q"], bt[l], seq_lens, lay.scale,
                                     out=outs[l], partition_tokens=part, workspace=ws)
            if ev is not None:
                ev[l][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # the same step from a plan built once per step (pa_decode_plan, then one
    # pa_decode_planned append + decode per layer)
    plan = torch.empty(ops.pa_decode_plan_bytes(lay.B, lay.max_blocks, part), dtype=torch.uint8, device=dev)

    def step_planned():
        ops.pa_decode_plan(seq_lens, lay.max_blocks, part, plan=plan)
        for l in range(lay.n_layers):
            x = inputs[l]
            ops.pa_decode_planned(x["q"], k_pool, v_pool, bt[l], plan, lay.scale, k_new=x["k_new"], v_new=x["v_new"],
                                  out=outs[l], partition_tokens=part, workspace=ws)

    for _ in range(args.warmup):
        step_planned()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step_planned()
    t1.record()
    torch.cuda.synchronize()
    ms_step_planned = t0.elapsed_time(t1) / args.steps

    # the same step as two calls per layer (pa_append, then pa_decode)
    for _ in range(args.warmup):
        step(separate=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step(separate=True)
    t1.record()
    torch.cuda.synchronize()
    ms_step_sep = t0.elapsed_time(t1) / args.steps

    # the same step with RoPE of q and the new key at position L-1 fused into
    # the launch (pa_rope_append_decode); the next steps append the plain rows again
    table = synth.rope_table(lay.max_blocks * 16, device=dev)

    def step_rope():
        for l in range(lay.n_layers):
            x = inputs[l]
            ops.pa_rope_append_decode(x["k_new"], x["v_new"], k_pool, v_pool, x["q"], table, bt[l], seq_lens,
                                      lay.scale, out=outs[l], partition_tokens=part, workspace=ws)

    for _ in range(args.warmup):
        step_rope()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step_rope()
    t1.record()
    torch.cuda.synchronize()
    ms_step_rope = t0.elapsed_time(t1) / args.steps

    # decode launches timed one by one (separate pass, same work)
    dec_ms = []
    for _ in range(args.steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(lay.n_layers)]
        step(ev)
        torch.cuda.synchronize()
        dec_ms += [a.elapsed_time(b) for a, b in ev]
    dec_ms_mean = float(np.mean(dec_ms))

    # the step's spread: each of K steps bracketed by its own events
    step_ms = []
    for _ in range(args.steps):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        step()
        a1.record()
        torch.cuda.synchronize()
        step_ms.append(a0.elapsed_time(a1))

    graph_ms = None
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step()
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    step()
            torch.cuda.synchronize()
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            t0.record()
            for _ in range(args.steps):
                g.replay()
            t1.record()
            torch.cuda.synchronize()
            graph_ms = t0.elapsed_time(t1) / args.steps
        except Exception as e:  # report, keep the stream number
            log(f"graph capture failed: {e!r}")

    stream_gbs = stream_read_reference(torch, dev)

    # the other workloads, each on its own pool, after the headline's timings
    configs = {}
    names = [c for c in args.configs.split(",") if c and c != "none" and c != lay.name]
    if names:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        for name in names:
            configs[name] = time_workload(name, args.steps, args.warmup, stream_gbs, flush)
        del flush

    kv_step = lay.kv_bytes_per_step
    best_ms = min(x for x in (ms_step, graph_ms, ms_step_planned) if x is not None)
    value = kv_step / (best_ms * 1e-3) / 1e9
    # launch duration: the back-to-back stream timing divided by the launches
    # (dispatch gaps included; rocprofv3's per-kernel average is the check)
    launch_ms = ms_step / lay.n_layers
    achieved = lay.kv_bytes_per_layer / (launch_ms * 1e-3) / 1e9
    # Counter traffic from the committed profile, attached only when it was
    # taken on this kernel source and its traced kernel average fits inside this
    # run's own step time (16 launches of it cannot take longer than the step).
    prof = decode_profile() if (lay.name == "full" and args.partition == 0 and not args.pv_valu) else None
    prof_avg = prof["kernel_avg_us"] if prof else None
    prof_fits = prof_avg is not None and lay.n_layers * prof_avg <= best_ms * 1e3
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(best_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{lay.name}: B={lay.B}, L={'2048' if lay.name == 'full' else 'mixed'}, "
                        f"{lay.n_layers} layers, 32 q / 8 kv heads, D=64, 16-token BF16 pages",
            "batch": lay.B,
            "seq_len_max": int(lay.seq_lens.max()),
            "layers": lay.n_layers,
            "kv_bytes_per_step": kv_step,
            "partition_tokens": part if part else "auto",
            "timing": ("graph replay" if best_ms == graph_ms else
                       "stream launches, plan built once per step" if best_ms == ms_step_planned else
                       "stream launches"),
            "kv_dtype": "bf16",
            "parallelism": "single GPU",
        },
        "us_per_step": round(best_ms * 1e3, 2),
        "us_per_step_stream": round(ms_step * 1e3, 2),
        "us_per_step_graph": None if graph_ms is None else round(graph_ms * 1e3, 2),
        "us_per_step_planned": round(ms_step_planned * 1e3, 2),
        "us_per_step_each": {"median": round(float(np.median(step_ms)) * 1e3, 2),
                             "min": round(float(np.min(step_ms)) * 1e3, 2),
                             "p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2)},
        "us_per_step_separate_append_decode": round(ms_step_sep * 1e3, 2),
        "us_per_step_rope_append_decode": round(ms_step_rope * 1e3, 2),
        "seq_steps_per_s": round(lay.B / (best_ms * 1e-3), 1),
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "stream_read_GBps": None if stream_gbs is None else round(stream_gbs, 1),
        "frac_stream_read": None if stream_gbs is None else round(value / stream_gbs, 4),
        "roofline": {
            "kernel": ("decode_kernel<fused append> (one launch per layer: append, attention, split merge)"
                       + (", PV on the VALU (comparison build)" if args.pv_valu else "")),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": prof["traffic"] if (prof and prof_fits) else None,
            "bytes_per_launch": lay.kv_bytes_per_layer,
            "mean_launch_us": round(launch_ms * 1e3, 3),
            "event_bracketed_launch_us": round(dec_ms_mean * 1e3, 3),
            "profile_kernel_avg_us": prof_avg,
            "profile_frac": (None if not prof_avg else
                             round(lay.kv_bytes_per_layer / (prof_avg * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)),
        },
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
