#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: build the new tokens'
cache slots, store their K/V and attend.  Decode workloads run it as one
launch (pa_decode_step: slot, store and attention fused); ``--unfused`` runs
pa_build_slot_mapping + pa_write_kv + pa_decode instead.  Packed workloads run
pa_build_slot_mapping + pa_write_kv + pa_varlen_prefill.  The
default workload is the LLaMA-2-7B-shaped decode batch (64 sequences, contexts
U[128,384], 32 q = 32 kv heads, head_dim 128, bf16, 16-token blocks from a
4096-block pool).

Consecutive timed steps read different layers' caches (same block tables,
different values, as in a model whose layers share the block manager), so no
step reads K/V that the previous one left in the 256 MB Infinity Cache.

Prints one JSON line.  `value` is the step's algorithmic HBM bytes over its
time (GB/s); `roofline` covers the attention kernel, timed with HIP events on
the stream it is launched on; `cpu_baseline` is the float64 CPU oracle timed on
a bounded sample of the same workload on this host, over a pool of worker
processes.  The default run adds `configs`: one sub-record (value, unit,
roofline, cpu_baseline, step time, graph replay) for each other configuration
-- the tiny fp32 decode, GQA decode, the mixed step (whole call) and its
prefill chunks alone (TFLOP/s against the matrix-core peak), and the
shared-prefix decode through pa_decode_step and through pa_cascade_decode.
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
sys.path.insert(0, ROOT)

METRIC = "paged decode KV-read GB/s (% of HBM peak); prefill TFLOP/s; seq-steps/s"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6  # MI355X dense bf16 matrix peak
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "decode": ["paged_kv_cache_token_amd/csrc/pa_decode.hip",
               "paged_kv_cache_token_amd/csrc/pa_internal.h"],
    "prefill": ["paged_kv_cache_token_amd/csrc/pa_prefill.hip",
                "paged_kv_cache_token_amd/csrc/pa_internal.h"],
    # every kernel file: calls running decode and matrix-core kernels together
    "cascade": ["paged_kv_cache_token_amd/csrc/pa_decode.hip",
                "paged_kv_cache_token_amd/csrc/pa_prefill.hip",
                "paged_kv_cache_token_amd/csrc/pa_internal.h"],
}


def _code_only(text: str) -> str:
    """A kernel source with its comments and layout removed: the counters
    stored under profiles/ stay valid across edits that change no code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(kind: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        h.update(_code_only(open(os.path.join(ROOT, p), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def make_batch(name: str):
    import workloads as W
    return {
        "llama2_decode": W.llama2_decode,
        "gqa_decode": W.gqa_decode,
        "shared_prefix_decode": W.shared_prefix_decode,
        "shared_prefix_cascade": W.shared_prefix_decode,
        "long_prefix_decode": W.long_prefix_decode,
        "long_prefix_cascade": W.long_prefix_decode,
        "mixed_step": W.mixed_step,
        "prefill_chunks": W.prefill_only,
        "prefill_long": W.prefill_long,
        "tiny_decode": W.tiny_decode,
    }[name]()


# --------------------------------------------------------------------------
# algorithmic work (what the step must move / compute at minimum)
# --------------------------------------------------------------------------

def attention_bytes(b) -> int:
    """K/V of every attended token (a physical block shared by several
    sequences counted once), q, out, live block-table entries, lengths."""
    e = b.elem_bytes
    tile = b.num_kv_heads * b.block_size * b.head_dim * e
    ctx = b.context_lens.astype(np.int64)
    if b.notes.get("prefix_tokens") and not b.notes.get("unshared"):
        # unique tokens: the shared prompt once plus every private suffix
        p = b.notes["prefix_tokens"]
        kv_tokens = p + int((ctx - p).sum())
    else:
        kv_tokens = int(ctx.sum())
    kv = 2 * kv_tokens * b.num_kv_heads * b.head_dim * e
    qo = 2 * b.total_q * b.num_q_heads * b.head_dim * e
    live_entries = int(sum(-(-int(c) // b.block_size) for c in ctx))
    meta = 4 * live_entries + 4 * (2 * b.num_seqs + 1)
    del tile
    return kv + qo + meta


def write_bytes(b) -> int:
    """pa_build_slot_mapping + pa_write_kv of the step's new tokens."""
    row = b.num_kv_heads * b.head_dim * b.elem_bytes
    slot_map = 4 * (2 * b.num_seqs + 1) + 4 * b.total_q + 8 * b.total_q
    write = 2 * 2 * b.total_q * row + 8 * b.total_q
    return slot_map + write


def fused_write_bytes(b) -> int:
    """pa_decode_step's store of the new tokens: their K/V read and written,
    one table entry each."""
    row = b.num_kv_heads * b.head_dim * b.elem_bytes
    return 2 * 2 * b.total_q * row + 4 * b.total_q


def prefill_flops(b) -> int:
    """Causal (q, k) pairs of the multi-token chunks x 4 * Hq * d (QK^T and PV)."""
    pairs = 0
    for c, l in zip(b.context_offsets.astype(np.int64), b.q_lens.astype(np.int64)):
        if l > 1:
            pairs += int(l * c + l * (l + 1) // 2)
    return 4 * b.num_q_heads * b.head_dim * pairs


# --------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample, over all host cores
# --------------------------------------------------------------------------

_CPU = {}  # the batch and host state the forked workers read (copy-on-write)


def _cpu_init():
    # one BLAS thread per worker: the pool supplies the parallelism
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass


def _cpu_seq(i):
    from oracle_side import expected
    expected(_CPU["b"], _CPU["hs"], seqs=[i])
    return i


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers() -> int:
    """Worker processes: the host cores this process may run on, at most 16
    (the CPU share of one GPU on a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(b, budget_s: float = 10.0, unit: str = "GB/s") -> dict:
    """The float64 oracle (tests/oracle_side.py) on host copies of the same
    inputs, one sequence per task over a process pool (one BLAS thread per
    worker), for about budget_s seconds of wall time; `unit` GB/s (the same
    algorithmic bytes as the GPU figure) or TFLOP/s (causal prefill pairs)."""
    import multiprocessing as mp
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_side import host_state

    t_setup = time.perf_counter()
    hs = host_state(b, device="cuda")
    setup_s = time.perf_counter() - t_setup
    _CPU["b"], _CPU["hs"] = b, hs
    n = b.num_seqs
    work_bytes = _per_seq_attention_bytes(b)
    work_flops = _per_seq_prefill_flops(b)
    workers = cpu_workers()
    # sequences in a fixed shuffled order (long and short mixed), repeated
    order = list(np.random.default_rng(0).permutation(n))
    done, done_bytes, done_flops, passes = 0, 0, 0, 0
    ctx = mp.get_context("fork")  # workers only run numpy on inherited host arrays
    with ctx.Pool(workers, initializer=_cpu_init) as pool:
        t0 = time.perf_counter()
        # tasks taken as workers free up; counted as they finish, up to the
        # budget (the pool is terminated with the tasks still in flight)
        tasks = (order[k % n] for k in range(n * 1000))
        for i in pool.imap_unordered(_cpu_seq, tasks, chunksize=1):
            done += 1
            done_bytes += work_bytes[i]
            done_flops += work_flops[i]
            if time.perf_counter() - t0 >= budget_s and done >= min(n, 8):
                break
        wall = time.perf_counter() - t0
        passes = done // n
    _CPU.clear()
    del hs
    value = done_bytes / wall / 1e9 if unit == "GB/s" else done_flops / wall / 1e12
    return {
        "value": round(value, 4 if unit == "GB/s" else 6),
        "unit": unit,
        "cores": workers,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"float64 numpy oracle ({'decode' if b.kind == 'decode' else 'varlen_prefill'})"
                   f" over {done} sequences of the workload ({passes} full passes), "
                   f"{workers} worker processes x 1 BLAS thread, {wall:.1f} s wall "
                   f"(+{setup_s:.1f} s building the host copy of the inputs)"),
        "seq_steps_per_s": round(done / wall, 3),
    }


def _per_seq_prefill_flops(b) -> list[int]:
    out = []
    for c, l in zip(b.context_offsets.astype(np.int64), b.q_lens.astype(np.int64)):
        out.append(int(4 * b.num_q_heads * b.head_dim * (l * c + l * (l + 1) // 2)) if l > 1 else 0)
    return out


def _per_seq_attention_bytes(b) -> list[int]:
    e = b.elem_bytes
    out = []
    for i, c in enumerate(b.context_lens.astype(np.int64)):
        ql = int(b.q_lens[i])
        out.append(int(2 * c * b.num_kv_heads * b.head_dim * e + 2 * ql * b.num_q_heads * b.head_dim * e))
    return out


# --------------------------------------------------------------------------
# traffic from committed rocprofv3 counter summaries
# --------------------------------------------------------------------------

def traffic_from_profiles(workload: str, kind: str):
    path = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_hash(kind):
        return None  # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


# --------------------------------------------------------------------------
# main
# --------------------------------------------------------------------------

def context_figures(dbs, run_step, stream, steps, dev) -> dict:
    """Figures reported beside the measurement, none of them `value`: the
    warm median (every step on the same layer's caches, so K/V may sit in
    the 256 MB MALL) and a plain device copy's and read's bandwidth."""
    import torch
    out = {}
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for s in range(steps):
        run_step(dbs[0], ev[s])
    torch.cuda.synchronize()
    out["warm_call_us_p50"] = round(float(np.median([a.elapsed_time(z) for a, z in ev])) * 1e3, 2)

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    z.record(stream)
    torch.cuda.synchronize()
    out["copy_gbs_read_plus_write"] = round(2 * n * reps / (a.elapsed_time(z) * 1e-3) / 1e9, 1)
    # a read-only stream (a sum over 1 GiB of fp32): the nearest plain
    # figure to a decode kernel's traffic, which is almost all reads
    x = src.view(torch.float32)
    x.sum()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        x.sum()
    z.record(stream)
    torch.cuda.synchronize()
    out["read_gbs_sum_1gib"] = round(n * reps / (a.elapsed_time(z) * 1e-3) / 1e9, 1)
    del src, dst, x
    return out


def graph_figures(dbs, run_step, stream, steps) -> dict:
    """The step replayed from HIP graphs (the library makes no allocation,
    synchronisation or memset, so a captured call is the same launches):
    every layer's step captured into one graph, as a model's forward pass
    would be, and, for comparison, one graph per layer's step."""
    import torch
    out = {}
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for d in dbs:
                run_step(d)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        whole = torch.cuda.CUDAGraph()
        with torch.cuda.graph(whole):
            for d in dbs:
                run_step(d)
        per_layer = []
        for d in dbs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(d)
            per_layer.append(g)
        whole.replay()
        for g in per_layer:
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, -(-steps // len(dbs)))
        a.record(stream)
        for _ in range(reps):
            whole.replay()
        z.record(stream)
        torch.cuda.synchronize()
        out["graph_ms_per_step"] = round(a.elapsed_time(z) / (reps * len(dbs)), 5)
        a.record(stream)
        for s in range(steps):
            per_layer[s % len(per_layer)].replay()
        z.record(stream)
        torch.cuda.synchronize()
        out["graph_ms_per_step_one_graph_per_step"] = round(a.elapsed_time(z) / steps, 5)
        out["graph_layers_per_replay"] = len(dbs)
        del whole, per_layer
    except Exception as e:  # reported, never fatal: the eager figures stand alone
        out["graph_ms_per_step"] = None
        out["graph_error"] = str(e)[:200]
    return out


def bench_block_swap(args, dev) -> int:
    """pa_swap_blocks on LLaMA-2-7B-shaped pools (4096 blocks of 32 kv heads x
    16 x 128 bf16, 128 KiB per block per K or V pool): 1024 random blocks of K
    and of V copied inside device memory (timed: HBM read + write), swapped
    out to pinned host pools and back in (host-link rates, reported beside)."""
    import torch

    import paged_kv_cache_token_amd as pa
    nb, hkv, d, moved = 4096, 32, 128, 1024
    rng = np.random.default_rng(6)
    pools = [torch.randn(nb, hkv, 16, d, device=dev).to(torch.bfloat16) for _ in range(2)]
    ids = rng.permutation(nb)
    copy_pairs = torch.from_numpy(np.stack([ids[:moved], ids[moved:2 * moved]], 1).astype(np.int64)).to(dev)
    out_pairs = torch.from_numpy(np.stack([ids[:moved], np.arange(moved)], 1).astype(np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(moved), ids[2 * moved:3 * moved]], 1).astype(np.int64)).to(dev)
    host = [torch.empty(moved, hkv, 16, d, dtype=torch.bfloat16).pin_memory() for _ in range(2)]
    block_bytes = hkv * 16 * d * 2
    stream = torch.cuda.current_stream(dev)

    def timed(fn, steps):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        z.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(z) / steps

    def copy_step():
        for p in pools:
            pa.swap_blocks(p, p, copy_pairs)

    ms = timed(copy_step, args.steps)
    step_bytes = 2 * 2 * moved * block_bytes  # K and V, read + write
    value = step_bytes / (ms * 1e-3) / 1e9
    ms_out = timed(lambda: [pa.swap_blocks(h, p, out_pairs) for h, p in zip(host, pools)], 20)
    ms_in = timed(lambda: [pa.swap_blocks(p, h, in_pairs) for h, p in zip(host, pools)], 20)
    link_bytes = 2 * moved * block_bytes
    cpu = None
    if not args.no_cpu_baseline:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import oracle
        src = pools[0].cpu().view(torch.int16).numpy()
        dst = src.copy()
        pairs = copy_pairs.cpu().numpy()
        t0, c0, reps = time.perf_counter(), time.process_time(), 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 5.0):
            oracle.swap_blocks(dst, src, pairs)
            reps += 1
        wall = time.perf_counter() - t0
        cpu = {"value": round(reps * moved * block_bytes * 2 / wall / 1e9, 3), "unit": "GB/s",
               "cores": max(1, int(round((time.process_time() - c0) / wall))), "kind": "oracle",
               "sample": f"oracle block copy of one pool's {moved} pairs, {reps} passes in {wall:.1f} s"}
    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "block_swap_llama2_pools", "pool_blocks": nb, "kv_heads": hkv,
                   "head_dim": d, "block_size": 16, "blocks_moved_per_pool": moved,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "swap_out_gbs_device_to_pinned_host": round(link_bytes / (ms_out * 1e-3) / 1e9, 2),
        "swap_in_gbs_pinned_host_to_device": round(link_bytes / (ms_in * 1e-3) / 1e9, 2),
        "step_calls": "pa_swap_blocks x2 (K and V pools)",
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_block_manager(args) -> int:
    """The host block manager (pa_bm_*) on the LLaMA-2-7B-shaped decode
    configuration: 64 running sequences (contexts U[128, 384], blocks from a
    4096-block pool).  One step = allocate_batch (one new token for every
    sequence), then build_step, which writes the decode step's block tables,
    lengths and slot mapping.  Timed on the host through the binding (its per-call cost
    included); build_step alone is reported beside.  No GPU work."""
    import paged_kv_cache_token_amd as pa
    rng = np.random.default_rng(2)
    n, nb, maxb = 64, 4096, 64
    ctx = rng.integers(128, 384 + 1, size=n)
    bm = pa.BlockManager(nb)
    for i, c in enumerate(ctx):
        if not bm.allocate_slots(i, int(c)):
            raise RuntimeError("pool too small for the initial contexts")
    ids = np.arange(n, dtype=np.int64)
    ql = np.ones(n, dtype=np.int32)

    def step():
        if bm.allocate_batch(ids, ql) != n:
            raise RuntimeError("pool exhausted")
        return bm.build_step(ids, ql, maxb)

    for _ in range(args.warmup):
        step()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        meta = step()
    wall = time.perf_counter() - t0
    s_per_step = wall / args.steps
    t1 = time.perf_counter()
    reps = 200
    for _ in range(reps):
        bm.build_step(ids, ql, maxb)
    build_us = (time.perf_counter() - t1) / reps * 1e6
    # the same allocation with one binding call per sequence, for comparison
    t3 = time.perf_counter()
    for _ in range(20):
        for i in range(n):
            bm.allocate_slots(i, 1)
    one_by_one_us = (time.perf_counter() - t3) / 20 * 1e6
    cpu = None
    if not args.no_cpu_baseline:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import oracle
        bt, cu, co = meta["block_tables"], meta["cu_seqlens"], meta["context_offsets"]
        t2, c2, k = time.perf_counter(), time.process_time(), 0
        while time.perf_counter() - t2 < 2.0:
            oracle.slot_mapping(bt, cu, co)
            k += 1
        w2 = time.perf_counter() - t2
        cpu = {"value": round(k * n / w2, 1), "unit": "seq-steps/s",
               "cores": max(1, int(round((time.process_time() - c2) / w2))), "kind": "oracle",
               "sample": f"oracle slot mapping of the same step's tables, {k} passes in {w2:.1f} s"}
    rec = {
        "metric": METRIC, "value": round(n / s_per_step, 1), "unit": "seq-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(s_per_step * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": "block_manager_llama2_decode", "num_seqs": n, "pool_blocks": nb,
                   "block_size": 16, "context_min_max": [int(ctx.min()), int(ctx.max())],
                   "parallelism": "host"},
        "roofline": None,
        "roofline_note": "host code, no GPU kernel: the figure is host time per step",
        "cpu_baseline": cpu,
        "build_step_us": round(build_us, 2),
        "allocate_slots_one_call_per_sequence_us": round(one_by_one_us, 2),
        "step_calls": "pa_bm_allocate_batch + pa_bm_build_step",
    }
    print(json.dumps(rec), flush=True)
    return 0


# configurations carried as sub-records of the default run's line: every
# configuration the metric is quoted on, beside the LLaMA-2 decode headline
SUB_WORKLOADS = ["tiny_decode", "gqa_decode", "mixed_step", "prefill_chunks",
                 "shared_prefix_decode", "shared_prefix_cascade"]


def measure(name: str, args, dev, headline: bool) -> dict:
    """Time `args.steps` steps of one workload; the record of its line (the
    headline) or of its sub-record."""
    import torch

    from device_batch import DeviceBatch

    b = make_batch(name)
    kind = "decode" if b.kind == "decode" else "prefill"
    # the shared-prefix batch through pa_cascade_decode (new tokens stored first)
    cascade = name.endswith("_cascade")
    fused = kind == "decode" and not args.unfused and not cascade
    att_bytes = attention_bytes(b)
    # the fused step reads the new K/V rows and stores them: no slot array traffic
    wr_bytes = fused_write_bytes(b) if fused else write_bytes(b)
    per_layer_ws = att_bytes + wr_bytes
    layers = args.layers or max(1, min(8, math.ceil((1 << 30) / per_layer_ws)))
    dbs = [DeviceBatch(b.with_layer(l), device=dev) for l in range(layers)]
    torch.cuda.synchronize()

    if args.calib_copy_mib and headline:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream(dev)

    def run_step(d, ev_pair=None):
        if fused:
            if ev_pair:
                ev_pair[0].record(stream)
            d.fused_step()
            if ev_pair:
                ev_pair[1].record(stream)
            return
        d.write_new()
        if ev_pair:
            ev_pair[0].record(stream)
        if cascade:
            d.cascade()
        else:
            d.attend()
        if ev_pair:
            ev_pair[1].record(stream)

    for s in range(args.warmup):
        run_step(dbs[s % layers])
    torch.cuda.synchronize()

    # timed region 1: exactly K steps, synchronized on both sides, events only at
    # its ends -> ms_per_step and value
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        run_step(dbs[s % layers])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # timed region 2: the same K steps with a HIP event pair around every
    # attention launch, on its launch stream -> the kernel's average duration
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        run_step(dbs[s % layers], ev[s])
    torch.cuda.synchronize()
    att_ms = [a.elapsed_time(z) for a, z in ev]
    att_avg_ms = float(np.mean(att_ms))

    extras = {}
    if not args.no_extras:
        if headline:
            extras.update(context_figures(dbs, run_step, stream, args.steps, dev))
        extras.update(graph_figures(dbs, run_step, stream, args.steps))

    step_bytes = att_bytes + wr_bytes
    fl = prefill_flops(b)
    prefill_only = kind == "prefill" and int((b.q_lens == 1).sum()) == 0
    if prefill_only:
        unit = "TFLOP/s"
        value = fl / (ms_per_step * 1e-3) / 1e12
    else:
        unit = "GB/s"
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # the dominant kernel's average duration: with the fused decode step a step
    # is exactly one launch of it (single-partition contexts), so timed region 1
    # gives it without the per-launch event overhead; otherwise the event pairs
    # of region 2 (the whole attention call)
    kern_ms = ms_per_step if fused else att_avg_ms
    if not prefill_only:
        kern_bytes = att_bytes + (wr_bytes if fused else 0)
        achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
        traffic = traffic_from_profiles(name, "cascade" if (cascade or kind == "prefill") else "decode")
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic}
    else:
        achieved = fl / (att_avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
                    "traffic": traffic_from_profiles(name, "prefill")}

    del dbs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b, args.cpu_budget if headline else args.sub_cpu_budget, unit)

    ctx = b.context_lens
    rec = {
        "value": round(value, 1 if unit == "GB/s" else 2),
        "unit": unit,
        "ms_per_step": round(ms_per_step, 5),
        "dtype": "bf16" if b.dtype == "bf16" else "f32",
        "config": {
            "workload": b.name,
            "num_seqs": b.num_seqs,
            "q_heads": b.num_q_heads,
            "kv_heads": b.num_kv_heads,
            "head_dim": b.head_dim,
            "block_size": b.block_size,
            "pool_blocks": b.num_blocks,
            "total_q_tokens": b.total_q,
            "context_min_mean_max": [int(ctx.min()), round(float(ctx.mean()), 1), int(ctx.max())],
            "layer_caches_rotated": layers,
            "parallelism": "single-gpu",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "seq_steps_per_s": round(b.num_seqs / (ms_per_step * 1e-3), 1),
        "attention_call_us": round(att_avg_ms * 1e3, 2),
        "dominant_kernel_us": round(kern_ms * 1e3, 2),
        "step_calls": "pa_decode_step (fused)" if fused else (
            "pa_build_slot_mapping + pa_write_kv + " +
            ("pa_cascade_decode" if cascade else
             "pa_decode" if kind == "decode" else "pa_varlen_prefill_ex")),
        "attention_bytes": att_bytes,
        "write_bytes": wr_bytes,
        "step_bytes": step_bytes,
        "wall_s_timed": round(wall, 4),
        "kernel_source_hash": kernel_hash("prefill" if prefill_only else
                                          "cascade" if (cascade or kind == "prefill") else "decode"),
        "call_us_p10_p50_p90": [round(float(np.percentile(att_ms, q)) * 1e3, 2)
                                for q in (10, 50, 90)],
    }
    if b.notes.get("prefix_tokens") and not b.notes.get("unshared"):
        rec["logical_kv_bytes"] = 2 * int(ctx.astype(np.int64).sum()) * b.num_kv_heads * \
            b.head_dim * b.elem_bytes
    if kind == "prefill":
        rec["prefill_flops"] = fl
        rec["prefill_tflops_whole_call"] = round(fl / (att_avg_ms * 1e-3) / 1e12, 2)
    rec.update(extras)
    return rec


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama2_decode",
                    choices=["llama2_decode", "gqa_decode", "shared_prefix_decode",
                             "shared_prefix_cascade", "long_prefix_decode",
                             "long_prefix_cascade", "mixed_step", "prefill_chunks", "prefill_long",
                             "tiny_decode", "block_swap", "block_manager"])
    ap.add_argument("--layers", type=int, default=0,
                    help="layer caches to rotate through (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the headline's CPU baseline")
    ap.add_argument("--sub-cpu-budget", type=float, default=6.0,
                    help="seconds of oracle time for each sub-record's CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="the default workload alone, without the other configurations")
    ap.add_argument("--unfused", action="store_true",
                    help="decode: three calls (slot mapping, write, decode) instead of one")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the context figures (warm median, copy bandwidth, graph replay)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        return 2

    import torch

    import paged_kv_cache_token_amd as pa  # fails loudly if libpa.so is missing
    del pa

    if args.workload == "block_manager":
        return bench_block_manager(args)  # host code only
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload == "block_swap":
        return bench_block_swap(args, dev)
    head = measure(args.workload, args, dev, headline=True)
    rec = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": head.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic",
    }
    rec.update(head)
    if args.workload == "llama2_decode" and not args.headline_only:
        subs = {}
        for w in SUB_WORKLOADS:
            print(f"[bench] {w}", file=sys.stderr, flush=True)
            subs[w] = measure(w, args, dev, headline=False)
        rec["configs"] = subs
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
