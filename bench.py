"""Benchmark of one paged decode step (append + attention) on one MI355X.

A step is one pass of the whole path over one batch: every sequence's new token is
written into its slot and attention runs over the paged context. By default the step is one
pkv_paged_decode_step call: two kernels, the split-KV decode kernel (which takes the new
token's K/V straight from the input rows and stores them into the pool) and the merge
kernel when a sequence spans several partitions; --separate-append times pkv_kv_append followed by
pkv_paged_decode_attention instead, and the default line also reports that two-launch
step's time. Inputs are seeded synthetic workloads resident in HBM before timing; the same
step is repeated (the new token is rewritten into the same slot, so every step does
identical work).

Prints ONE JSON line: the metric is KV GB/s read (whole step), with the decode launch's
achieved bandwidth against the 8 TB/s HBM peak in "roofline", and the fp64 CPU oracle timed
on a bounded sample of the same workload in "cpu_baseline".

The default line times the GQA bf16 layer (workload 3) and, in the same run, the
long-context GQA layer (workload 4), summarised under "also_measured".

    python bench.py [--steps K] [--warmup W] [--config 3] [--also 4] [--partition 0]
                    [--all] [--separate-append]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published peak

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs, each scaled by
# what the counter reads for a 1 GiB device copy. Decode step lines are keyed by (workload
# id, partition_tokens, fused step) and cover the decode + merge kernels; the component
# lines by ("multi-query", q_len) (decode + merge of the attention call), ("shared-prefix",)
# (split kernel with the prefix tasks + merge) and ("quantized", format) (decode + merge). Each entry
# records the sha256 prefix of the decode kernel sources it was measured on (pkv_decode.hip,
# then pkv_internal.h with the launch constants); it is reported only while those sources
# are unchanged.
MEASURED_TRAFFIC = {
    (3, 0, True): {"bytes": 1587575569, "decode_source_sha256": "7d0c5f462cc26f68"},
    (3, 0, False): {"bytes": 1586996592, "decode_source_sha256": "7d0c5f462cc26f68"},
    (4, 0, True): {"bytes": 1352698833, "decode_source_sha256": "7d0c5f462cc26f68"},
    (4, 0, False): {"bytes": 1352623975, "decode_source_sha256": "7d0c5f462cc26f68"},
    (2, 0, True): {"bytes": 1194508606, "decode_source_sha256": "7d0c5f462cc26f68"},
    (2, 0, False): {"bytes": 1193405791, "decode_source_sha256": "7d0c5f462cc26f68"},
    ("multi-query", 4): {"bytes": 1628098490, "decode_source_sha256": "7d0c5f462cc26f68"},
    ("shared-prefix",): {"bytes": 390049623, "decode_source_sha256": "7d0c5f462cc26f68"},
    ("quantized", "int8"): {"bytes": 849889453, "decode_source_sha256": "7d0c5f462cc26f68"},
    ("quantized", "fp8"): {"bytes": 849799654, "decode_source_sha256": "7d0c5f462cc26f68"},
}
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_26_amd", "csrc", name)
                  for name in ("pkv_decode.hip", "pkv_internal.h")]


def decode_source_sha() -> str:
    """sha256 prefix of the decode kernel sources, read in DECODE_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(*key):
    entry = MEASURED_TRAFFIC.get(tuple(key))
    if entry is None:
        return None
    return entry["bytes"] if decode_source_sha() == entry["decode_source_sha256"] else None


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; 50 for the block manager)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 1000, a fraction of a second: step "
                         "times fall by ~1.5%% over the first tens of milliseconds of load as "
                         "the GPU's clocks settle; 10 for the block manager)")
    ap.add_argument("--config", type=int, default=3,
                    help="workload id 1..5 (default 3, the GQA bf16 layer: 64 sequences of "
                         "4096-8192 tokens, the largest workload that the step reads)")
    ap.add_argument("--also", type=str, default=None, metavar="IDS",
                    help="comma-separated workload ids timed in the same run after --config and "
                         "summarised under also_measured in its line (default: 4, the "
                         "long-context GQA layer, when --config is 3; '' for none)")
    ap.add_argument("--partition", type=int, default=0,
                    help="tokens per KV partition; 0 = the library's balanced split")
    ap.add_argument("--all", action="store_true", help="one line per workload 1..5")
    ap.add_argument("--separate-append", action="store_true",
                    help="time pkv_kv_append + pkv_paged_decode_attention (two launches) "
                         "instead of the fused pkv_paged_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, copy a buffer of this many MiB 3 times (a dispatch of "
                         "known traffic for scaling hardware byte counters)")
    ap.add_argument("--kv-format", choices=["int8", "fp8"], default="int8",
                    help="quantized cache format (--component quantized)")
    ap.add_argument("--component",
                    choices=["decode", "block-manager", "multi-query", "shared-prefix",
                             "quantized"],
                    default="decode",
                    help="decode: the decode step (default); block-manager: the native block "
                         "manager and the copy-on-write block copy; multi-query: q_len new "
                         "tokens per sequence (speculative verification) on the GQA workload; "
                         "shared-prefix: the shared-prefix workload with each group's common "
                         "blocks read once; quantized: the GQA workload with an 8-bit KV cache")
    ap.add_argument("--q-len", type=int, default=4, help="new tokens per sequence (multi-query)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time for the oracle sample")
    args = ap.parse_args(argv)
    gpu_steps = args.component != "block-manager"
    if args.steps is None:
        args.steps = 200 if gpu_steps else 50
    if args.warmup is None:
        args.warmup = 1000 if gpu_steps else 10
    return args


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per step (see the design notes for the definition)."""
    s = wl.spec
    e = {"f32": 4, "f16": 2, "bf16": 2}[s.dtype]
    kv = wl.kv_bytes_logical()
    q_out = 2 * s.batch * s.n_heads * s.d_head * e
    tables = int(sum(-(-int(n) // 16) for n in wl.context_lens)) * 4 + s.batch * 4
    append = 2 * s.batch * s.n_kv_heads * s.d_head * e * 2 + s.batch * 4 * 2
    return {"kv": kv, "kv_unique": wl.kv_bytes_unique(), "decode": kv + q_out + tables,
            "append": append}


def run_config(args, cfg: int, want_cpu: bool) -> dict:
    import torch

    from paged_kv_cache_26_amd import pkv
    from paged_kv_cache_26_amd import workload as wlm

    pkv.load_library()
    t0 = time.time()
    wl = wlm.make_workload(cfg)
    gen_s = time.time() - t0
    dev = torch.device("cuda:0")
    t = wlm.to_torch(wl, dev)
    out = torch.empty_like(t["q"])
    need = pkv.pkv_decode_workspace_bytes(wl.batch, wl.spec.n_heads, wl.spec.n_kv_heads,
                                          wl.spec.d_head, wl.max_context_len, args.partition)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def separate_step(mid_event=None):
        pkv.pkv_kv_append(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"],
                          t["block_tables"], t["positions"], stream=stream)
        if mid_event is not None:
            mid_event.record(stream)
        pkv.pkv_paged_decode_attention(out, t["q"], t["k_pool"], t["v_pool"],
                                       t["block_tables"], t["context_lens"],
                                       wl.max_context_len, wl.scale, args.partition, ws, stream)

    def fused_step(mid_event=None):
        if mid_event is not None:
            mid_event.record(stream)
        pkv.pkv_paged_decode_step(out, t["q"], t["k_pool"], t["v_pool"], t["k_new"],
                                  t["v_new"], t["block_tables"], t["context_lens"],
                                  wl.max_context_len, wl.scale, args.partition, ws, stream)

    fused = not args.separate_append
    step = fused_step if fused else separate_step
    K = args.steps

    def run(fn, per_step):
        """K steps after W warm-up ones; per_step brackets each step (and, for the
        two-launch step, its decode launch) with events, otherwise only the K-step
        region is bracketed. The events are made before the warm-up, so the GPU does not
        sit idle between the warm-up and the timed region (after idle time it needs tens
        of steps to return to its sustained rate)."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        for i in range(K):
            if per_step:
                ev[i][0].record(stream)
                fn(ev[i][1] if fn is separate_step else None)
                ev[i][2].record(stream)
            else:
                fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - w0
        total = e0.elapsed_time(e1)
        if not per_step:
            return total, wall_s, None, None
        st = np.array([e[0].elapsed_time(e[2]) for e in ev])
        la = (np.array([e[1].elapsed_time(e[2]) for e in ev]) if fn is separate_step else st)
        return total, wall_s, st, la

    # The split grid of the step's decode kernel (a host query, which also loads the kernel's
    # code object now rather than during the warm-up).
    split_grid = pkv.pkv_decode_split_workgroups(wl.spec.n_heads, wl.spec.n_kv_heads,
                                                 wl.spec.d_head, 1, t["q"].dtype, 0, fused)
    # The streaming-read ceiling of the line, measured first and right before the warm-up:
    # its ~50 full-bandwidth sweeps keep the GPU busy up to the step's own warm-up (its
    # buffers are released after the timed region, so nothing idles the GPU in between).
    ceiling = stream_ceiling(algorithmic_bytes(wl)["kv"], dev, release=False)
    # The timed region. The fused step is one call (decode kernel + merge kernel), so the
    # region's time per step is that call's duration (the gap between the kernels included)
    # and no per-step events (each costs a few microseconds of GPU time) are recorded in
    # it; the two-call step brackets its decode call with events to time it apart from the
    # append.
    total_ms, wall, step_ms, dec_ms = run(step, per_step=not fused)
    ms_per_step = total_ms / K
    by = algorithmic_bytes(wl)
    value = by["kv"] / (ms_per_step * 1e-3) / 1e9
    dec_avg_s = ms_per_step * 1e-3 if fused else float(dec_ms.mean()) * 1e-3
    launch_bytes = by["decode"] + (by["append"] if fused else 0)
    achieved = launch_bytes / dec_avg_s / 1e9
    torch.cuda.empty_cache()                 # the ceiling's buffers
    # After the timed region: per-step event spread of the fused step, and the other
    # form of the step timed like the timed region.
    if fused:
        _, _, step_ms, _ = run(step, per_step=True)
        dec_ms = step_ms
    other = separate_step if fused else fused_step
    other_us = run(other, per_step=False)[0] / K * 1e3

    spec = wl.spec
    res = {
        "metric": "paged decode attention: KV GB/s read and % of MI355X HBM peak; us/step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded)",
        "config": {
            "workload": spec.name,
            "batch": spec.batch, "n_heads": spec.n_heads, "n_kv_heads": spec.n_kv_heads,
            "d_head": spec.d_head, "block_size": 16,
            "context_tokens": int(wl.context_lens.sum()),
            "max_context_len": wl.max_context_len,
            "kv_split": (f"balanced split over the GPU ({split_grid} workgroups)"
                         if args.partition == 0 else f"fixed {args.partition}-token partitions"),
            "step": ("one call, pkv_paged_decode_step: the decode kernel with the append fused "
                     "in, then the partition merge kernel"
                     if fused else "two calls: pkv_kv_append, then pkv_paged_decode_attention "
                                   "(decode kernel + partition merge kernel)"),
            "kv_bytes_per_step": by["kv"], "kv_unique_bytes_per_step": by["kv_unique"],
            "parallelism": "single GPU",
        },
        "timing": {
            "step_us_median": round(float(np.median(step_ms)) * 1e3, 2),
            "step_us_p10": round(float(np.percentile(step_ms, 10)) * 1e3, 2),
            "step_us_p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2),
            "step_spread_from": ("a second run of K steps with per-step events" if fused
                                 else "per-step events in the timed region"),
            "decode_us_mean": round(dec_avg_s * 1e6, 2),
            "decode_us_median": round(float(np.median(dec_ms)) * 1e3, 2),
            "decode_kv_gbps": round(by["kv"] / dec_avg_s / 1e9, 2),
            ("separate_step_us" if fused else "fused_step_us"): round(other_us, 2),
            "host_wall_us_per_step": round(wall / K * 1e6, 2),
            "workload_gen_s": round(gen_s, 1),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("pkv_paged_decode_step call: decode kernel with the fused append, "
                       "then the partition merge kernel" if fused else
                       "pkv_paged_decode_attention call: decode kernel, then the partition "
                       "merge kernel"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(cfg, args.partition, fused),
            "algorithmic_bytes_per_launch": launch_bytes,
        },
    }
    res["ceiling"] = ceiling
    res["ceiling"]["frac_of_ceiling"] = round(achieved / ceiling["gbps"], 4)
    if cfg == 5:
        res["cold"] = cold_steps(step, args, by, dev, stream)
    if args.copy_calibration:
        res["copy_calibration_bytes"] = copy_calibration(args.copy_calibration)
    if cfg == 5:
        res["timing"]["decode_unique_gbps"] = round(by["kv_unique"] / dec_avg_s / 1e9, 2)
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    # free device memory before the next workload
    del t, out, ws
    torch.cuda.empty_cache()
    return res


def copy_calibration(mib: int) -> dict:
    """Three device copies of exactly mib MiB: dispatches of known traffic for scaling the
    hardware byte counters (FETCH_SIZE, WRITE_SIZE)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    return {"read": n, "write": n}


def stream_ceiling(nbytes: int, dev, reps: int = 10, release: bool = True) -> dict:
    """The achievable read rate: pkv_stream_read over a fresh buffer of nbytes (rounded up
    to 16), best over a few grid sizes, HIP events on the current stream. release=False
    leaves the buffers in torch's cache (no device free, no idle gap) for the caller to
    release later."""
    import torch

    from paged_kv_cache_26_amd import pkv

    n = (nbytes + 15) // 16 * 16
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 32 * 256, dtype=torch.int32, device=dev)
    best, best_wg = 0.0, 0
    for per_cu in (4, 8, 16, 32):
        wg = cus * per_cu
        for _ in range(2):
            pkv.pkv_stream_read(buf, sink, wg)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            pkv.pkv_stream_read(buf, sink, wg)
        e1.record()
        torch.cuda.synchronize()
        gbps = n / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
        if gbps > best:
            best, best_wg = gbps, wg
    del buf, sink
    if release:
        torch.cuda.empty_cache()
    return {"kind": "streaming read (pkv_stream_read, 16-byte non-temporal loads) of a buffer "
                    "of the step's KV bytes", "gbps": round(best, 1), "workgroups": best_wg}


def _flush_buffer(dev):
    """A 1 GiB buffer, written once. Reading it (flush_caches) evicts the 256 MB last-level
    cache (MALL) and the L2s and leaves them holding clean lines: a flush by writing would
    leave ~0.3 GB of dirty lines that the next kernel has to write back first."""
    import torch
    buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    flush_caches(buf)
    return buf


def flush_caches(buf):
    buf.sum()                                # a reduction kernel reads every byte


def cold_steps(step, args, by, dev, stream) -> dict:
    """The same step with the 256 MB last-level cache (MALL) and the L2s flushed before
    each one by reading a 1 GiB buffer outside the timed region (shared blocks then come
    from HBM every step)."""
    import torch

    flush = _flush_buffer(dev)
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        flush_caches(flush)
        ev[i][0].record(stream)
        step(ev[i][1])
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in ev])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    del flush
    torch.cuda.empty_cache()
    dec_s = float(dec_ms.mean()) * 1e-3
    return {"us_per_step_median": round(float(np.median(step_ms)) * 1e3, 2),
            "decode_us_mean": round(dec_s * 1e6, 2),
            "decode_kv_gbps_logical": round(by["kv"] / dec_s / 1e9, 1),
            "decode_unique_gbps": round(by["kv_unique"] / dec_s / 1e9, 1),
            "flush": "a 1 GiB buffer read before each step, outside the timed region"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, target_s: float) -> dict:
    """The fp64 oracle, unchanged, on a bounded sample: whole sequences in order until the
    time budget is spent; GB/s = KV bytes of those sequences / oracle time."""
    from threadpoolctl import threadpool_limits

    from oracle import pkv_oracle as orc

    kp, vp = orc.kv_append(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.block_tables,
                           wl.positions, 16)
    s = wl.spec
    e = {"f32": 4, "f16": 2, "bf16": 2}[s.dtype]

    def passes(budget_s):
        done_bytes, done_seqs, spent = 0, 0, 0.0
        while spent < budget_s:
            for b in range(wl.batch):
                pairs = [(b, h) for h in range(s.n_heads)]
                t0 = time.perf_counter()
                orc.paged_decode_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                           wl.scale, wl.dtype, pairs=pairs)
                spent += time.perf_counter() - t0
                done_bytes += int(wl.context_lens[b]) * 2 * s.n_kv_heads * s.d_head * e
                done_seqs += 1
                if spent >= budget_s:
                    break
        return done_bytes, done_seqs, spent

    with threadpool_limits(limits=1):
        done_bytes, done_seqs, spent = passes(target_s)
    cpus = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cpus):     # the same oracle with BLAS free to use every core
        all_bytes, _, all_spent = passes(target_s / 2)
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_seqs} sequence passes (all heads) over the {wl.batch}-sequence "
                  f"batch in order; {done_bytes} KV bytes in {spent:.1f} s",
        "all_cores_value": round(all_bytes / all_spent / 1e9, 4),
        "all_cores": cpus,
        "cpu": _cpu_model(),
        "host_cpus_available": cpus,
    }


def run_block_manager(args) -> dict:
    """Native block manager on the shared-prefix batch shape, and the GPU block copy.

    Host: 8 groups x 16 sequences forked from a 2048-token prefix; a step reserves the
    next token's slot for all 128 sequences with one batched call (the prefix is block
    aligned, so no copy; 1 step in 16 opens a new block per sequence). Timed against the
    reference manager of the workload module doing the same operations one by one.
    GPU: copy 2048 random 32 KiB blocks in both pools (128 MiB read + 128 MiB written).
    """
    import torch

    from paged_kv_cache_26_amd import pkv
    from paged_kv_cache_26_amd import workload as wlm
    from paged_kv_cache_26_amd.block_manager import NativeBlockManager

    groups, per_group, prefix, steps = 8, 16, 2048, 1024
    n_blocks = groups * 128 + groups * per_group * (steps // 16 + 1)

    def drive(mgr, append):
        for g in range(groups):
            mgr.add_sequence(-1 - g)
            mgr.grow(-1 - g, prefix)
            for i in range(per_group):
                mgr.fork(-1 - g, g * per_group + i)
        t0 = time.perf_counter()
        for t in range(prefix, prefix + steps):
            for sq in range(groups * per_group):
                append(mgr, sq, t)
        return time.perf_counter() - t0

    nat = NativeBlockManager(n_blocks, 16)
    seqs = np.arange(groups * per_group, dtype=np.int64)
    for g in range(groups):
        nat.add_sequence(-1 - g)
        nat.grow(-1 - g, prefix)
        for i in range(per_group):
            nat.fork(-1 - g, g * per_group + i)
    # one C call per step on buffers prepared once (as a native scheduler would call it)
    import ctypes
    toks = np.empty(len(seqs), dtype=np.int32)
    blocks = np.empty(len(seqs), dtype=np.int32)
    slots = np.empty(len(seqs), dtype=np.int32)
    pairs_h = np.empty((len(seqs), 2), dtype=np.int32)
    done = ctypes.c_int32(0)
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    p_seqs, p_toks, p_blk, p_slot, p_pairs = map(ptr, (seqs, toks, blocks, slots, pairs_h))
    fn, handle, n_seq = nat._lib.pkv_bm_append_slots, nat._h, len(seqs)
    t0 = time.perf_counter()
    for t in range(prefix, prefix + steps):
        toks.fill(t)
        if fn(handle, p_seqs, p_toks, n_seq, p_blk, p_slot, p_pairs, ctypes.byref(done)) != 0:
            raise RuntimeError("block manager ran out of blocks")
    t_nat = time.perf_counter() - t0

    def ref_append(m, sq, t):
        m.grow(sq, t + 1)
        m.make_writable(sq, t // 16)

    t_ref = drive(wlm.BlockManager(n_blocks, 16), ref_append)
    appends = steps * groups * per_group

    pkv.load_library()
    dev = torch.device("cuda:0")
    nb, hkv, d = 8192, 8, 128
    kp = torch.empty((nb, 16, hkv, d), dtype=torch.bfloat16, device=dev).normal_()
    vp = torch.empty_like(kp).normal_()
    rng = np.random.default_rng(0)
    perm = rng.permutation(nb)
    pairs = torch.from_numpy(np.stack([perm[:2048], perm[2048:4096]], 1).astype(np.int32)).to(dev)
    for _ in range(args.warmup):
        pkv.pkv_copy_blocks(kp, vp, pairs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        pkv.pkv_copy_blocks(kp, vp, pairs)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    moved = 2 * 2 * 2048 * 16 * hkv * d * 2          # K and V, read and write
    gbps = moved / (ms * 1e-3) / 1e9
    return {
        "metric": "block manager: slot reservations per second (host); copy-on-write block "
                  "copy GB/s (GPU)",
        "value": round(appends / t_nat, 1),
        "unit": "appends/s",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "config": {"workload": "shared-prefix batch: 8 groups x 16 sequences, 2048-token prefix, "
                               f"{steps} decode steps of slot reservations"},
        "host": {"native_us_per_step": round(t_nat / steps * 1e6, 2),
                 "reference_python_us_per_step": round(t_ref / steps * 1e6, 2),
                 "speedup_vs_reference": round(t_ref / t_nat, 1)},
        "copy_blocks": {"blocks": 2048, "block_bytes": 16 * hkv * d * 2, "us": round(ms * 1e3, 2),
                        "GB_per_s": round(gbps, 1),
                        "roofline": {"bound": "hbm", "achieved": round(gbps, 1),
                                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                     "frac": round(gbps / HBM_PEAK_GBPS, 4)}},
    }


def _time_launches(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e-3           # seconds per launch sequence


def _time_cold(fn, steps, dev):
    """Mean duration (s) of fn with the 256 MB last-level cache (MALL) and the L2s flushed
    before each call by reading a 1 GiB buffer; HIP events bracket each call alone."""
    import torch
    flush = _flush_buffer(dev)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        flush_caches(flush)
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    del flush
    torch.cuda.empty_cache()
    return t


def run_multi_query(args) -> dict:
    """q_len new tokens per sequence verified in one pass vs q_len single-token steps.

    Workload: the GQA shape (bf16, 64 sequences, 32 query / 8 KV heads, d 128, contexts
    U{4096..8192}) with q_len new tokens per sequence; the step appends all of them and
    attends in one call (pkv_paged_multi_query_step: decode kernel + merge kernel); the line
    also reports the two-call step (pkv_kv_append_tokens + pkv_paged_multi_query_attention).
    The comparison runs q_len single-query steps (append + decode) over the same growing
    context.
    """
    import dataclasses

    import torch

    from paged_kv_cache_26_amd import pkv
    from paged_kv_cache_26_amd import workload as wlm

    ql = args.q_len
    spec = dataclasses.replace(wlm.SPECS[3], name=f"gqa-bf16-verify{ql}", q_len=ql)
    wl = wlm.make_workload(spec, seed=3)
    t = wlm.to_torch(wl, torch.device("cuda:0"))
    out = torch.empty_like(t["q"])
    need = pkv.pkv_multi_query_workspace_bytes(wl.batch, ql, spec.n_heads, spec.n_kv_heads,
                                               spec.d_head, wl.max_context_len, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")

    def mq_step():
        pkv.pkv_paged_multi_query_step(out, t["q"], t["k_pool"], t["v_pool"], t["k_new"],
                                       t["v_new"], t["block_tables"], t["context_lens"],
                                       wl.max_context_len, wl.scale, 0, ws)

    def mq_two_launches():
        pkv.pkv_kv_append_tokens(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"],
                                 t["block_tables"], t["positions"])
        pkv.pkv_paged_multi_query_attention(out, t["q"], t["k_pool"], t["v_pool"],
                                            t["block_tables"], t["context_lens"],
                                            wl.max_context_len, wl.scale, 0, ws)

    def mq_attn():
        pkv.pkv_paged_multi_query_attention(out, t["q"], t["k_pool"], t["v_pool"],
                                            t["block_tables"], t["context_lens"],
                                            wl.max_context_len, wl.scale, 0, ws)

    # sequential alternative: q_len single-query steps, context growing by one each time
    qs = [t["q"][:, i].contiguous() for i in range(ql)]
    kn = [t["k_new"][:, i].contiguous() for i in range(ql)]
    vn = [t["v_new"][:, i].contiguous() for i in range(ql)]
    lens = [(t["context_lens"] - ql + i + 1).contiguous() for i in range(ql)]
    pos = [(t["positions"] + i).contiguous() for i in range(ql)]
    out1 = torch.empty_like(qs[0])
    need1 = pkv.pkv_decode_workspace_bytes(wl.batch, spec.n_heads, spec.n_kv_heads,
                                           spec.d_head, wl.max_context_len, 0)
    ws1 = torch.empty(max(need1, 1), dtype=torch.uint8, device="cuda:0")

    def seq_steps():
        for i in range(ql):
            pkv.pkv_kv_append(t["k_pool"], t["v_pool"], kn[i], vn[i], t["block_tables"], pos[i])
            pkv.pkv_paged_decode_attention(out1, qs[i], t["k_pool"], t["v_pool"],
                                           t["block_tables"], lens[i], wl.max_context_len,
                                           wl.scale, 0, ws1)

    s_step = _time_launches(mq_step, args.steps, args.warmup)
    s_two = _time_launches(mq_two_launches, args.steps, args.warmup)
    s_attn = _time_launches(mq_attn, args.steps, args.warmup)
    s_seq = _time_launches(seq_steps, args.steps, args.warmup)
    kv = wl.kv_bytes_logical()
    alg = kv + 2 * wl.q.nbytes + int(sum(-(-int(n) // 16) for n in wl.context_lens)) * 4
    gbps = alg / s_attn / 1e9
    return {
        "metric": f"multi-query paged attention (q_len {ql}): KV GB/s read; us/step",
        "value": round(kv / s_step / 1e9, 2),
        "unit": "GB/s",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "dtype": spec.dtype,
        "us_per_step": round(s_step * 1e6, 2),
        "config": {"workload": spec.name, "batch": spec.batch, "q_len": ql,
                   "n_heads": spec.n_heads, "n_kv_heads": spec.n_kv_heads, "d_head": spec.d_head,
                   "context_tokens": int(wl.context_lens.sum())},
        "step": "one call, pkv_paged_multi_query_step: the decode kernel with the q_len tokens "
                "appended inside it, then the partition merge kernel",
        "two_launch_step_us": round(s_two * 1e6, 2),
        "attention_us": round(s_attn * 1e6, 2),
        "sequential_single_query_us": round(s_seq * 1e6, 2),
        "speedup_vs_sequential": round(s_seq / s_step, 2),
        "roofline": {"bound": "hbm", "kernel": "pkv_paged_multi_query_attention call: decode "
                     "kernel, then the merge kernel", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("multi-query", ql),
                     "algorithmic_bytes_per_launch": alg},
    }


def run_shared_prefix(args) -> dict:
    """The shared-prefix workload (bf16, 128 sequences in 8 groups of 16 over a 2048-token
    prefix, suffixes U{64..1024}, 32 query / 8 KV heads, d 128): one step appends every new
    token and runs pkv_paged_decode_attention_shared_prefix, which reads each group's 128
    shared blocks once. Compared with pkv_paged_decode_attention on the same batch, which
    reads them once per sequence."""
    import torch

    from paged_kv_cache_26_amd import pkv
    from paged_kv_cache_26_amd import workload as wlm
    from paged_kv_cache_26_amd.block_manager import find_shared_prefixes

    pkv.load_library()
    wl = wlm.make_workload(5)
    spec = wl.spec
    dev = torch.device("cuda:0")
    t = wlm.to_torch(wl, dev)
    out = torch.empty_like(t["q"])
    t_host = time.perf_counter()
    grp = find_shared_prefixes(wl.block_tables, wl.context_lens)
    group_us = (time.perf_counter() - t_host) * 1e6
    sg = torch.from_numpy(grp.seq_group).to(dev)
    gb = torch.from_numpy(grp.group_blocks).to(dev)
    need = pkv.pkv_shared_prefix_workspace_bytes(wl.batch, spec.n_heads, spec.n_kv_heads,
                                                 spec.d_head, grp.max_shared_blocks)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    need1 = pkv.pkv_decode_workspace_bytes(wl.batch, spec.n_heads, spec.n_kv_heads, spec.d_head,
                                           wl.max_context_len, 0)
    ws1 = torch.empty(max(need1, 1), dtype=torch.uint8, device=dev)

    def append():
        pkv.pkv_kv_append(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"], t["block_tables"],
                          t["positions"])

    def shared():
        pkv.pkv_paged_decode_attention_shared_prefix(
            out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"], t["context_lens"], sg, gb,
            grp.max_group_size, grp.max_shared_blocks, wl.max_context_len, wl.scale, ws)

    def plain():
        pkv.pkv_paged_decode_attention(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                                       t["context_lens"], wl.max_context_len, wl.scale, 0, ws1)

    def step():
        append()
        shared()

    s_step = _time_launches(step, args.steps, args.warmup)
    s_shared = _time_launches(shared, args.steps, args.warmup)
    s_plain = _time_launches(plain, args.steps, args.warmup)
    cold_shared = _time_cold(shared, args.steps, dev)
    cold_plain = _time_cold(plain, args.steps, dev)
    by = algorithmic_bytes(wl)
    q_out = 2 * wl.q.nbytes
    tables = int(sum(-(-int(n) // 16) for n in wl.context_lens)) * 4
    alg = by["kv_unique"] + q_out + tables
    gbps = alg / s_shared / 1e9
    return {
        "metric": "shared-prefix paged decode: logical KV GB/s (tokens attended x bytes); us/step",
        "value": round(by["kv"] / s_step / 1e9, 2),
        "unit": "GB/s",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "dtype": spec.dtype,
        "data": "synthetic (seeded)",
        "us_per_step": round(s_step * 1e6, 2),
        "config": {"workload": spec.name, "batch": spec.batch, "groups": spec.groups,
                   "prefix_len": spec.prefix_len, "suffix_range": list(spec.suffix_range),
                   "n_heads": spec.n_heads, "n_kv_heads": spec.n_kv_heads,
                   "d_head": spec.d_head, "context_tokens": int(wl.context_lens.sum()),
                   "kv_bytes_per_step": by["kv"], "kv_unique_bytes_per_step": by["kv_unique"]},
        "attention_us": round(s_shared * 1e6, 2),
        "plain_decode_attention_us": round(s_plain * 1e6, 2),
        "speedup_vs_plain_decode": round(s_plain / s_shared, 2),
        "unique_kv_gbps": round(by["kv_unique"] / s_shared / 1e9, 1),
        "cold": {"attention_us_mean": round(cold_shared * 1e6, 2),
                 "plain_decode_attention_us_mean": round(cold_plain * 1e6, 2),
                 "unique_kv_gbps": round(by["kv_unique"] / cold_shared / 1e9, 1),
                 "frac_of_hbm_peak_unique": round(alg / cold_shared / 1e9 / HBM_PEAK_GBPS, 4),
                 "flush": "a 1 GiB buffer read before each call, outside the timed call, so "
                          "the shared prefix comes from HBM"},
        "host_grouping_us": round(group_us, 1),
        "roofline": {"bound": "hbm", "kernel": "pkv_paged_decode_attention_shared_prefix call: "
                     "split kernel with the prefix tasks, then the merge", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("shared-prefix"),
                     "algorithmic_bytes_per_launch": alg},
    }


def run_quantized(args) -> dict:
    """The GQA workload shape (64 sequences of U{4096..8192} tokens, 32 query / 8 KV heads,
    d 128, q and out bf16) with an 8-bit KV cache: a step quantizes every new token into
    the cache (pkv_kv_append_quantized) and runs pkv_paged_decode_attention_quantized.
    Compared with the bf16-cache step on the same shape and lengths."""
    import torch

    from paged_kv_cache_26_amd import pkv
    from paged_kv_cache_26_amd import workload as wlm

    pkv.load_library()
    fmt = args.kv_format
    wl = wlm.make_workload(wlm.QUANT_SPECS[fmt], seed=3)
    spec = wl.spec
    dev = torch.device("cuda:0")
    t = wlm.to_torch(wl, dev)
    out = torch.empty_like(t["q"])
    need = pkv.pkv_decode_workspace_bytes(wl.batch, spec.n_heads, spec.n_kv_heads, spec.d_head,
                                          wl.max_context_len, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def append():
        pkv.pkv_kv_append_quantized(t["k_pool"], t["v_pool"], t["k_scales"], t["v_scales"],
                                    t["k_new"], t["v_new"], t["block_tables"], t["positions"],
                                    fmt)

    def attend():
        pkv.pkv_paged_decode_attention_quantized(out, t["q"], t["k_pool"], t["v_pool"],
                                                 t["k_scales"], t["v_scales"], t["block_tables"],
                                                 t["context_lens"], wl.max_context_len, fmt,
                                                 wl.scale, 0, ws)

    def step():
        append()
        attend()

    s_step = _time_launches(step, args.steps, args.warmup)
    s_attn = _time_launches(attend, args.steps, args.warmup)
    del t, out, ws
    torch.cuda.empty_cache()
    # the same shape and lengths with a bf16 cache (workload 3, same seed)
    ref = wlm.make_workload(3)
    assert np.array_equal(ref.context_lens, wl.context_lens)
    tr = wlm.to_torch(ref, dev)
    out16 = torch.empty_like(tr["q"])
    ws16 = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    s_bf16 = _time_launches(
        lambda: pkv.pkv_paged_decode_attention(out16, tr["q"], tr["k_pool"], tr["v_pool"],
                                               tr["block_tables"], tr["context_lens"],
                                               ref.max_context_len, ref.scale, 0, ws16),
        args.steps, args.warmup)
    kv = wl.kv_bytes_logical()
    tables = int(sum(-(-int(n) // 16) for n in wl.context_lens)) * 4
    alg = kv + 2 * wl.q.nbytes + tables + 4 * wl.batch
    gbps = alg / s_attn / 1e9
    tokens = int(wl.context_lens.sum())
    return {
        "metric": f"paged decode attention over a {fmt} KV cache: KV GB/s read; us/step",
        "value": round(kv / s_step / 1e9, 2),
        "unit": "GB/s",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "dtype": f"{fmt} KV, bf16 q/out",
        "data": "synthetic (seeded)",
        "us_per_step": round(s_step * 1e6, 2),
        "config": {"workload": spec.name, "batch": spec.batch, "n_heads": spec.n_heads,
                   "n_kv_heads": spec.n_kv_heads, "d_head": spec.d_head,
                   "context_tokens": tokens, "kv_bytes_per_token": wl.kv_bytes_per_token(),
                   "kv_bytes_per_step": kv},
        "attention_us": round(s_attn * 1e6, 2),
        "bf16_cache_attention_us": round(s_bf16 * 1e6, 2),
        "speedup_vs_bf16_cache": round(s_bf16 / s_attn, 2),
        "context_tokens_per_s": round(tokens / s_attn, 1),
        "roofline": {"bound": "hbm", "kernel": f"pkv_paged_decode_attention_quantized call "
                     f"({fmt} cache): decode kernel, then the merge kernel",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("quantized", fmt),
                     "algorithmic_bytes_per_launch": alg},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") != "1":
        print("the benchmark runs on one GPU only", file=sys.stderr)
        sys.exit(2)
    if args.component == "block-manager":
        print(json.dumps(run_block_manager(args)), flush=True)
        return
    if args.component != "decode" and args.copy_calibration:
        copy_calibration(args.copy_calibration)
    if args.component == "multi-query":
        print(json.dumps(run_multi_query(args)), flush=True)
        return
    if args.component == "shared-prefix":
        print(json.dumps(run_shared_prefix(args)), flush=True)
        return
    if args.component == "quantized":
        print(json.dumps(run_quantized(args)), flush=True)
        return
    cfgs = [1, 2, 3, 4, 5] if args.all else [args.config]
    for cfg in cfgs:
        res = run_config(args, cfg, want_cpu=not args.no_cpu_baseline)
        if not args.all:
            also = also_workloads(args)
            if also:
                res["also_measured"] = [also_summary(run_config(args, c, want_cpu=False))
                                        for c in also]
        print(json.dumps(res), flush=True)


def also_workloads(args) -> list:
    """Workloads timed after the main one in the same line: --also, else the long-context
    GQA layer (4) beside the GQA layer (3)."""
    if args.also is None:
        return [4] if args.config == 3 else []
    ids = [int(x) for x in args.also.split(",") if x.strip()]
    bad = [i for i in ids if i not in (1, 2, 3, 4, 5)]
    if bad:
        raise SystemExit(f"--also: unknown workload ids {bad}")
    return [i for i in ids if i != args.config]


def also_summary(res: dict) -> dict:
    """The figures of a secondary workload's line, timed the same way as the main one."""
    keys = ("value", "unit", "us_per_step", "pct_of_hbm_peak", "dtype", "steps", "warmup")
    out = {"workload": res["config"]["workload"]}
    out.update({k: res[k] for k in keys})
    out["config"] = res["config"]
    out["roofline"] = res["roofline"]
    out["ceiling"] = res["ceiling"]
    out["timing"] = {k: res["timing"][k] for k in ("step_us_median", "decode_kv_gbps",
                                                     "separate_step_us")
                     if k in res["timing"]}
    return out


if __name__ == "__main__":
    main()
