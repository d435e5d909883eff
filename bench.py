#!/usr/bin/env python3
"""Benchmark of the stable co-rank merge on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path over resident inputs: the
partition kernel (one co-rank per segment boundary) and the segment merge
kernel, launched through the C ABI on the current torch stream.  The default
workload is 2^28 + 2^28 int32 keys iid uniform over the int32 range, sorted.

Before timing, the merged output of one untimed launch is compared with the
CPU oracle on every element (a wrong answer never produces a number); that
oracle run is the first run of the reported CPU baseline, whose other runs
come after the GPU timing.  Then W untimed steps (the default 50, ~40 ms,
covers the device's clock ramp after the seconds of CPU work), then exactly
K timed steps back to back between device synchronisations (the step rate).  The same K steps are then run again with a HIP event pair around
every segment-merge launch, which gives that kernel's mean duration for the
roofline figure.  A streaming copy of the same byte count is timed beside it
as the bandwidth this device actually delivers.

Prints ONE JSON line on stdout; the device banner and extra figures go to
stderr.  Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
SORT_SEED = 20261207  # inputs of the sort and batched-merge timings
METRIC = "merged elements/sec and achieved HBM GB/s (% of MI355X peak), int32 m=n=2^28"
COUNTER_FILE = os.path.join(ROOT, "profiles", "merge_segments_uniform_i32_2p28x2p28_traffic.md")
KERNEL_SOURCES = ["corank.hpp", "merge_kernel.hpp", "omerge.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the headline kernel's sources with comments and whitespace
    removed: it changes when the code does, not when a comment does."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "ordered_merge_sorted_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per segment-merge launch from the committed counter summary,
    if it was taken on the kernel source as it is now; else None."""
    if not os.path.exists(COUNTER_FILE):
        return None
    text = open(COUNTER_FILE).read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def device_banner(torch):
    p = torch.cuda.get_device_properties(0)
    arch = getattr(p, "gcnArchName", "?")
    log("GPU: %s (%s), %d CUs, %.1f GiB, L2 %s MiB" % (
        p.name, arch, p.multi_processor_count, p.total_memory / 2**30,
        getattr(p, "L2_cache_size", 0) / 2**20 if hasattr(p, "L2_cache_size") else "?"))
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    log("host: %d cores available to this process (nproc %s)" % (cores, os.cpu_count()))
    return arch


def run_oracle(w, arrs):
    """One single-threaded run of the CPU oracle on the full workload.
    Returns (out, seconds)."""
    import oracle
    t0 = time.perf_counter()
    out = oracle.merge_kv(*arrs) if w.kv else oracle.merge_i32(*arrs)
    return out, time.perf_counter() - t0


def time_oracle(w, arrs, first_s, want_runs_s=12.0, max_runs=8):
    """Rates of the single-threaded CPU oracle on the full workload: the run
    already made for the check (first_s seconds), then more runs until about
    want_runs_s seconds have passed (at most max_runs in all)."""
    secs = [first_s]
    while len(secs) < max_runs and sum(secs) < want_runs_s:
        secs.append(run_oracle(w, arrs)[1])
    for r, dt in enumerate(secs):
        log("oracle run %d: %.2f s, %.3g elements/s" % (r, dt, w.total / dt))
    return [w.total / dt for dt in secs]


def ablation(om, d_arrs, want, w, stream):
    """Global-memory kernels of the pages (no LDS) on the same inputs: one
    co-rank search then a walk, or two searches per slice, at 1..256 outputs
    per lane.  Each is checked against the oracle before it is timed."""
    import torch
    out = torch.empty(w.total, dtype=torch.int32, device=d_arrs[0].device)
    log("ablation: global-memory merge kernels vs the LDS-tiled segment merge")
    log("%-28s %10s %10s %8s" % ("kernel", "ms", "GB/s", "% peak"))
    for two in (False, True):
        for per in (1, 4, 16, 64, 256):
            def go():
                om.merge_i32_direct(d_arrs[0], d_arrs[1], per_thread=per, two_searches=two,
                                    out=out, stream=stream)
            out.fill_(-1)
            go()
            torch.cuda.synchronize()
            if not np.array_equal(out.cpu().numpy(), want):
                log("FAILED: direct kernel per=%d two_searches=%s differs from the oracle" % (per, two))
                sys.exit(1)
            for _ in range(2):
                go()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                go()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 5
            gbs = w.roofline_bytes / (ms * 1e-3) / 1e9
            log("%-28s %10.3f %10.1f %8.1f" % ("%s, %d per lane" % ("two searches" if two else "search+walk", per),
                                                ms, gbs, 100 * gbs / HBM_PEAK_GBS))


def typed_orders(om, d_arrs, c_ref, w, stream):
    """The key orders of omerge_merge_keys on inputs derived from the int32
    workload on the device: uint32 keys x ^ 2^31, float32 keys with bits
    (x ^ 2^31) >> 1 (non-negative patterns, so bit order is totalOrder; some
    are infinities and NaNs), int64 keys x * 2^32 and float64 keys with bits
    (x ^ 2^31 as uint32) << 31, each ascending and reversed for descending.
    Each output is checked against the same map of the int32 merge output
    (keys only: the sorted multiset is unique) before it is timed."""
    import torch
    log("key orders (omerge_merge_keys, %s)" % w.name)
    log("%-28s %10s %10s %8s" % ("order", "ms", "GB/s", "% peak"))
    sign = torch.tensor(-(1 << 31), dtype=torch.int32, device=c_ref.device)
    maps = {
        "int32": (lambda x: x, torch.int32),
        "uint32": (lambda x: x ^ sign, getattr(torch, "uint32", torch.int32)),
        "float32": (lambda x: torch.bitwise_right_shift((x ^ sign).view(torch.int32), 1) &
                    0x7FFFFFFF, torch.float32),
        # 64-bit keys: x * 2^32 (int64), and the 32-bit unsigned image shifted
        # into a non-negative binary64 pattern (float64)
        "int64": (lambda x: x.to(torch.int64) << 32, torch.int64),
        "float64": (lambda x: ((x ^ sign).to(torch.int64) & 0xFFFFFFFF) << 31, torch.float64),
    }
    for name, (f, tdt) in maps.items():
        if name == "uint32" and tdt is torch.int32:
            continue
        for desc in (False, True):
            a, b = (f(x) for x in d_arrs[:2])
            want = f(c_ref)
            if desc:
                a, b, want = a.flip(0), b.flip(0), want.flip(0)
            a, b = a.contiguous().view(tdt), b.contiguous().view(tdt)
            out = torch.empty(w.total, dtype=tdt, device=c_ref.device)

            def go():
                om.merge(a, b, descending=desc, out=out, stream=stream)
            go()
            torch.cuda.synchronize()
            bits = torch.int32 if out.element_size() == 4 else torch.int64
            if not torch.equal(out.view(bits), want.contiguous()):
                log("FAILED: key order %s%s differs from the mapped int32 merge" %
                    (name, " desc" if desc else ""))
                sys.exit(1)
            _warm(go)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                go()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            gbs = 2 * w.total * out.element_size() / (ms * 1e-3) / 1e9
            log("%-28s %10.3f %10.1f %8.1f" % (name + (" descending" if desc else " ascending"),
                                                ms, gbs, 100 * gbs / HBM_PEAK_GBS))
            del a, b, out, want


def _warm(fn, seconds=0.03):
    """Runs fn (synchronising) until `seconds` have passed, at least twice:
    the device leaves its idle clocks before anything is timed."""
    import torch
    t0, n = time.perf_counter(), 0
    while n < 2 or time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()
        n += 1


def _time(fn, stream, reps=5):
    import torch
    _warm(fn)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def sort_and_batch(om, stream):
    """The merge sort and the batched merge on 2^28 int32 keys (and 2^27
    key+payload pairs), each checked against torch's stable sort before it
    is timed; torch.sort is timed beside it for context."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(SORT_SEED)
    log("merge sort and batched merge (int32)")
    log("%-44s %10s %14s" % ("case", "ms", "elements/s"))
    n = 1 << 28
    keys = torch.randint(-(1 << 31), (1 << 31) - 1, (n,), dtype=torch.int32, device=dev,
                         generator=g)
    out = torch.empty_like(keys)
    om.sort(keys, out=out, stream=stream)
    ref = torch.sort(keys, stable=True).values
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        log("FAILED: omerge sort differs from torch's stable sort")
        sys.exit(1)
    ms = _time(lambda: om.sort(keys, out=out, stream=stream), stream)
    log("%-44s %10.3f %14.4g" % ("omerge sort, 2^28 int32 keys", ms, n / (ms * 1e-3)))
    ms_t = _time(lambda: torch.sort(keys, stable=True), stream)
    log("%-44s %10.3f %14.4g" % ("torch.sort(stable=True), same keys", ms_t, n / (ms_t * 1e-3)))
    del out, ref
    n2 = 1 << 27
    k2 = keys[:n2].clone()
    v2 = torch.arange(n2, dtype=torch.int32, device=dev)
    ok_, ov_ = torch.empty_like(k2), torch.empty_like(v2)
    om.sort(k2, v2, out=ok_, out_vals=ov_, stream=stream)
    rk, ri = torch.sort(k2, stable=True)
    torch.cuda.synchronize()
    if not (torch.equal(ok_, rk) and torch.equal(ov_, ri.to(torch.int32))):
        log("FAILED: omerge pair sort differs from torch's stable sort")
        sys.exit(1)
    ms = _time(lambda: om.sort(k2, v2, out=ok_, out_vals=ov_, stream=stream), stream)
    log("%-44s %10.3f %14.4g" % ("omerge sort, 2^27 int32 keys + payloads", ms, n2 / (ms * 1e-3)))
    del k2, v2, ok_, ov_, rk, ri
    # other key types: float32 descending and int64
    for name, tens, desc in (
            ("float32 descending", torch.randn(1 << 27, device=dev, generator=g), True),
            ("int64", torch.randint(-(1 << 62), 1 << 62, (1 << 27,), dtype=torch.int64, device=dev,
                                    generator=g), False)):
        o = torch.empty_like(tens)
        om.sort(tens, descending=desc, out=o, stream=stream)
        ref = torch.sort(tens, stable=True, descending=desc).values
        torch.cuda.synchronize()
        if not torch.equal(o, ref):
            log("FAILED: omerge sort (%s) differs from torch's stable sort" % name)
            sys.exit(1)
        ms = _time(lambda: om.sort(tens, descending=desc, out=o, stream=stream), stream)
        ms_t = _time(lambda: torch.sort(tens, stable=True, descending=desc), stream)
        log("%-44s %10.3f %14.4g  (torch.sort %.3f ms)" % (
            "omerge sort, 2^27 %s keys" % name, ms, tens.numel() / (ms * 1e-3), ms_t))
        del tens, o, ref
    # 2^15 merges of 4096 + 4096 sorted keys each (2^28 outputs)
    pairs, L = 1 << 15, 4096
    a = torch.sort(keys[:pairs * L].view(pairs, L), dim=1).values.reshape(-1)
    b = torch.sort(keys[pairs * L:2 * pairs * L].view(pairs, L), dim=1).values.reshape(-1)
    offs = torch.arange(0, pairs * L + 1, L, dtype=torch.int64, device=dev)
    c = torch.empty(2 * pairs * L, dtype=torch.int32, device=dev)
    om.merge_batched(a, offs, b, offs, out=c, stream=stream)
    ref = torch.sort(torch.cat([a.view(pairs, L), b.view(pairs, L)], dim=1), dim=1).values
    torch.cuda.synchronize()
    if not torch.equal(c.view(pairs, 2 * L), ref):
        log("FAILED: omerge batched merge differs from torch's per-merge sort")
        sys.exit(1)
    ms = _time(lambda: om.merge_batched(a, offs, b, offs, out=c, stream=stream), stream)
    gbs = 2 * c.numel() * 4 / (ms * 1e-3) / 1e9
    log("%-44s %10.3f %14.4g  (%.0f GB/s, %.1f%% of peak)" % (
        "batched: 2^15 merges of 4096+4096", ms, c.numel() / (ms * 1e-3), gbs,
        100 * gbs / HBM_PEAK_GBS))
    # 2^22 merges of 16 + 16 keys each (the tile path for short merges)
    pairs, L = 1 << 22, 16
    a = torch.sort(keys[:pairs * L].view(pairs, L), dim=1).values.reshape(-1)
    b = torch.sort(keys[pairs * L:2 * pairs * L].view(pairs, L), dim=1).values.reshape(-1)
    offs = torch.arange(0, pairs * L + 1, L, dtype=torch.int64, device=dev)
    c = torch.empty(2 * pairs * L, dtype=torch.int32, device=dev)
    om.merge_batched(a, offs, b, offs, out=c, stream=stream)
    ref = torch.sort(torch.cat([a.view(pairs, L), b.view(pairs, L)], dim=1), dim=1).values
    torch.cuda.synchronize()
    if not torch.equal(c.view(pairs, 2 * L), ref):
        log("FAILED: omerge batched merge (short merges) differs from torch's per-merge sort")
        sys.exit(1)
    ms = _time(lambda: om.merge_batched(a, offs, b, offs, out=c, stream=stream), stream)
    gbs = 2 * c.numel() * 4 / (ms * 1e-3) / 1e9
    log("%-44s %10.3f %14.4g  (%.0f GB/s, %.1f%% of peak)" % (
        "batched: 2^22 merges of 16+16", ms, c.numel() / (ms * 1e-3), gbs,
        100 * gbs / HBM_PEAK_GBS))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None, help="workload name (default: the int32 2^28+2^28 merge)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the oracle (the output check still runs)")
    ap.add_argument("--ablation", action="store_true",
                    help="also time the global-memory (no LDS) merge kernels at 1..256 outputs "
                         "per lane, each checked against the oracle, every key order of "
                         "omerge_merge_keys, the merge sort and the batched merge; tables on "
                         "stderr")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    import torch

    import ordered_merge_sorted_amd as om
    from ordered_merge_sorted_amd.workloads import HEADLINE, WORKLOADS

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    arch = device_banner(torch)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    t0 = time.perf_counter()
    arrs = w.make()
    log("workload %s: m=%d n=%d (%s); generated in %.1f s" % (name, w.m, w.n, w.description,
                                                             time.perf_counter() - t0))

    # Inputs resident in HBM before anything is timed.
    def to_dev(x):
        return torch.from_numpy(x.view(np.int32) if x.dtype == np.uint32 else x).to(dev)

    d_arrs = [to_dev(x) for x in arrs]
    total = w.total
    seg_len = om.segment_length(w.m, w.n, kv=w.kv)
    count = om.partition_count(total, seg_len)
    part = torch.empty(count, dtype=torch.int64, device=dev)
    if w.kv:
        out_k = torch.empty(total, dtype=torch.int32, device=dev)
        out_v = torch.empty(total, dtype=torch.int32, device=dev)
    else:
        out = torch.empty(total, dtype=torch.int32, device=dev)

    def launch_partition():
        om.partition(d_arrs[0], d_arrs[2] if w.kv else d_arrs[1], seg_len, out=part, stream=stream)

    def launch_merge():
        if w.kv:
            om.merge_segments_kv(d_arrs[0], d_arrs[1], d_arrs[2], d_arrs[3], part, seg_len,
                                 out_keys=out_k, out_vals=out_v, stream=stream)
        else:
            om.merge_segments_i32(d_arrs[0], d_arrs[1], part, seg_len, out=out, stream=stream)

    # One untimed, checked step (every element against the oracle).
    launch_partition()
    launch_merge()
    torch.cuda.synchronize()
    # The oracle's run for the check is also the first CPU-baseline run; the
    # rest of the CPU baseline is timed after the GPU, so that the GPU
    # timing does not start from a device left idle for seconds.
    want, oracle_s = run_oracle(w, arrs)
    if args.ablation and not w.kv:
        ablation(om, d_arrs, want, w, stream)
    if w.kv:
        ok = np.array_equal(out_k.cpu().numpy(), want[0]) and \
            np.array_equal(out_v.cpu().numpy().view(np.uint32), want[1])
    else:
        ok = np.array_equal(out.cpu().numpy(), want)
    if not ok:
        log("FAILED: the merged output differs from the oracle; no number is reported")
        sys.exit(1)
    log("checked: output bit-exact against the oracle (%d elements)" % total)
    del want
    if args.ablation and not w.kv:
        typed_orders(om, d_arrs, out, w, stream)
        sort_and_batch(om, stream)

    # Warmup, then exactly K timed steps.
    for _ in range(args.warmup):
        launch_partition()
        launch_merge()
    torch.cuda.synchronize()

    # Timed region 1 (the step rate): exactly K steps back to back, bracketed
    # by device synchronisation, one event pair and the host clock.
    start_all = torch.cuda.Event(enable_timing=True)
    stop_all = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    start_all.record(stream)
    for k in range(args.steps):
        launch_partition()
        launch_merge()
    stop_all.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    ms_total = start_all.elapsed_time(stop_all)
    ms_step = ms_total / args.steps

    # Timed region 2 (the roofline figure): the same K steps with a HIP event
    # pair around every segment-merge launch on its stream.  (The extra event
    # packets cost ~1.5% of a step, so region 1 alone gives the step rate.)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        launch_partition()
        ev[k][0].record(stream)
        launch_merge()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    merge_ms = [a.elapsed_time(b) for a, b in ev]
    merge_ms_mean = float(np.mean(merge_ms))

    bpe = w.bytes_per_element
    alg_bytes = 2 * total * bpe  # each element read once and written once
    value = total / (ms_step * 1e-3)
    step_gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    kern_gbs = alg_bytes / (merge_ms_mean * 1e-3) / 1e9

    # Streaming copy of the same byte count: the bandwidth this device gives.
    src = torch.empty(total * bpe // 4, dtype=torch.int32, device=dev)
    src.random_(0, 1 << 30)
    dst = torch.empty_like(src)
    for _ in range(3):
        om.stream_copy(src, out=dst, stream=stream)
    cs, ce = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    cs.record(stream)
    for _ in range(reps):
        om.stream_copy(src, out=dst, stream=stream)
    ce.record(stream)
    torch.cuda.synchronize()
    copy_ms = cs.elapsed_time(ce) / reps
    copy_gbs = alg_bytes / (copy_ms * 1e-3) / 1e9
    del src, dst

    # One-call API (includes its stream-ordered scratch allocation).
    if not w.kv:
        onecall_ms = _time(lambda: om.merge_i32(d_arrs[0], d_arrs[1], out=out, stream=stream),
                           stream, reps=10)
    else:
        onecall_ms = None

    log("step: %.4f ms (host clock %.4f ms/step) -> %.4g elements/s, %.1f GB/s (%.1f%% of %.0f)" % (
        ms_step, t_host * 1e3 / args.steps, value, step_gbs, 100 * step_gbs / HBM_PEAK_GBS, HBM_PEAK_GBS))
    log("segment merge kernel: %.4f ms mean (min %.4f, max %.4f) -> %.1f GB/s" % (
        merge_ms_mean, min(merge_ms), max(merge_ms), kern_gbs))
    log("partition kernel + gaps: %.4f ms per step" % (ms_step - merge_ms_mean))
    log("stream copy of the same bytes: %.4f ms -> %.1f GB/s; merge step at %.1f%% of it" % (
        copy_ms, copy_gbs, 100 * step_gbs / copy_gbs))
    if onecall_ms is not None:
        log("merge_i32 one call (with its scratch allocation): %.4f ms" % onecall_ms)

    cpu = None
    rates = [] if args.no_cpu_baseline else time_oracle(w, arrs, oracle_s)
    if rates:
        cpu = {"value": float(np.median(rates)), "unit": "merged elements/s", "cores": 1,
               "kind": "oracle",
               "sample": "full workload (%d + %d elements), %d run(s), median; single-threaded C "
                         "two-pointer merge" % (w.m, w.n, len(rates))}

    traffic = recorded_traffic() if name == HEADLINE else None
    line = {
        "metric": METRIC if name == HEADLINE else "merged elements/sec (%s)" % name,
        "value": value,
        "unit": "merged elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32+uint32" if w.kv else "int32",
        "data": "synthetic",
        "config": {"workload": name, "m": w.m, "n": w.n, "key_payload": w.kv,
                   "seg_len": seg_len, "segments": count - 1, "gpu_arch": arch},
        "gbps": step_gbs,
        "pct_hbm_peak": 100 * step_gbs / HBM_PEAK_GBS,
        "copy_gbps_same_bytes": copy_gbs,
        "roofline": {"bound": "hbm", "achieved": kern_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kern_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "merge_segments_kernel", "kernel_ms": merge_ms_mean,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
