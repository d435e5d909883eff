#!/usr/bin/env python3
"""Benchmark of the stable co-rank merge on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path over resident inputs: the
partition kernel (one co-rank per segment boundary) and the segment merge
kernel, launched through the C ABI on the current torch stream.  The default
workload is 2^28 + 2^28 int32 keys iid uniform over the int32 range, sorted.

Order of work (a wrong answer never produces a number, and the timed steps
never follow seconds of device idle):
  1. The inputs are generated and the CPU oracle merges them, before anything
     runs on the device.  That oracle run is the first run of the reported
     CPU baseline.
  2. One untimed step is checked against the oracle on every element.
  3. The bandwidth references run on the same byte count: the library's
     16-byte streaming copy kernel and, independently, a device-to-device
     hipMemcpyAsync (torch's copy_); then the one-call merge_i32.  They keep
     the device busy right up to the warm-up.
  4. Exactly W untimed steps, then exactly K timed steps back to back between
     device synchronisations: the step rate.
  5. The same K steps again with a HIP event pair around each kernel on its
     stream: the partition's and the segment merge's mean launch durations
     (the roofline figure is the merge kernel's).
  6. The output of the last timed step is checked against the oracle again.
  7. The other four workloads, each checked on every element before it is
     timed, one row each on stderr (and in the JSON line).
  8. More oracle runs, up to about 12 s of CPU work in all: the CPU baseline.

Prints ONE JSON line on stdout; the device banner and the tables go to
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
MALL_BYTES = 256 << 20  # MI355X Infinity Cache: footprints below it are cache resident
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
    log("host: %d cores available to this process (nproc %s)" % (host_cores(), os.cpu_count()))
    return arch


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


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


def _warm(fn, seconds=0.03, at_least=2):
    """Runs fn (synchronising) until `seconds` have passed, at least
    `at_least` times: the device leaves its idle clocks before anything is
    timed."""
    import torch
    t0, n = time.perf_counter(), 0
    while n < at_least or time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()
        n += 1


def _time(fn, stream, reps=5, warm=True):
    """Mean ms of fn over `reps` back-to-back calls between one event pair."""
    import torch
    if warm:
        _warm(fn)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


class Resident:
    """One workload's inputs resident in HBM, its partition array and its
    outputs, with the two launches of a step."""

    def __init__(self, om, torch, w, arrs, dev, stream):
        def to_dev(x):
            return torch.from_numpy(x.view(np.int32) if x.dtype == np.uint32 else x).to(dev)

        self.om, self.w, self.stream = om, w, stream
        self.d = [to_dev(x) for x in arrs]
        self.seg_len = om.segment_length(w.m, w.n, kv=w.kv)
        self.count = om.partition_count(w.total, self.seg_len)
        self.part = torch.empty(self.count, dtype=torch.int64, device=dev)
        self.out = torch.empty(w.total, dtype=torch.int32, device=dev)
        self.out_v = torch.empty(w.total, dtype=torch.int32, device=dev) if w.kv else None

    def partition(self):
        d = self.d
        self.om.partition(d[0], d[2] if self.w.kv else d[1], self.seg_len, out=self.part,
                          stream=self.stream)

    def merge(self):
        d = self.d
        if self.w.kv:
            self.om.merge_segments_kv(d[0], d[1], d[2], d[3], self.part, self.seg_len,
                                      out_keys=self.out, out_vals=self.out_v, stream=self.stream)
        else:
            self.om.merge_segments_i32(d[0], d[1], self.part, self.seg_len, out=self.out,
                                       stream=self.stream)

    def step(self):
        self.partition()
        self.merge()

    def one_call(self):
        d = self.d
        if self.w.kv:
            self.om.merge_kv(d[0], d[1], d[2], d[3], out_keys=self.out, out_vals=self.out_v,
                             stream=self.stream)
        else:
            self.om.merge_i32(d[0], d[1], out=self.out, stream=self.stream)

    def matches(self, want) -> bool:
        import torch
        torch.cuda.synchronize()
        if self.w.kv:
            return (np.array_equal(self.out.cpu().numpy(), want[0]) and
                    np.array_equal(self.out_v.cpu().numpy().view(np.uint32), want[1]))
        return np.array_equal(self.out.cpu().numpy(), want)

    def timed_steps(self, steps):
        """Exactly `steps` steps back to back between device synchronisations:
        (event ms per step, host-clock ms per step)."""
        import torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        e0.record(self.stream)
        for _ in range(steps):
            self.step()
        e1.record(self.stream)
        torch.cuda.synchronize()
        t = time.perf_counter() - t
        return e0.elapsed_time(e1) / steps, t * 1e3 / steps

    def graph_step_ms(self, want, per_graph=20, replays=10):
        """ms per step with `per_graph` steps captured in one HIP graph and
        the graph replayed `replays` times on the same stream: the device's
        time for a step without the host's per-launch costs.  The steps'
        launches allocate nothing; the first replay's output is checked
        against the oracle before anything is timed (None if it differs)."""
        import torch
        g = torch.cuda.CUDAGraph()
        keep, self.stream = self.stream, None  # launch on torch's capture stream
        try:
            with torch.cuda.graph(g):
                for _ in range(per_graph):
                    self.step()
        finally:
            self.stream = keep
        self.out.fill_(-1)
        with torch.cuda.stream(self.stream):
            g.replay()
        if not self.matches(want):
            return None

        def replay():
            with torch.cuda.stream(self.stream):
                g.replay()
        _warm(replay, seconds=0.03)
        ms = _time(replay, self.stream, reps=replays, warm=False) / per_graph
        del g
        return ms

    def kernel_times(self, steps):
        """`steps` steps with an event before the partition, between the two
        launches and after the merge: per-launch ms of each kernel."""
        import torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            ev[k][0].record(self.stream)
            self.partition()
            ev[k][1].record(self.stream)
            self.merge()
            ev[k][2].record(self.stream)
        torch.cuda.synchronize()
        part = [e[0].elapsed_time(e[1]) for e in ev]
        merge = [e[1].elapsed_time(e[2]) for e in ev]
        return part, merge


def copy_references(om, torch, nbytes, dev, stream, reps=10):
    """ms of the library's streaming copy kernel and of a device-to-device
    hipMemcpyAsync (torch copy_ of contiguous same-dtype tensors), each over
    `nbytes` bytes read and as many written."""
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    src.random_(0, 1 << 30)
    dst = torch.empty_like(src)
    copy_ms = _time(lambda: om.stream_copy(src, out=dst, stream=stream), stream, reps=reps)
    if not torch.equal(src, dst):
        log("FAILED: the streaming copy kernel's output differs from its input")
        sys.exit(1)
    dst.zero_()
    with torch.cuda.stream(stream):
        memcpy_ms = _time(lambda: dst.copy_(src), stream, reps=reps)
    if not torch.equal(src, dst):
        log("FAILED: the device-to-device copy's output differs from its input")
        sys.exit(1)
    del src, dst
    return copy_ms, memcpy_ms


def workload_row(om, torch, name, dev, stream, warmup, steps):
    """One workload: generated, merged by the oracle, checked on every
    element, then timed (at least `warmup` untimed steps and 50 ms, then at
    least `steps` timed steps and 20 ms).  Returns the row as a dict."""
    from ordered_merge_sorted_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    arrs = w.make()
    want, _ = run_oracle(w, arrs)
    r = Resident(om, torch, w, arrs, dev, stream)
    r.out.fill_(-1)
    r.step()
    if not r.matches(want):
        log("FAILED: workload %s: the merged output differs from the oracle" % name)
        sys.exit(1)
    graph_ms = r.graph_step_ms(want)
    if graph_ms is None:
        log("FAILED: workload %s: a graph replay's output differs from the oracle" % name)
        sys.exit(1)
    del want
    _warm(r.step, seconds=0.05, at_least=max(warmup, 2))
    one_ms = r.timed_steps(1)[0]
    reps = max(steps, int(20.0 / max(one_ms, 1e-3)) + 1)
    ms, _ = r.timed_steps(reps)
    part, merge = r.kernel_times(reps)
    one_call_ms = _time(r.one_call, stream, reps=reps)
    alg = w.roofline_bytes
    # a copy of a cache-resident row's few bytes times launches, not
    # bandwidth: no copy reference for those rows
    copy_ms = None
    if alg > MALL_BYTES:
        copy_ms = copy_references(om, torch, alg // 2, dev, stream)[0]
    gbs = alg / (ms * 1e-3) / 1e9
    row = {"step_ms": ms, "steps": reps,
           "elements_per_s": w.total / (ms * 1e-3),
           "gbps": gbs, "pct_peak": 100 * gbs / HBM_PEAK_GBS,
           "pct_copy": None if copy_ms is None else 100 * copy_ms / ms,
           "merge_kernel_ms": float(np.mean(merge)),
           "partition_kernel_ms": float(np.mean(part)),
           "graph_step_ms": graph_ms,
           "one_call_ms": one_call_ms,
           "graph_pct_peak": 100 * alg / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "cache_resident": alg <= MALL_BYTES,
           "checked": "bit-exact vs oracle"}
    del r
    torch.cuda.empty_cache()
    return row


def ablation(om, torch, name, dev, stream, arrs=None, want=None):
    """The pages' global-memory merge kernels (no LDS) beside the LDS-tiled
    step, on one workload: one co-rank search then a walk, or two searches
    per slice, at 1, 4, 16, 64 and 256 outputs per lane.  Every variant is
    checked against the oracle on every element before it is timed.
    Launch order (the profiles' tables rely on it): for each of the ten
    variants one checked launch then `reps` timed ones; then the LDS-tiled
    step (partition + segment merge) once checked, warmed for 30 ms, and
    `reps` times timed."""
    from ordered_merge_sorted_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    if arrs is None:
        arrs = w.make()
    if want is None:
        want = run_oracle(w, arrs)[0]
    r = Resident(om, torch, w, arrs, dev, stream)
    d_a, d_b = r.d[0], r.d[1]
    reps = 5
    log("ablation on %s: the pages' global-memory merge kernels (no LDS), %d timed launches "
        "each after one checked launch" % (name, reps))
    log("%-34s %10s %10s %8s" % ("kernel", "ms", "GB/s", "% peak"))
    for two in (False, True):
        for per in (1, 4, 16, 64, 256):
            def go():
                om.merge_i32_direct(d_a, d_b, per_thread=per, two_searches=two,
                                    out=r.out, stream=stream)
            r.out.fill_(-1)
            go()
            if not r.matches(want):
                log("FAILED: direct kernel per=%d two_searches=%s differs from the oracle" % (per, two))
                sys.exit(1)
            ms = _time(go, stream, reps=reps, warm=False)
            gbs = w.roofline_bytes / (ms * 1e-3) / 1e9
            log("%-34s %10.3f %10.1f %8.1f" % ("%s, %d per lane" % ("two searches" if two else "search+walk", per),
                                                ms, gbs, 100 * gbs / HBM_PEAK_GBS))
    r.out.fill_(-1)
    r.step()
    if not r.matches(want):
        log("FAILED: the LDS-tiled step differs from the oracle")
        sys.exit(1)
    # (warmed first: after the global-memory kernels' seconds of sparse
    # traffic the device needs a few steps to reach its streaming rate)
    ms = _time(r.step, stream, reps=reps)
    gbs = w.roofline_bytes / (ms * 1e-3) / 1e9
    log("%-34s %10.3f %10.1f %8.1f" % ("LDS-tiled step (partition + merge)", ms, gbs,
                                        100 * gbs / HBM_PEAK_GBS))
    del r
    torch.cuda.empty_cache()


def typed_orders(om, torch, d_arrs, c_ref, w, stream):
    """The key orders of omerge_merge_keys on inputs derived from the int32
    workload on the device: uint32 keys x ^ 2^31, float32 keys with bits
    (x ^ 2^31) >> 1 (non-negative patterns, so bit order is totalOrder; some
    are infinities and NaNs), int64 keys x * 2^32 and float64 keys with bits
    (x ^ 2^31 as uint32) << 31, each ascending and reversed for descending.
    Each output is checked against the same map of the int32 merge output
    (keys only: the sorted multiset is unique) before it is timed."""
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
            ms = _time(go, stream, reps=20)
            gbs = 2 * w.total * out.element_size() / (ms * 1e-3) / 1e9
            log("%-28s %10.3f %10.1f %8.1f" % (name + (" descending" if desc else " ascending"),
                                                ms, gbs, 100 * gbs / HBM_PEAK_GBS))
            del a, b, out, want


def sort_and_batch(om, torch, stream):
    """The merge sort and the batched merge on 2^28 int32 keys (and 2^27
    key+payload pairs), each checked against torch's stable sort before it
    is timed; torch.sort is timed beside it for context."""
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
    # one 4-way pass against one 2-way pass (a batch of merges of adjacent
    # runs) over the same keys in sorted runs of 2^20: the 4-way pass does
    # two doublings of the run length, the 2-way pass one
    run = 1 << 20
    runs = torch.sort(keys.view(-1, run), dim=1).values.reshape(-1)
    o4 = torch.empty_like(runs)
    om.merge_runs4(runs, run, out=o4, stream=stream)
    torch.cuda.synchronize()
    if not torch.equal(o4.view(-1, 4 * run), torch.sort(runs.view(-1, 4 * run), dim=1).values):
        log("FAILED: omerge 4-way pass differs from torch's per-group sort")
        sys.exit(1)
    ms4 = _time(lambda: om.merge_runs4(runs, run, out=o4, stream=stream), stream)
    half = runs.view(-1, 2, run)
    a2, b2 = half[:, 0].reshape(-1).contiguous(), half[:, 1].reshape(-1).contiguous()
    offs = torch.arange(0, a2.numel() + 1, run, dtype=torch.int64, device=dev)
    ms2 = _time(lambda: om.merge_batched(a2, offs, b2, offs, out=o4, stream=stream), stream)
    for label, ms_p in (("4-way pass (merge_runs4), runs of 2^20", ms4),
                        ("2-way pass (batched), runs of 2^20", ms2)):
        gbs = 2 * n * 4 / (ms_p * 1e-3) / 1e9
        log("%-44s %10.3f %14.4g  (%.0f GB/s, %.1f%% of peak)" % (
            label, ms_p, n / (ms_p * 1e-3), gbs, 100 * gbs / HBM_PEAK_GBS))
    del runs, o4, half, a2, b2, offs
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
    for pairs, L, label in ((1 << 15, 4096, "batched: 2^15 merges of 4096+4096"),
                            (1 << 22, 16, "batched: 2^22 merges of 16+16")):
        a = torch.sort(keys[:pairs * L].view(pairs, L), dim=1).values.reshape(-1)
        b = torch.sort(keys[pairs * L:2 * pairs * L].view(pairs, L), dim=1).values.reshape(-1)
        offs = torch.arange(0, pairs * L + 1, L, dtype=torch.int64, device=dev)
        c = torch.empty(2 * pairs * L, dtype=torch.int32, device=dev)
        om.merge_batched(a, offs, b, offs, out=c, stream=stream)
        ref = torch.sort(torch.cat([a.view(pairs, L), b.view(pairs, L)], dim=1), dim=1).values
        torch.cuda.synchronize()
        if not torch.equal(c.view(pairs, 2 * L), ref):
            log("FAILED: omerge batched merge (%s) differs from torch's per-merge sort" % label)
            sys.exit(1)
        ms = _time(lambda: om.merge_batched(a, offs, b, offs, out=c, stream=stream), stream)
        gbs = 2 * c.numel() * 4 / (ms * 1e-3) / 1e9
        log("%-44s %10.3f %14.4g  (%.0f GB/s, %.1f%% of peak)" % (
            label, ms, c.numel() / (ms * 1e-3), gbs, 100 * gbs / HBM_PEAK_GBS))
        del a, b, offs, c, ref


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None, help="workload name (default: the int32 2^28+2^28 merge)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the extra oracle runs of the CPU baseline (the output checks "
                         "still run)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the rows of the other workloads (e.g. under a profiler)")
    ap.add_argument("--ablation", action="store_true",
                    help="also time the global-memory (no LDS) merge kernels at 1..256 outputs "
                         "per lane on the headline and even/odd workloads, each checked against "
                         "the oracle, every key order of omerge_merge_keys, the merge sort and "
                         "the batched merge; tables on stderr")
    ap.add_argument("--ablation-direct", action="store_true",
                    help="only the global-memory kernels' tables of --ablation (headline and "
                         "even/odd workloads), e.g. under a profiler")
    ap.add_argument("--ablation-sort", action="store_true",
                    help="only the merge sort, 4-way pass and batched merge rows of --ablation, "
                         "each checked first (tables on stderr, no JSON line), e.g. under a "
                         "profiler")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    import torch

    import ordered_merge_sorted_amd as om
    from ordered_merge_sorted_amd.workloads import HEADLINE, ORDER, WORKLOADS

    name = args.workload or HEADLINE
    if name not in WORKLOADS:
        ap.error("unknown workload %s (one of %s)" % (name, ", ".join(ORDER)))
    w = WORKLOADS[name]
    arch = device_banner(torch)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.ablation_sort:
        sort_and_batch(om, torch, stream)
        return

    # 1. Inputs and the oracle's reference, before anything runs on the device.
    t0 = time.perf_counter()
    arrs = w.make()
    log("workload %s: m=%d n=%d (%s); generated in %.1f s" % (name, w.m, w.n, w.description,
                                                             time.perf_counter() - t0))
    want, oracle_s = run_oracle(w, arrs)
    log("oracle reference: %.2f s on one host core" % oracle_s)

    # 2. Resident inputs; one untimed step checked on every element.
    r = Resident(om, torch, w, arrs, dev, stream)
    r.out.fill_(-1)
    r.step()
    if not r.matches(want):
        log("FAILED: the merged output differs from the oracle; no number is reported")
        sys.exit(1)
    log("checked: output bit-exact against the oracle (%d elements)" % w.total)
    # The same step replayed from a HIP graph, checked first (reported on
    # stderr; before the references below, which keep the device busy up to
    # the timed steps).
    graph_ms = r.graph_step_ms(want)
    if graph_ms is None:
        log("FAILED: a graph replay's output differs from the oracle; no number is reported")
        sys.exit(1)
    if (args.ablation or args.ablation_direct) and not w.kv:
        ablation(om, torch, name, dev, stream, arrs, want)
        if name != "even_odd_2p21":
            ablation(om, torch, "even_odd_2p21", dev, stream)
    if args.ablation and not w.kv:
        typed_orders(om, torch, r.d, r.out, w, stream)

    # 3. Bandwidth references and the one-call API over the same bytes; they
    # run right before the warm-up, so the device is busy from here on.
    alg_bytes = w.roofline_bytes  # each element read once and written once
    copy_ms, memcpy_ms = copy_references(om, torch, alg_bytes // 2, dev, stream)
    onecall_ms = _time(r.one_call, stream, reps=10)

    # 4. Exactly W untimed steps, then exactly K timed steps (the step rate).
    for _ in range(args.warmup):
        r.step()
    ms_step, host_ms = r.timed_steps(args.steps)

    # 5. The same K steps with an event pair around each kernel.
    part_ms, merge_ms = r.kernel_times(args.steps)
    merge_ms_mean = float(np.mean(merge_ms))
    part_ms_mean = float(np.mean(part_ms))

    # 6. The last timed step's output against the oracle.
    if not r.matches(want):
        log("FAILED: the output of the timed steps differs from the oracle; no number is reported")
        sys.exit(1)
    del want

    value = w.total / (ms_step * 1e-3)
    step_gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    kern_gbs = alg_bytes / (merge_ms_mean * 1e-3) / 1e9
    copy_gbs = alg_bytes / (copy_ms * 1e-3) / 1e9
    memcpy_gbs = alg_bytes / (memcpy_ms * 1e-3) / 1e9
    log("step: %.4f ms (host clock %.4f ms/step) -> %.4g elements/s, %.1f GB/s (%.1f%% of %.0f)" % (
        ms_step, host_ms, value, step_gbs, 100 * step_gbs / HBM_PEAK_GBS, HBM_PEAK_GBS))
    log("segment merge kernel: %.4f ms mean (min %.4f, max %.4f) -> %.1f GB/s (%.1f%% of peak)" % (
        merge_ms_mean, min(merge_ms), max(merge_ms), kern_gbs, 100 * kern_gbs / HBM_PEAK_GBS))
    log("partition kernel: %.4f ms mean (min %.4f, max %.4f); step - merge kernel: %.4f ms" % (
        part_ms_mean, min(part_ms), max(part_ms), ms_step - merge_ms_mean))
    log("the step replayed from a HIP graph (20 steps per graph): %.4f ms" % graph_ms)
    log("streaming copy kernel, same bytes: %.4f ms -> %.1f GB/s; step at %.1f%% of it" % (
        copy_ms, copy_gbs, 100 * copy_ms / ms_step))
    log("hipMemcpyAsync device to device, same bytes: %.4f ms -> %.1f GB/s" % (memcpy_ms, memcpy_gbs))
    log("%s one call (with its scratch allocation): %.4f ms" % (
        "merge_kv" if w.kv else "merge_i32", onecall_ms))
    seg_len, count = r.seg_len, r.count
    del r
    torch.cuda.empty_cache()

    # 7. The other workloads, one row each.
    rows = {}
    if not args.headline_only:
        log("%-24s %9s %11s %9s %7s %7s %9s %9s %9s %9s  %s" % (
            "workload", "step ms", "elements/s", "GB/s", "% peak", "% copy", "merge ms",
            "part. ms", "graph ms", "1 call ms", "note"))
        for other in ORDER:
            if other == name:
                continue
            row = workload_row(om, torch, other, dev, stream, args.warmup, args.steps)
            rows[other] = row
            log("%-24s %9.4f %11.4g %9.1f %7.1f %7s %9.4f %9.4f %9.4f %9.4f  %s" % (
                other, row["step_ms"], row["elements_per_s"], row["gbps"], row["pct_peak"],
                "n/a" if row["pct_copy"] is None else "%.1f" % row["pct_copy"],
                row["merge_kernel_ms"], row["partition_kernel_ms"],
                row["graph_step_ms"], row["one_call_ms"],
                "cache resident (%.0f MB moved)" % (WORKLOADS[other].roofline_bytes / 1e6)
                if row["cache_resident"] else "checked bit-exact"))
    if args.ablation and not w.kv:
        sort_and_batch(om, torch, stream)

    # 8. The CPU baseline: more runs of the oracle on the headline workload.
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
        "memcpy_d2d_gbps_same_bytes": memcpy_gbs,
        "partition_kernel_ms": part_ms_mean,
        "one_call_ms": onecall_ms,
        "roofline": {"bound": "hbm", "achieved": kern_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kern_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "merge_segments_kernel", "kernel_ms": merge_ms_mean,
                     "scope": "segment merge kernel alone; the whole step is pct_hbm_peak",
                     "step_frac": step_gbs / HBM_PEAK_GBS,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
        "workloads": rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
