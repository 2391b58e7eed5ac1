#!/usr/bin/env python3
"""Throughput of the fixed-order fold on one MI355X.

Headline workload: fold_ranks over a stacked [8][16777216] float32 arena
(64 MiB per slot), slot r = vecf(2^24, 1000 + r), into a separate output.
One step is one fold_ranks call; it moves (W+1)*len*4 = 603,979,776 bytes
(W slots read, one output written).  The inputs are resident in HBM before
the timed region starts.  Each step folds the next of 3 copies of the arena
into the next of 8 outputs (1 GiB of other arena copies between two reads of
one copy, 512 MiB of outputs: four and two times the memory-side cache), so
that no step finds its operands in that cache; the line's cache_controls
give the rates with one arena and with every operand reused, interleaved.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

prints one JSON line: metric, value (GB/s of algorithmic bytes), the roofline
of the fold kernel (nominal and against the streaming ceiling measured on the
same box), single launches after a cache scrub (event pair around the call and
the kernel's own duration), the CPU oracle timed on the host as a reported
baseline, the 16 KiB in-place fold latency, and two secondary fold workloads
in the same line: W=4 x 1e8 mixed magnitudes scaled by 1/4, and W=16 x
10,000,019 at base+1 element, whole and as 16 owner shards (each bit-checked
against the oracle).  Other modes (not the headline):

    --workload {w8,w4,w16,w32}    other fold configurations, same JSON shape
    --workload {join,round,pair,procs}
                                  the in-place fold's latency, the one-GPU
                                  round, two ranks on two streams, and ranks
                                  as processes sharing device memory
    --sweep                       launch-geometry sweep of the headline fold
    --copy-calibration            a plain device copy of known size, for
                                  scaling rocprofv3 FETCH_SIZE / WRITE_SIZE
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD public specification
MEMORY_SIDE_CACHE_BYTES = 256 << 20  # MI355X's last-level cache on the memory side of the fabric
METRIC = "fold GB/s (W+1 bufs moved) and % HBM peak at W=8, 64 MiB/slot; 16 KiB latency"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fold_w8_64mib_hbm_counters.md")
LIB_SOURCES = sorted(glob.glob(os.path.join(ROOT, "deterministic_fixed_order_amd", "csrc", "*.hip")) +
                     glob.glob(os.path.join(ROOT, "deterministic_fixed_order_amd", "csrc", "*.cpp")) +
                     glob.glob(os.path.join(ROOT, "deterministic_fixed_order_amd", "csrc", "*.h"))) + \
    [os.path.join(ROOT, "include", "detfold.h")]

WORKLOADS = {
    # name: (family, W, len, seed0, scaled inv_w or None, base offset in elements)
    "w8": ("vecf", 8, 1 << 24, 1000, None, 0),
    "w4": ("mixed", 4, 100_000_000, 2000, 0.25, 0),
    "w16": ("vecf", 16, 10_000_019, 3000, None, 1),
    "w32": ("vecf", 32, 8_000_001, 4000, None, 1),
}
WORKLOAD_NAMES = {
    "w8": "fold_ranks W=8 stacked [8][16777216] f32 (64 MiB/slot), uniform [-1,1)",
    "w4": "fold_ranks_scaled W=4 stacked [4][100000000] f32, mixed magnitudes, inv_w=0.25",
    "w16": "fold_ranks W=16 stacked [16][10000019] f32 at base+1 element, uniform [-1,1)",
    "w32": "fold_ranks W=32 stacked [32][8000001] f32 at base+1 element, uniform [-1,1)",
    "join": "fold_into n=4096 f32 (16 KiB per buffer)",
    "round": "loopback_round W=8 arenas of 16777216 f32 (64 MiB each): staged, direct and fused",
    "pair": "two-stream pair all-reduce at the decode-join sizes",
    "procs": "ranks as processes: W=4 arenas of 16777216 f32 shared by device memory handles; "
             "one-shot ranks at n=4096",
}


def code_text(src: str) -> str:
    """The C++ source with comments removed and whitespace runs collapsed, so
    that the hash below changes with the code, not with its commentary.
    String and character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """sha256[:16] of the library's code: every source under csrc/ and the public
    header, each by file name, comments and layout excluded."""
    h = hashlib.sha256()
    for path in LIB_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode() + b"\n" + code_text(f.read()).encode() + b"\n")
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_counters():
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        text = open(COUNTERS_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec


class Timer:
    """HIP events on the stream the fold is launched on (timing enabled)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def region(self, fn, reps: int) -> float:
        torch = self.torch
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(self.stream)
        for _ in range(reps):
            fn()
        end.record(self.stream)
        end.synchronize()
        torch.cuda.synchronize()
        return start.elapsed_time(end)  # ms


def make_workload(name, torch, dev, want_host=False):
    import numpy as np
    import fold_inputs

    family, W, n, seed0, inv_w, offset = WORKLOADS[name]
    host = fold_inputs.slots(family, W, n, seed0)
    alloc = torch.empty(W * n + offset, dtype=torch.float32, device=dev)
    stacked = alloc[offset:].view(W, n)
    stacked.copy_(torch.from_numpy(host))
    out = torch.empty(n, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    return host, stacked, out, W, n, inv_w


def output_set(torch, out):
    """`out` and more buffers like it, together at least twice the memory-side
    cache.  A timed region writes each step into the next of them in turn, so
    no line an earlier step wrote can still sit in that cache when a step
    writes it, and every step's stores reach HBM.  Folded into one output
    back to back, the cache takes part of each step's writes: with the
    stores written through, W=8 x 2^24 ran at 7,050-7,072 GB/s into one or
    two outputs, 6,922 into four (256 MiB) and 6,668 into eight."""
    count = max(2, -(-2 * MEMORY_SIDE_CACHE_BYTES // (out.numel() * 4)))
    return [out] + [torch.empty_like(out) for _ in range(count - 1)]


def arena_set(torch, stacked, offset):
    """`stacked` and copies of it, each in an allocation of its own at the same
    element offset (so every copy keeps the arena's 16-byte phases), enough of
    them that at least 1 GiB of the other copies -- four times the
    memory-side cache -- is read between two reads of any one copy.  A
    timed region folds the copies in turn, so no step's slots can still sit
    in that cache from an earlier step.  Folding one arena over and over, the
    cache fed 1.1-1.7% of the W=8 x 2^24 rate and 1.3-1.4% at W=16 x
    10,000,019; nothing at W=4 x 1e8, whose arena is six times the cache."""
    W, n = stacked.shape
    count = 1 + max(1, -(-4 * MEMORY_SIDE_CACHE_BYTES // (W * n * 4)))
    copies = [stacked]
    for _ in range(count - 1):
        alloc = torch.empty(W * n + offset, dtype=stacked.dtype, device=stacked.device)
        copy = alloc[offset:].view(W, n)
        copy.copy_(stacked)
        copies.append(copy)
    return copies


def fold_call(df, inv_w):
    """call(out, stacked): one fold_ranks (or fold_ranks_scaled) on the current stream."""
    if inv_w is None:
        return lambda o, s: df.fold_ranks(o, s)
    return lambda o, s: df.fold_ranks_scaled(o, s, inv_w)


def fold_step(df, outs, arenas, inv_w):
    """One fold per call: call i folds arenas[i % A] into outs[i % R]."""
    call = fold_call(df, inv_w)
    state = [0]

    def step():
        i = state[0]
        state[0] += 1
        call(outs[i % len(outs)], arenas[i % len(arenas)])
    return step


def fill_outputs(torch, df, outs, arenas, inv_w):
    """Output k := the fold of arena copy k mod A, then wait: with at least as
    many outputs as copies, the bit checks of the outputs cover every copy."""
    call = fold_call(df, inv_w)
    for k, o in enumerate(outs):
        call(o, arenas[k % len(arenas)])
    torch.cuda.synchronize()


def all_equal(torch, outs, ref):
    return all(bool(torch.equal(o.view(torch.int32), ref.view(torch.int32))) for o in outs)


def timing_events(torch, stream, count):
    """`count` (start, stop) pairs of timing-enabled events, each recorded once
    so that its device event exists before a dispatch records it."""
    pairs = []
    for _ in range(count):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return pairs


def kernel_only_ms(torch, df, stream, outs, arenas, inv_w, calls):
    """Durations (ms) of `calls` back-to-back fold kernels, each timed by
    events its own dispatch records (detfold_fold_ranks_timed), call i
    folding arenas[i % A] into outs[i % R] as the timed steps do."""
    pairs = timing_events(torch, stream, calls)
    for i, (a, b) in enumerate(pairs):
        df.fold_ranks_timed(outs[i % len(outs)], arenas[i % len(arenas)], a, b,
                            scaled=inv_w is not None, inv_w=inv_w if inv_w is not None else 1.0)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def oracle_check(host, inv_w, outs):
    """The first output against the CPU oracle bit for bit, and every other
    output of the rotation against the first."""
    import numpy as np
    import oracle
    import torch
    want = oracle.fold_stacked(host) if inv_w is None else \
        oracle.fold_stacked_scaled(host, np.float32(inv_w))
    got = outs[0].cpu().numpy()
    return bool(np.array_equal(got.view(np.uint32), want.view(np.uint32))) and \
        all_equal(torch, outs[1:], outs[0])


def traffic_for(name):
    """HBM bytes per launch of workload `name` from the committed counter
    record, if it was taken on the current library code; else None."""
    counters = read_counters()
    if not counters:
        return None
    if name == "w8":
        return counters.get("hbm_bytes_per_launch")
    return counters.get("other_workloads", {}).get(name, {}).get("hbm_bytes_per_launch")


def roofline(gbs, ms, bytes_per_step, kernel, traffic, kernel_ms=None, attainable=None):
    r = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
         "algorithmic_bytes_per_launch": bytes_per_step, "avg_launch_ms": round(ms, 6)}
    if traffic:
        r["traffic_over_algorithmic"] = round(traffic / bytes_per_step, 4)
    if kernel_ms is not None:
        r["kernel_only_avg_ms"] = round(kernel_ms, 6)
    if attainable:
        r["attainable_GBps"] = attainable
        r["frac_of_attainable"] = round(gbs / attainable, 4)
    return r


def bench_fold(args, torch, df, dev):
    name = args.workload
    host, stacked, out, W, n, inv_w = make_workload(name, torch, dev)
    bytes_per_step = (W + 1) * n * 4
    stream = torch.cuda.current_stream(dev)
    timer = Timer(torch, stream)
    arenas = arena_set(torch, stacked, WORKLOADS[name][5])
    outs = output_set(torch, out)
    step = fold_step(df, outs, arenas, inv_w)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done (%d steps); timing %d steps of %s, folding %d copies of the arena in turn, "
        "each into the next of %d outputs" % (args.warmup, args.steps, name, len(arenas), len(outs)))
    ms_total = timer.region(step, args.steps)
    ms_per_step = ms_total / args.steps
    gbs = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    log("timed region: %.3f ms per step, %.1f GB/s" % (ms_per_step, gbs))
    kern = kernel_only_ms(torch, df, stream, outs, arenas, inv_w, args.steps)
    kern_avg = statistics.mean(kern)
    log("kernel-only (dispatch-recorded events), %d back-to-back launches: average %.4f ms, "
        "median %.4f ms" % (len(kern), kern_avg, statistics.median(kern)))
    sustained = bench_sustained(args, timer, step, bytes_per_step)
    controls = bench_cache_controls(args, df, timer, outs, arenas, inv_w, bytes_per_step) \
        if args.controls else None
    fill_outputs(torch, df, outs, arenas, inv_w)

    singles = bench_singles(args, torch, df, dev, timer, out, stacked, inv_w, bytes_per_step) \
        if args.singles > 0 else None
    ceiling = bench_ceiling(args, torch, dev, timer, arenas, outs) if args.ceiling else None
    attainable = ceiling["attainable_GBps"] if ceiling else None

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded xorshift64 generators, resident in HBM)",
        "config": {"workload": WORKLOAD_NAMES[name], "W": W, "len": n,
                   "bytes_per_step": bytes_per_step, "parallelism": "single GPU",
                   "arena_copies_rotated": len(arenas), "outputs_rotated": len(outs)},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "sustained": sustained,
        "cache_controls": controls,
    }
    result["roofline"] = roofline(gbs, ms_per_step, bytes_per_step,
                                  kernel_name(df, torch, dev, out, stacked, W, n, inv_w is not None),
                                  traffic_for(name), kern_avg, attainable)
    if singles:
        result["scrubbed_single_launch"] = singles
    if ceiling:
        result["streaming_ceiling"] = ceiling
    result["device"] = device_info(torch, dev)
    if args.workload == "w8" and not args.no_latency:
        result["latency_16KiB"] = bench_join(args, torch, df, dev, timer)
    if args.workload == "w16" and args.owner_shards:
        result["owner_shards"] = bench_owner_shards(args, torch, df, timer, arenas, out, W, n)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, host, inv_w, outs, W, n, bytes_per_step)
    else:
        result["bit_exact_vs_oracle"] = oracle_check(host, inv_w, outs)
    if args.workload == "w8" and args.secondary:
        del host, stacked, out, outs, arenas, step
        torch.cuda.empty_cache()
        result["secondary"] = {w: bench_secondary(args, torch, df, dev, w) for w in ("w4", "w16")}
    return result


def bench_secondary(args, torch, df, dev, name):
    """Another fold workload in the same run: back-to-back throughput, the
    kernel's own duration, the roofline against the nominal peak, the HBM
    traffic record, and the whole output checked against the CPU oracle bit
    for bit; for the W=16 arena also its 16 owner shards."""
    host, stacked, out, W, n, inv_w = make_workload(name, torch, dev)
    bytes_per_step = (W + 1) * n * 4
    stream = torch.cuda.current_stream(dev)
    timer = Timer(torch, stream)
    arenas = arena_set(torch, stacked, WORKLOADS[name][5])
    outs = output_set(torch, out)
    step = fold_step(df, outs, arenas, inv_w)
    settle(timer, step)
    for _ in range(args.warmup):
        step()
    ms = timer.region(step, args.steps) / args.steps
    gbs = bytes_per_step / (ms * 1e-3) / 1e9
    kern = kernel_only_ms(torch, df, stream, outs, arenas, inv_w, args.steps)
    sustained = bench_sustained(args, timer, step, bytes_per_step)
    controls = bench_cache_controls(args, df, timer, outs, arenas, inv_w, bytes_per_step) \
        if args.controls else None
    fill_outputs(torch, df, outs, arenas, inv_w)
    exact = oracle_check(host, inv_w, outs)
    log("%s: %.4f ms per step, %.1f GB/s (%.1f%% of peak); kernel-only average %.4f ms; bit-exact vs "
        "the oracle: %s" % (name, ms, gbs, 100 * gbs / HBM_PEAK_GBS, statistics.mean(kern), exact))
    if not exact:
        raise RuntimeError("%s: the GPU fold differs from the oracle" % name)
    res = {"workload": WORKLOAD_NAMES[name], "W": W, "len": n, "bytes_per_step": bytes_per_step,
           "arena_copies_rotated": len(arenas), "outputs_rotated": len(outs), "steps": args.steps,
           "ms_per_step": round(ms, 6), "GBps": round(gbs, 2), "sustained": sustained,
           "cache_controls": controls,
           "kernel_only_median_ms": round(statistics.median(kern), 6),
           "roofline": roofline(gbs, ms, bytes_per_step,
                                kernel_name(df, torch, dev, out, stacked, W, n, inv_w is not None),
                                traffic_for(name), statistics.mean(kern)),
           "bit_exact_vs_oracle": exact}
    if name == "w16" and args.owner_shards:
        res["owner_shards"] = bench_owner_shards(args, torch, df, timer, arenas, out, W, n)
    del host, stacked, out, outs, arenas
    torch.cuda.empty_cache()
    return res


def bench_sustained(args, timer, step, bytes_per_step):
    """The headline's step over one long region right after the headline's
    (--sustained-steps, about 0.2 s at W=8): the rate under continuous load,
    which the device's power and thermal management can hold below that of a
    short region after a pause."""
    if args.sustained_steps <= 0:
        return None
    ms = timer.region(step, args.sustained_steps) / args.sustained_steps
    gbs = bytes_per_step / (ms * 1e-3) / 1e9
    log("sustained, %d steps: %.4f ms per step, %.1f GB/s" % (args.sustained_steps, ms, gbs))
    return {"steps": args.sustained_steps, "ms_per_step": round(ms, 6), "GBps": round(gbs, 2),
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_cache_controls(args, df, timer, outs, arenas, inv_w, bytes_per_step):
    """What the rotation keeps out of the headline: regions of the headline's
    own step (arena copies and outputs in turn) interleaved with regions that
    fold one arena into the rotating outputs, and one arena into one output
    (every operand reused), three regions each, so that all three see the same
    device state (clocks, temperature, what ran before)."""
    call = fold_call(df, inv_w)
    forms = {"rotating": fold_step(df, outs, arenas, inv_w),
             "one_arena": fold_step(df, outs, arenas[:1], inv_w),
             "one_arena_one_output": lambda: call(outs[0], arenas[0])}
    samples = {k: [] for k in forms}
    for _ in range(3):
        for key, fn in forms.items():
            for _ in range(4):
                fn()
            samples[key].append(timer.region(fn, args.steps) / args.steps)
    res = {"regions_each": 3, "steps_per_region": args.steps,
           "note": "interleaved regions; rotating is the headline's step"}
    for key, v in samples.items():
        ms = statistics.median(v)
        res[key] = {"ms_per_step": round(ms, 6), "GBps": round(bytes_per_step / (ms * 1e-3) / 1e9, 2)}
    log("cache controls: rotating %.1f GB/s, one arena %.1f GB/s, one arena into one output %.1f GB/s"
        % (res["rotating"]["GBps"], res["one_arena"]["GBps"], res["one_arena_one_output"]["GBps"]))
    return res

def bench_singles(args, torch, df, dev, timer, out, stacked, inv_w, bytes_per_step):
    """Single launches, each after a 1 GiB scrub (more than four times the
    256 MB memory-side cache, so it holds none of the fold's operands when the
    call starts).  Two scrubs: writing the buffer and then reading it back
    (the cache is left holding clean lines), and writing it only (the cache
    is left holding dirty lines, whose write-back then competes with the
    fold).  A third set has no scrub, only the host synchronization before
    each call, so the device idles between folds: it separates what a launch
    from idle costs from what the scrub leaves behind.  Every call is timed
    twice at once: by an event pair recorded around it on the stream (launch
    and event latency included), and by the start/stop events its own
    dispatch records (the kernel alone)."""
    stream = timer.stream
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    gb = lambda ms: round(bytes_per_step / (ms * 1e-3) / 1e9, 2)
    res = {"calls": args.singles}
    for key, fill, read_back in (("write_then_read_scrub", True, True), ("write_scrub", True, False),
                                 ("no_scrub", False, False)):
        pairs = timing_events(torch, stream, args.singles)
        outer, inner = [], []
        for i, (a, b) in enumerate(pairs):
            if fill:
                scrub.fill_(float(i))
            if read_back:
                scrub.amax()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            df.fold_ranks_timed(out, stacked, a, b, scaled=inv_w is not None,
                                inv_w=inv_w if inv_w is not None else 1.0)
            e1.record(stream)
            e1.synchronize()
            outer.append(e0.elapsed_time(e1))
            inner.append(a.elapsed_time(b))
        med_o, med_i = statistics.median(outer), statistics.median(inner)
        log("single launches, %s: event pair around the call median %.4f ms (%.1f GB/s), "
            "kernel alone median %.4f ms (%.1f GB/s)" % (key.replace("_", " "), med_o, gb(med_o), med_i,
                                                           gb(med_i)))
        res[key] = {"kernel_only_median_ms": round(med_i, 6), "kernel_only_best_ms": round(min(inner), 6),
                    "kernel_only_median_GBps": gb(med_i), "kernel_only_frac": round(gb(med_i) / HBM_PEAK_GBS, 4),
                    "event_pair_median_ms": round(med_o, 6), "event_pair_best_ms": round(min(outer), 6),
                    "event_pair_median_GBps": gb(med_o)}
    del scrub
    torch.cuda.synchronize()
    res["note"] = ("kernel_only: start/stop events recorded by the fold's own dispatch; event_pair: events "
                   "recorded on the stream before and after the call; scrub: 1 GiB filled (and, in the "
                   "first set, then read back with amax) before each call; no_scrub: only the host "
                   "synchronization between calls, the device idle")
    return res


def settle(timer, step, target_ms=100.0):
    """Untimed calls for about target_ms, so that clocks that dropped while
    the device idled (host-side setup, the CPU oracle) are back up before a
    timed region starts.  The queue is drained here: the first launches after
    a drain of a thousand queued calls measured slow (about 40-80 us over a
    20-step region), so the caller's warm-up calls, not its timed region,
    come right after the drain."""
    ms = timer.region(step, 3) / 3
    for _ in range(min(2000, int(target_ms / max(ms, 1e-3)))):
        step()
    timer.torch.cuda.synchronize()


def bench_ceiling(args, torch, dev, timer, arenas, outs):
    """What plain streaming reaches on this machine with library kernels: torch
    reductions over the slot axis of the arena (the fold's byte mix, W reads
    to one write: amax carries no additions, sum other ones), a device copy of
    the whole arena (1:1), a fill of it (writes only) and a sum of it to one
    value (reads only).  Like the fold's steps, call i takes arena copy
    i mod A, a reduction output i mod R (R buffers of the fold's output's size,
    not the fold's own outputs, which the oracle check reads afterwards) and
    scratch buffer i mod 2 (two arena-sized buffers, twice the memory-side
    cache together), so no probe finds its operands in that cache either.  Each rate counts the bytes the operation
    must move, over back-to-back calls timed with events.  attainable_GBps is
    the best of them."""
    W, n = arenas[0].shape
    arena = W * n * 4
    scratch = [torch.empty_like(arenas[0]) for _ in range(2)]
    tmps = [torch.empty_like(o) for o in outs]
    A, R = len(arenas), len(tmps)
    probes = {
        "amax_over_slots": (lambda i: torch.amax(arenas[i % A], dim=0, out=tmps[i % R]), arena + n * 4),
        "sum_over_slots": (lambda i: torch.sum(arenas[i % A], dim=0, out=tmps[i % R]), arena + n * 4),
        "copy_arena": (lambda i: scratch[i % 2].copy_(arenas[i % A]), 2 * arena),
        "fill_arena": (lambda i: scratch[i % 2].fill_(1.0), arena),
        "sum_arena_to_scalar": (lambda i: arenas[i % A].sum(), arena),
    }
    reps = max(6, min(args.steps, 48))
    res = {}
    for key, (fn, moved) in probes.items():
        state = [0]

        def step():
            fn(state[0])
            state[0] += 1
        for _ in range(3):
            step()
        ms = timer.region(step, reps) / reps
        res[key] = {"ms": round(ms, 6), "bytes": moved, "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}
        log("ceiling probe %-20s %.4f ms, %.1f GB/s" % (key, ms, res[key]["GBps"]))
    del scratch, tmps
    torch.cuda.empty_cache()
    best = max(res, key=lambda k: res[k]["GBps"])
    return {"probes": res, "attainable_GBps": res[best]["GBps"], "best_probe": best,
            "note": "library streaming kernels on the headline arena (torch reductions, copy, fill), "
                    "back-to-back, operands rotating as the fold's do, bytes each operation must move"}

def device_info(torch, dev):
    """What the device reports: CU count, peak memory clock and bus width (HIP
    device attributes), and the HBM rate they imply at four transfers per
    reported memory clock (HBM3E signals 8 Gb/s per pin against the 2 GHz
    clock this part reports; MI300X's HBM3 has the same ratio, 5.2 Gb/s per
    pin against 1.3 GHz)."""
    import ctypes
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count, "total_memory_bytes": props.total_memory}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int()
        attrs = {"memory_clock_khz": 60, "memory_bus_width_bits": 59, "core_clock_khz": 5}
        for key, attr in attrs.items():  # hipDeviceAttribute_t values of hip_runtime_api.h
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev.index or 0) == 0:
                info[key] = v.value
        if info.get("memory_clock_khz") and info.get("memory_bus_width_bits"):
            info["hbm_GBps_at_4_transfers_per_clock"] = round(
                4 * info["memory_clock_khz"] * 1e3 * info["memory_bus_width_bits"] / 8 / 1e9, 1)
    except OSError:
        pass
    return info


def bench_owner_shards(args, torch, df, timer, arenas, out, W, n):
    """The owner-shard form of the offset arena: each of the W owners' shards
    is gathered once (untimed, device copies of the W slices) into a [W][l_p]
    scratch; then per step all W shard folds run into one output at the
    owners' offsets, as W separate fold_ranks launches and as one
    fold_ranks_batch launch; and, with no gather, one launch whose jobs read
    the owners' shards in place from the arena (row stride len).  Each must
    equal the whole-arena fold bit for bit.  Same algorithmic bytes as the
    whole fold.  As in the whole fold, the steps take the arena copies (and
    their gathered shards) and the outputs in turn."""
    import torch as _torch
    shards = df.shard_plan(n, W)
    scratch = []  # per arena copy, its W gathered shards
    for a in arenas:
        sc = [_torch.empty((W, l), dtype=_torch.float32, device=out.device) for _, l in shards]
        for (s, l), buf in zip(shards, sc):
            buf.copy_(a[:, s:s + l])
        scratch.append(sc)
    in_place = [[a[:, s:s + l] for s, l in shards] for a in arenas]  # row stride n: no gather
    outs = output_set(_torch, _torch.empty_like(out))
    views = [[o[s:s + l] for s, l in shards] for o in outs]

    def separate(v, src):
        for o, sc in zip(v, src):
            df.fold_ranks(o, sc)

    def one_launch(v, src):
        df.fold_ranks_batch(v, src)
    moved = (W + 1) * n * 4
    res = {"shards": W, "shard_len_max": max(l for _, l in shards), "outputs_rotated": len(outs),
           "arena_copies_rotated": len(arenas),
           "note": "shards gathered once by device copies (untimed); per step every shard fold, "
                   "as separate launches and as one batched launch, from the next arena copy into "
                   "the next output of the rotation"}
    for key, call, srcs in (("separate_launches", separate, scratch), ("one_launch", one_launch, scratch),
                            ("one_launch_shards_read_from_the_arena", one_launch, in_place)):
        for o in outs:
            o.fill_(float("nan"))  # what this variant does not write fails the check below
        state = [0]

        def fn():
            i = state[0]
            state[0] += 1
            call(views[i % len(views)], srcs[i % len(srcs)])
        settle(timer, fn)
        for _ in range(args.warmup):
            fn()
        ms = timer.region(fn, args.steps) / args.steps
        gbs = moved / (ms * 1e-3) / 1e9
        for k, v in enumerate(views):
            call(v, srcs[k % len(srcs)])
        _torch.cuda.synchronize()
        res[key] = {"ms_per_set": round(ms, 5), "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "bits_equal_whole_fold": all_equal(_torch, outs, out)}
    same_sep = res["separate_launches"]["bits_equal_whole_fold"]
    same_one = res["one_launch"]["bits_equal_whole_fold"]
    same_arena = res["one_launch_shards_read_from_the_arena"]["bits_equal_whole_fold"]
    res["one_launch"]["traffic"] = traffic_for("w16_shards_one_launch")
    log("owner shards: %d shard folds of about %d elements: %d launches %.4f ms per set (%.1f GB/s), one "
        "batched launch %.4f ms (%.1f GB/s); bits equal to the whole fold: %s / %s"
        % (W, shards[0][1], W, res["separate_launches"]["ms_per_set"], res["separate_launches"]["GBps"],
           res["one_launch"]["ms_per_set"], res["one_launch"]["GBps"], same_sep, same_one))
    log("owner shards read in place from the arena (row stride n), one launch: %.4f ms (%.1f GB/s); bits "
        "equal: %s" % (res["one_launch_shards_read_from_the_arena"]["ms_per_set"],
                       res["one_launch_shards_read_from_the_arena"]["GBps"], same_arena))
    if not (same_sep and same_one and same_arena):
        raise RuntimeError("the owner-shard folds differ from the whole-arena fold")
    return res

def kernel_name(df, torch, dev, out, stacked, W, n, scaled) -> str:
    """Name of the kernel instance the default launch uses (from the host plan)."""
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    return plan_kernel_name(df, df.plan_fold_ranks(out.data_ptr(), stacked.data_ptr(), W, n, cu), W, scaled)


def plan_kernel_name(df, p, W, scaled) -> str:
    """The kernel instance a host plan names: the row bodies by slots per wave
    (W over the plan's waves, rounded up) and XCD tile group, the wide body by
    its pass shape."""
    if p["path"] == df.PATH_ROWS and W > 16:
        shape = "16,1,4" if p["block"] == 1024 else "8,2,1"  # waves, slots per wave, KiB
        return "k_fold_rows_wide<%s,%s> grid=%d block=%d tile=%d" % (
            shape, str(scaled).lower(), p["grid"], p["block"], p["tile"])
    if p["path"] == df.PATH_ROWS:
        return "k_fold_rows<%d,%d,%s> grid=%d block=%d tile=%d xcd_group=%d" % (
            W, -(-W // (p["block"] // 64)), str(scaled).lower(), p["grid"], p["block"], p["tile"],
            p.get("group", 1))
    body = "k_fold_vector" if p["path"] == df.PATH_VECTOR else "k_fold_scalar"
    ws = W if W in (1, 2, 4, 8, 16) else 0
    pol = 1 if p["policy"] == df.POLICY_STREAM else 0
    return "%s<%d,%d,%s,%d> grid=%d block=%d" % (body, ws, p["unroll"], str(scaled).lower(), pol,
                                                  p["grid"], p["block"])


JOIN_SIZES = (1, 4, 1024, 4096, 16384, 65536)  # decode-join payloads, up to 256 KiB per buffer


def bench_join(args, torch, df, dev, timer):
    """In-place fold dst += stage at the decode-join payload sizes.

    Per size: (a) back-to-back calls through the Python binding (bounded by
    host launch cost), (b) the same calls captured once in a HIP graph and
    replayed (device-side time per call, launch gaps included, no host cost),
    and at 16 KiB (c) the host-observed enqueue-to-complete time of one call.
    """
    import fold_inputs

    sweep = []
    k_graph = 200
    for n in JOIN_SIZES:
        xa = torch.from_numpy(fold_inputs.vecf(n, 11 + n)).to(dev)
        stage = torch.from_numpy(fold_inputs.vecf(n, 77 + n)).to(dev)
        for _ in range(20):
            df.fold_into(xa, stage)
        torch.cuda.synchronize()
        reps = 1000
        b2b = timer.region(lambda: df.fold_into(xa, stage), reps) / reps
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(3):
                df.fold_into(xa, stage)
        torch.cuda.current_stream(dev).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(k_graph):
                df.fold_into(xa, stage)
        graph.replay()
        torch.cuda.synchronize()
        in_graph = timer.region(graph.replay, 10) / (10 * k_graph)
        del graph
        row = {"n": n, "bytes_per_call": 12 * n,
               "python_back_to_back_us_per_call": round(b2b * 1e3, 3),
               "graph_replay_us_per_call": round(in_graph * 1e3, 3)}
        if n == 4096:
            host_us = []
            for _ in range(reps):
                t0 = time.perf_counter()
                df.fold_into(xa, stage)
                torch.cuda.current_stream(dev).synchronize()
                host_us.append((time.perf_counter() - t0) * 1e6)
            row["host_enqueue_to_complete_us_median"] = round(statistics.median(host_us), 3)
        sweep.append(row)
        log("fold_into n=%6d: %.3f us/call via python, %.3f us/call in a graph"
            % (n, b2b * 1e3, in_graph * 1e3))
    at16 = dict(next(r for r in sweep if r["n"] == 4096))
    at16["sweep"] = sweep
    at16["launch_floor_graph_us_per_call"] = round(launch_floor(torch, dev, timer, k_graph) * 1e3, 3)
    log("launch floor (a 1-element fill kernel, same graph method): %.3f us/call"
        % at16["launch_floor_graph_us_per_call"])
    at16["note"] = ("graph_replay_us_per_call: device time per in-place fold, 200 calls captured "
                    "in one HIP graph; python_back_to_back is bounded by host launch cost")
    return at16


def launch_floor(torch, dev, timer, k_graph) -> float:
    """ms per launch of a minimal kernel (torch's fill of one element), captured
    and replayed exactly as the fold_into calls are: the floor under them."""
    x = torch.zeros(1, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(3):
            x.fill_(1.0)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(k_graph):
            x.fill_(1.0)
    graph.replay()
    torch.cuda.synchronize()
    ms = timer.region(graph.replay, 10) / (10 * k_graph)
    del graph
    return ms


def cpu_baseline(args, host, inv_w, outs, W, n, bytes_per_step):
    """The CPU oracle on the same host arrays, single-threaded, repeated for a
    bounded time; its result is also checked bit for bit against the GPU's."""
    import numpy as np
    import torch
    import oracle

    fn = (lambda: oracle.fold_stacked(host)) if inv_w is None else \
        (lambda: oracle.fold_stacked_scaled(host, np.float32(inv_w)))
    want = fn()
    times = []
    t_start = time.perf_counter()
    while (time.perf_counter() - t_start < args.cpu_seconds or len(times) < 3) and len(times) < 5000:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    torch.cuda.synchronize()
    got = outs[0].cpu().numpy()
    bit_exact = bool(np.array_equal(got.view(np.uint32), want.view(np.uint32))) and \
        all_equal(torch, outs[1:], outs[0])
    log("cpu oracle: %d runs, median %.3f s (%.2f GB/s); GPU output bit-exact: %s"
        % (len(times), med, bytes_per_step / med / 1e9, bit_exact))
    threads = min(len(os.sched_getaffinity(0)), 16)
    threaded = None
    if inv_w is None and threads > 1:
        got_t, med_t, runs_t = oracle_threaded(host, threads, args.cpu_seconds / 2)
        same = bool(np.array_equal(got_t.view(np.uint32), want.view(np.uint32)))
        threaded = {"value": round(bytes_per_step / med_t / 1e9, 3), "unit": "GB/s", "cores": threads,
                    "runs": runs_t, "bit_identical_to_single_thread": same,
                    "sample": "the same arena split into %d contiguous element ranges, one thread "
                              "each running the serial oracle on its range" % threads}
        log("cpu oracle on %d threads: median %.3f s (%.2f GB/s); bits equal to one thread: %s"
            % (threads, med_t, bytes_per_step / med_t / 1e9, same))
    return {
        "value": round(bytes_per_step / med / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "the full workload arena (%d x %d f32), %d runs, median" % (W, n, len(times)),
        "cpu_model": cpu_model(),
        "host_cpus_available": len(os.sched_getaffinity(0)),
        "gpu_output_bit_exact_vs_oracle": bit_exact,
        "threaded": threaded,
    }


def oracle_threaded(host, threads, seconds):
    """The serial oracle, unchanged, on `threads` host threads at once: thread t
    folds elements [n*t/T, n*(t+1)/T) through the oracle's separate-slots entry
    (the C call releases the interpreter lock).  Returns the concatenated result,
    the median time of one full fold and the number of timed runs."""
    import threading
    import numpy as np
    import oracle

    W, n = host.shape
    bounds = [(n * t // threads, n * (t + 1) // threads) for t in range(threads)]
    parts = [None] * threads

    def work(t):
        a, b = bounds[t]
        parts[t] = oracle.fold([host[r, a:b] for r in range(W)])

    def once():
        pool = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
        for th in pool:
            th.start()
        for th in pool:
            th.join()
        return np.concatenate(parts)

    got = once()
    times = []
    t_start = time.perf_counter()
    while (time.perf_counter() - t_start < seconds or len(times) < 3) and len(times) < 5000:
        t0 = time.perf_counter()
        once()
        times.append(time.perf_counter() - t0)
    return got, statistics.median(times), len(times)


def bench_join_only(args, torch, df, dev):
    timer = Timer(torch, torch.cuda.current_stream(dev))
    lat = bench_join(args, torch, df, dev, timer)
    n = lat["n"]
    us = lat["graph_replay_us_per_call"]
    return {
        "metric": "16 KiB in-place fold latency (device time per call, graph replay)",
        "value": us, "unit": "us/call", "n_gpus": 1, "steps": 2000, "warmup": 23,
        "ms_per_step": us / 1e3, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES["join"], "n": n}, "latency_16KiB": lat,
    }


def bench_round(args, torch, df, dev):
    """One owner-shard reduction round over W=8 arenas of 64 MiB on one device.

    Bytes moved per round (direct): each owner reads its shard of all W arenas
    and writes its own ((W+1)*n*4 over all owners), then every reduced shard is
    read once and written to the other W-1 arenas (W*n*4).  Staged adds the
    gather copies into the stage (2*W*n*4).  Fused reads every arena once and
    writes it once (2*W*n*4)."""
    import fold_inputs

    W, n = 8, 1 << 24
    host = fold_inputs.slots("vecf", W, n, 1000)
    arenas = [torch.from_numpy(host[r]).to(dev) for r in range(W)]
    stage = torch.empty(df.round_stage_elems(n, W), dtype=torch.float32, device=dev)
    timer = Timer(torch, torch.cuda.current_stream(dev))
    res = {}
    for mode in ("direct", "staged", "fused"):
        direct, fused = mode == "direct", mode == "fused"

        def step():
            df.loopback_round(arenas, stage if mode == "staged" else None, direct=direct, fused=fused)
        for _ in range(args.warmup):
            step()
        ms = timer.region(step, args.steps) / args.steps
        moved = {"direct": (2 * W + 1) * n * 4, "staged": (4 * W + 1) * n * 4, "fused": 2 * W * n * 4}[mode]
        res[mode] = {"ms_per_round": round(ms, 4), "bytes_moved": moved,
                     "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}
        log("round %s: %.3f ms per round, %.1f GB/s of bytes moved" % (mode, ms, res[mode]["GBps"]))
    d = res["direct"]
    return {
        "metric": "one-GPU fixed-order reduction round, W=8 arenas of 64 MiB (bytes moved / time)",
        "value": d["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": d["ms_per_round"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES["round"], "W": W, "len": n}, "round": res,
    }


def bench_pair(args, torch, df, dev):
    """Two ranks on two streams: one all-reduce per call (push, event, fold on
    both ranks), back-to-back through the binding, one call with a host
    synchronization, and the device time per call (calls queued behind a
    spin kernel, so the host's enqueue cost is out of the measurement)."""
    import fold_inputs

    link = df.PairLink(max(JOIN_SIZES), device=dev)
    # the same link with both ranks on one stream: no hand-off between queues
    solo = torch.cuda.Stream(device=dev)
    same = df.PairLink(max(JOIN_SIZES), device=dev, streams=[solo, solo])
    shot = df.OneShotLink(max(JOIN_SIZES), device=dev, stream=torch.cuda.Stream(device=dev))
    cycles_per_ms = sleep_cycles_per_ms(torch)
    rows = []
    for n in JOIN_SIZES:
        xa = torch.from_numpy(fold_inputs.vecf(n, 11 + n)).to(dev)
        xb = torch.from_numpy(fold_inputs.vecf(n, 77 + n)).to(dev)
        torch.cuda.synchronize()
        for _ in range(20):
            link.all_reduce(xa, xb)
        torch.cuda.synchronize()
        reps = 500
        t0 = time.perf_counter()
        for _ in range(reps):
            link.all_reduce(xa, xb)
        torch.cuda.synchronize()
        b2b = (time.perf_counter() - t0) / reps * 1e6
        one = []
        for _ in range(200):
            t1 = time.perf_counter()
            link.all_reduce(xa, xb)
            for st in link.streams:
                st.synchronize()
            one.append((time.perf_counter() - t1) * 1e6)
        row = {"n": n, "back_to_back_us_per_call": round(b2b, 3),
               "enqueue_to_complete_us_median": round(statistics.median(one), 3),
               "device_us_per_call": round(pair_device_us(torch, link, xa, xb, cycles_per_ms), 3),
               "one_stream_device_us_per_call": round(pair_device_us(torch, same, xa, xb, cycles_per_ms), 3),
               "library_only_device_us_per_call": round(pair_raw_device_us(torch, df, link, xa, xb,
                                                                           cycles_per_ms), 3),
               "library_only_one_stream_device_us_per_call": round(
                   pair_raw_device_us(torch, df, same, xa, xb, cycles_per_ms), 3)}
        row["one_shot"] = bench_one_shot(torch, df, dev, shot, xa, xb)
        rows.append(row)
        log("pair all-reduce n=%6d: %.2f us/call back-to-back, %.2f us call+sync, %.2f us/call on the "
            "device (%.2f with both ranks on one stream; the library call alone %.2f, one stream %.2f); "
            "one-shot %s" % (n, b2b, statistics.median(one), row["device_us_per_call"],
                             row["one_stream_device_us_per_call"], row["library_only_device_us_per_call"],
                             row["library_only_one_stream_device_us_per_call"], row["one_shot"]))
    words = shot.barrier_words()
    if words != [0, 0]:
        raise RuntimeError("one-shot barrier words %s after the sweep" % words)
    at16 = next(r for r in rows if r["n"] == 4096)
    return {
        "metric": "two-stream pair all-reduce at 16 KiB (enqueue to completion)",
        "value": at16["enqueue_to_complete_us_median"], "unit": "us/call", "n_gpus": 1,
        "steps": 500, "warmup": 20, "ms_per_step": at16["enqueue_to_complete_us_median"] / 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": {"workload": WORKLOAD_NAMES["pair"], "n": 4096},
        "pair": rows,
    }


def sleep_cycles_per_ms(torch) -> float:
    """Cycles of torch's bounded device spin (torch.cuda._sleep) per ms."""
    probe = 1 << 22
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    torch.cuda._sleep(probe)
    t1.record()
    t1.synchronize()
    return probe / t0.elapsed_time(t1)


def pair_device_us(torch, link, xa, xb, cycles_per_ms, calls=100, hold_ms=20.0):
    """Device time per pair all-reduce, without the host: `calls` calls are
    enqueued while a bounded spin kernel holds the current stream (every call
    forks from it), so they run back to back once it ends; events on the
    current stream after the spin and after the last call's join bracket
    them.  (The link cannot be captured into a graph.)"""
    cur = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(hold_ms * cycles_per_ms))
    start.record(cur)
    t0 = time.perf_counter()
    for _ in range(calls):
        link.all_reduce(xa, xb)
    enqueue_ms = (time.perf_counter() - t0) * 1e3
    end.record(cur)
    end.synchronize()
    if enqueue_ms > hold_ms:
        log("pair device time: enqueueing %d calls took %.1f ms, longer than the %.1f ms hold"
            % (calls, enqueue_ms, hold_ms))
    return start.elapsed_time(end) * 1e3 / calls


def pair_raw_device_us(torch, df, link, xa, xb, cycles_per_ms, calls=100, hold_ms=20.0):
    """Device time per call of the library's pair all-reduce itself, without
    the binding's ordering against the caller's stream: both rank streams are
    held by a bounded spin kernel while `calls` calls are enqueued through the
    C ABI; events after the spins and after the last call bracket them (the
    later end of the two streams counts)."""
    import ctypes
    lib = df.load()
    torch.cuda.synchronize()
    streams = list(dict.fromkeys(link.streams))  # one or two distinct streams
    starts, ends = [], []
    for st in streams:
        with torch.cuda.stream(st):
            torch.cuda._sleep(int(hold_ms * cycles_per_ms))
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        starts.append(e)
    for _ in range(calls):
        rc = lib.detfold_pair_all_reduce(ctypes.byref(link._c), xa.data_ptr(), xb.data_ptr(), xa.numel())
        if rc != df.OK:
            raise df.DetfoldError(rc, "pair_all_reduce")
    for st in streams:
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        ends.append(e)
    torch.cuda.synchronize()
    first = starts[0]
    return max(first.elapsed_time(e) for e in ends) * 1e3 / calls


def bench_one_shot(torch, df, dev, shot, xa, xb):
    """The one-kernel all-reduce on the same buffers: back-to-back through the
    binding, one call with a host synchronization (both with the link's own
    stream as the caller's current stream, so no hand-off between queues),
    and 200 calls captured in one HIP graph (device time per call)."""
    st = shot.stream
    with torch.cuda.stream(st):
        for _ in range(20):
            shot.all_reduce(xa, xb)
        st.synchronize()
        reps = 500
        t0 = time.perf_counter()
        for _ in range(reps):
            shot.all_reduce(xa, xb)
        st.synchronize()
        b2b = (time.perf_counter() - t0) / reps * 1e6
        one = []
        for _ in range(200):
            t1 = time.perf_counter()
            shot.all_reduce(xa, xb)
            st.synchronize()
            one.append((time.perf_counter() - t1) * 1e6)
    k_graph = 200
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for _ in range(k_graph):
            shot.all_reduce(xa, xb)
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream(dev)
    ev0.record(cur)
    for _ in range(10):
        graph.replay()
    ev1.record(cur)
    torch.cuda.synchronize()
    in_graph = ev0.elapsed_time(ev1) * 1e3 / (10 * k_graph)
    del graph
    return {"back_to_back_us_per_call": round(b2b, 3),
            "enqueue_to_complete_us_median": round(statistics.median(one), 3),
            "graph_replay_us_per_call": round(in_graph, 3)}


def sweep(args, torch, df, dev):
    """Launch-geometry sweep of the headline fold, arena copies and outputs
    rotating (all results bit-checked against the default launch's output)."""
    host, stacked, out, W, n, _ = make_workload("w8", torch, dev)
    timer = Timer(torch, torch.cuda.current_stream(dev))
    df.fold_ranks(out, stacked)
    ref = out.clone()
    arenas = arena_set(torch, stacked, WORKLOADS["w8"][5])
    outs = output_set(torch, out)
    bytes_per_step = (W + 1) * n * 4
    configs = [(df.PATH_ROWS, df.POLICY_STREAM, 64 * W, 1, grid) for grid in (0, 512, 1024, 2048, 4096)]
    for policy in (df.POLICY_STREAM, df.POLICY_CACHED):
        for block in (128, 256, 512, 1024):
            for unroll in ((1, 2) if policy == df.POLICY_STREAM else (1,)):
                for grid in (0, 1024, 2048, 4096):
                    configs.append((df.PATH_VECTOR, policy, block, unroll, grid))
    samples = {c: [] for c in configs}
    for rnd in range(3):  # interleaved rounds: drift affects every configuration alike
        for c in configs:
            path, policy, block, unroll, grid = c

            def call(o, a):
                df.fold_ranks_ex(o, a, path=path, block=block, grid=grid, unroll=unroll,
                                 policy=policy)
            state = [0]

            def step():
                i = state[0]
                state[0] += 1
                call(outs[i % len(outs)], arenas[i % len(arenas)])
            for _ in range(3):
                step()
            samples[c].append(timer.region(step, 20) / 20)
            if rnd == 0:
                for k, o in enumerate(outs):
                    call(o, arenas[k % len(arenas)])
                torch.cuda.synchronize()
                if not all_equal(torch, outs, ref):
                    raise AssertionError("sweep configuration %s changed the bits" % (c,))
    rows = []
    for c in configs:
        ms = statistics.median(samples[c])
        gbs = bytes_per_step / (ms * 1e-3) / 1e9
        rows.append({"path": c[0], "policy": c[1], "block": c[2], "unroll": c[3], "grid": c[4],
                     "ms": round(ms, 5), "GBps": round(gbs, 1), "bit_exact": True})
        log("sweep path=%d policy=%d block=%4d unroll=%d grid=%5d: %.4f ms %.1f GB/s"
            % (c[0], c[1], c[2], c[3], c[4], ms, gbs))
    return {"sweep": rows, "workload": WORKLOAD_NAMES["w8"]}


def copy_calibration(args, torch, dev):
    """A plain device-to-device copy of a known 256 MiB, for calibrating the
    HBM byte counters (FETCH_SIZE should read the bytes copied, WRITE_SIZE the
    bytes written)."""
    nbytes = 256 << 20
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    timer = Timer(torch, torch.cuda.current_stream(dev))
    ms = timer.region(lambda: dst.copy_(src), args.steps) / args.steps
    return {"copy_calibration_bytes": nbytes, "ms_per_copy": round(ms, 5),
            "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


PROCS_W, PROCS_N, PROCS_SHOT_N = 4, 1 << 24, 4096


def _free_port() -> int:
    import socket
    with socket.socket(socket.AF_INET, socket.SOCK_STREAM) as so:
        so.bind(("127.0.0.1", 0))
        return so.getsockname()[1]


def _procs_join(rank, world, port):
    import torch.distributed as dist
    root = os.path.dirname(os.path.abspath(__file__))
    if root not in sys.path:
        sys.path.insert(0, root)
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    return dist


def _procs_fold_main(rank, arenas, want, steps, warmup, fused_steps, port, results):
    """Rank `rank`: time its owner-shard fold over the mapped arenas, in turn."""
    import torch
    world = len(arenas)
    dist = _procs_join(rank, world, port)
    try:
        import deterministic_fixed_order_amd as df
        torch.cuda.set_device(0)
        start, length = df.shard_plan(arenas[0].numel(), world)[rank]
        slots = [a[start:start + length] for a in arenas]
        out = torch.empty(length, dtype=torch.float32, device="cuda:0")
        timer = Timer(torch, torch.cuda.current_stream())
        for turn in range(world):
            dist.barrier()  # one rank folds at a time; the others wait on the host
            if turn != rank:
                continue
            for _ in range(warmup):
                df.fold_slots(out, slots)
            results[rank] = timer.region(lambda: df.fold_slots(out, slots), steps) / steps
            same = torch.equal(out.view(torch.int32), want[start:start + length].view(torch.int32))
            results[world + rank] = 1.0 if same else 0.0
        # every rank at once: the fused round over its own shard of all the arenas
        # (the values grow by a factor W per round; bits are checked by the tests)
        for _ in range(3):
            df.loopback_round(slots, fused=True)
        torch.cuda.synchronize()
        dist.barrier()
        results[2 * world + rank] = (timer.region(lambda: df.loopback_round(slots, fused=True), fused_steps)
                                     / fused_steps)
        dist.barrier()
    finally:
        dist.destroy_process_group()


def _procs_shot_main(rank, xs, buffers, calls, delay_cycles, port, results):
    """Rank `rank` of the one-shot link: `calls` back-to-back rank kernels,
    queued behind a delay kernel so that they run without host gaps."""
    import torch
    dist = _procs_join(rank, 2, port)
    try:
        import deterministic_fixed_order_amd as df
        torch.cuda.set_device(0)
        n = xs[rank].numel()
        link = df.OneShotLink(n, device="cuda:0", buffers=buffers, init=False,
                              stream=torch.cuda.Stream(device="cuda:0"))
        for _ in range(20):  # the code object is loaded and both sides are in step
            dist.barrier()
            link.rank(rank, xs[rank], stream=link.stream)
            link.stream.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        dist.barrier()
        with torch.cuda.stream(link.stream):
            torch.cuda._sleep(delay_cycles)  # bounded spin; the calls queue up behind it
            start.record(link.stream)
            for _ in range(calls):
                link.rank(rank, xs[rank], stream=link.stream)
            end.record(link.stream)
        end.synchronize()
        results[rank] = start.elapsed_time(end) * 1e3 / calls  # us per call
        dist.barrier()
    finally:
        dist.destroy_process_group()


def bench_procs(args, torch, df, dev):
    """Ranks as processes on one GPU.

    Fold: PROCS_W processes share PROCS_W arenas of PROCS_N floats (allocated
    by this process, mapped by each child through device memory handles).  In
    turn, each rank times back-to-back folds of its owner shard over all the
    mapped arenas (fold_slots into a buffer of its own, the direct round's
    phase A) while the others wait on a host barrier, and checks its result
    against the same fold run here on the unmapped arenas, bit for bit.

    One-shot: two processes, each launching its own rank's kernel
    (detfold_one_shot_rank) at n = PROCS_SHOT_N; the kernels meet only through
    the shared counters.  The calls are queued behind a bounded delay kernel
    so that the device runs them back to back; the time per call is taken on
    each rank from events around its calls (the rank whose delay ended first
    also counts the wait for its peer's first kernel)."""
    import torch.multiprocessing as mp
    import fold_inputs

    W, n = PROCS_W, PROCS_N
    host = fold_inputs.slots("vecf", W, n, 1000)
    arenas = [torch.from_numpy(host[r]).to(dev) for r in range(W)]
    want = torch.empty(n, dtype=torch.float32, device=dev)
    moved, local = [], []
    timer = Timer(torch, torch.cuda.current_stream(dev))
    for start, length in df.shard_plan(n, W):
        slots = [a[start:start + length] for a in arenas]
        df.fold_slots(want[start:start + length], slots)
        out = torch.empty(length, dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            df.fold_slots(out, slots)
        local.append(timer.region(lambda: df.fold_slots(out, slots), args.steps) / args.steps)
        moved.append((W + 1) * length * 4)
    torch.cuda.synchronize()

    steps_fused = min(args.steps, 20)  # the sums grow 4x per round: 4^(3 + 20) stays finite
    local_fused = timer.region(lambda: df.loopback_round(arenas, fused=True), steps_fused) / steps_fused
    for r in range(W):
        arenas[r].copy_(torch.from_numpy(host[r]))
    torch.cuda.synchronize()
    results = torch.zeros(3 * W, dtype=torch.float64).share_memory_()
    log("procs: %d ranks fold their owner shards over mapped arenas" % W)
    mp.spawn(_procs_fold_main, args=(arenas, want, args.steps, args.warmup, steps_fused, _free_port(), results),
             nprocs=W, join=True)
    torch.cuda.ipc_collect()
    ranks = []
    for r in range(W):
        ms = float(results[r])
        row = {"rank": r, "ms_per_fold": round(ms, 5), "GBps": round(moved[r] / (ms * 1e-3) / 1e9, 1),
               "unmapped_ms_per_fold": round(local[r], 5),
               "unmapped_GBps": round(moved[r] / (local[r] * 1e-3) / 1e9, 1),
               "bits_equal_unmapped": bool(results[W + r] == 1.0)}
        ranks.append(row)
        log("rank %d: %.4f ms per owner fold (%.1f GB/s) over mapped arenas; %.4f ms (%.1f GB/s) "
            "unmapped; bits equal %s" % (r, ms, row["GBps"], local[r], row["unmapped_GBps"],
                                         row["bits_equal_unmapped"]))
    if not all(x["bits_equal_unmapped"] for x in ranks):
        raise RuntimeError("a rank's fold over mapped arenas differs from the unmapped fold")
    fused_ms = max(float(results[2 * W + r]) for r in range(W))
    fused = {"ms_per_round_slowest_rank": round(fused_ms, 4),
             "GBps": round(2 * W * n * 4 / (fused_ms * 1e-3) / 1e9, 1),
             "one_process_one_kernel_ms": round(local_fused, 4),
             "one_process_GBps": round(2 * W * n * 4 / (local_fused * 1e-3) / 1e9, 1),
             "note": "every rank at once runs the fused round over its own shard of all the mapped "
                     "arenas; against one fused kernel over the whole arenas in one process"}
    log("fused round, %d ranks at once over mapped arenas: %.4f ms per round (%.1f GB/s); one "
        "process, one kernel: %.4f ms (%.1f GB/s)" % (W, fused_ms, fused["GBps"], local_fused,
                                                       fused["one_process_GBps"]))

    m, calls = PROCS_SHOT_N, 500
    link = df.OneShotLink(m, device=dev)  # zeroes the counters and the words
    xs = [torch.zeros(m, dtype=torch.float32, device=dev) for _ in range(2)]
    probe_cycles = 1 << 22
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    torch.cuda._sleep(probe_cycles)
    t1.record()
    t1.synchronize()
    ms_per_cycle = t0.elapsed_time(t1) / probe_cycles
    delay_cycles = int(20.0 / ms_per_cycle)  # about 20 ms: room to enqueue every call first
    torch.cuda.synchronize()
    shot = torch.zeros(2, dtype=torch.float64).share_memory_()
    log("procs: one-shot rank kernels in 2 processes, n=%d, %d calls behind a %.1f ms delay"
        % (m, calls, delay_cycles * ms_per_cycle))
    mp.spawn(_procs_shot_main, args=(xs, (link.stage, link.flags, link.words), calls, delay_cycles,
                                     _free_port(), shot), nprocs=2, join=True)
    torch.cuda.ipc_collect()
    words = link.barrier_words()
    if words != [0, 0]:
        raise RuntimeError("one-shot barrier words %s after the process calls" % words)
    per_call = [round(float(shot[r]), 3) for r in range(2)]
    log("one-shot ranks as processes: %s us per call (rank 0, rank 1)" % per_call)

    ms_sum = sum(x["ms_per_fold"] for x in ranks)
    return {
        "metric": "ranks as processes: owner-shard folds over arenas shared by device memory handles",
        "value": round(sum(moved) / (ms_sum * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_sum, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": {"workload": WORKLOAD_NAMES["procs"], "W": W, "len": n},
        "ranks": ranks, "fused_round_processes": fused,
        "one_shot_processes": {"n": m, "calls": calls, "us_per_call": per_call, "barrier_words": words},
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + ["join", "round", "pair", "procs"],
                    default="w8")
    ap.add_argument("--singles", type=int, default=50, help="scrubbed single-launch samples")
    ap.add_argument("--sustained-steps", type=int, default=2000,
                    help="steps of the long region after the headline's (0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--no-owner-shards", dest="owner_shards", action="store_false",
                    help="skip the owner-shard folds of the w16 workload (profiling runs that "
                         "summarize the whole fold's kernel)")
    ap.add_argument("--no-controls", "--no-alternate", dest="controls", action="store_false",
                    help="skip the interleaved cache controls (one arena, every operand reused)")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="skip the library streaming probes (the attainable ceiling)")
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="skip the W=4 and W=16 workloads after the headline")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the fold runs on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import __graft_entry__

    __graft_entry__.ensure_built()
    import deterministic_fixed_order_amd as df

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        res = copy_calibration(args, torch, dev)
    elif args.sweep:
        res = sweep(args, torch, df, dev)
    elif args.workload == "join":
        res = bench_join_only(args, torch, df, dev)
    elif args.workload == "round":
        res = bench_round(args, torch, df, dev)
    elif args.workload == "pair":
        res = bench_pair(args, torch, df, dev)
    elif args.workload == "procs":
        res = bench_procs(args, torch, df, dev)
    else:
        res = bench_fold(args, torch, df, dev)
    res["kernel_source_sha256_16"] = kernel_source_hash()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
