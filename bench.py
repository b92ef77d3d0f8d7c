#!/usr/bin/env python3
"""Benchmark of the N-rank reduction on one MI355X.

Default workload (one "step" = one RS/AG zero-copy allreduce call over all
ranks' chunks): 8 ranks x 64 MiB of f16 ~N(0,1) each, FP32 accumulation,
every output written.  Inputs are resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config c2]

Prints ONE JSON line.  ``value`` is algorithmic HBM bytes per call
(N * count * (e_in + e_out)) divided by the mean wall time per step; the
``roofline`` object divides the same bytes by the kernel's mean duration
measured with HIP events on the launch stream.  ``cpu_baseline`` times the
CPU oracle on a bounded sample of the same workload.

Other configurations (--config): c1 (2 x 1 MiB bf16), c3 (LL-packet allpair,
8 ranks, --size KiB), c4 (8 x 32 MiB FP8 -> f16, f32 or FP8 via --out; --fp8 picks
E4M3B15 or OCP E4M3FN),
c5 (N x 256 MiB bf16 via --nranks), custom (--nranks N --size KiB --dtype T; rank
counts outside 2/4/8/16/32 run the runtime-N kernel through mrr_allreduce),
codec (the standalone E4M3B15 codec over 8 x 32 MiB codes, --dir).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (and % of peak) for N-rank reduce at 64–256 MiB/rank"
PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MiB = 1 << 20
ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "fp8fn": 1}
PROFILE_DIR = os.path.join(ROOT, "profiles")
TIMING_EAGER = "HIP events around K eager calls on the launch stream"
TIMING_GRAPH = "HIP events around one replay of a HIP graph holding the K calls"
KERNEL_SOURCES = ["allreduce_reduction_nranks_amd/csrc/rsag.hip",
                  "allreduce_reduction_nranks_amd/csrc/mrr_device.hpp",
                  "allreduce_reduction_nranks_amd/csrc/mrr_internal.hpp"]
CODEC_SOURCES = ["allreduce_reduction_nranks_amd/csrc/codec.hip",
                 "allreduce_reduction_nranks_amd/csrc/mrr_device.hpp",
                 "allreduce_reduction_nranks_amd/csrc/mrr_internal.hpp"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str, sources=None):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or
    None when it is missing or was taken on different kernel sources."""
    path = os.path.join(PROFILE_DIR, "%s_pmc.txt" % workload_key)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        parts = line.split()
        if len(parts) >= 2 and not line.startswith("#"):
            vals[parts[0]] = parts[1]
    if vals.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """Times K back-to-back calls: host wall clock between synchronizations
    (ms_per_step) and HIP events on the launch stream (kernel mean)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps, warmup, prime=None):
        """prime(), when given, runs after the warm-up and before the timed
        region (the benchmark poisons the outputs there, so the parity check
        afterwards sees what the timed calls wrote)."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        if prime is not None:
            prime()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        wall_ms = (t1 - t0) * 1e3 / steps
        kern_ms = e0.elapsed_time(e1) / steps
        return wall_ms, kern_ms

    def per_call(self, fn, steps):
        """K more calls with an event between consecutive calls: the per-call
        durations' median, min and max in us (a pass of its own, so the
        extra events do not touch the mean above)."""
        import statistics
        torch = self.torch
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(steps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        d = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]
        return {"median": round(statistics.median(d), 2), "min": round(min(d), 2),
                "max": round(max(d), 2), "calls": steps}

    def run_graph(self, fn, steps, warmup, prime=None):
        """The K calls captured once into a HIP graph and replayed: per-call
        GPU time without the host's per-call launch cost (what a captured
        inference step sees).  The library's calls allocate nothing and keep
        their state on the device, so replays are valid calls.  prime() as
        for run(), before the timed replay."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(steps):
                    fn()
        torch.cuda.synchronize()
        g.replay()  # warm replay
        if prime is not None:
            prime()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def use_graph(args, alg_bytes):
    """--graph auto: graph timing for calls that move under 64 MiB, where the
    host's per-call cost (ctypes + launch, several us) would otherwise be
    what is measured."""
    return args.graph == "on" or (args.graph == "auto" and alg_bytes < 64 * MiB)


def copy_ceiling(torch, mrr, nbytes, steps=10):
    """Two plain device copies of nbytes (read nbytes + write nbytes), in GB/s:
    torch's copy_, and mrr_stream_copy, the library's copy on the launch
    scheme of its reduction kernels (the same 1:1 read/write mix without the
    arithmetic, so the practical ceiling a reduction is read against)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    _, kern = Timer(torch).run(lambda: b.copy_(a), steps, 3)
    torch_gbps = 2 * nbytes / (kern * 1e-3) / 1e9

    def stream_copy():
        st = mrr.mrr_stream_copy(a, b, nbytes)
        if st != mrr.MRR_OK:
            raise mrr.MrrError(st, "mrr_stream_copy")

    _, kern = Timer(torch).run(stream_copy, max(steps, 20), 3)
    stream_gbps = 2 * nbytes / (kern * 1e-3) / 1e9
    del a, b
    return torch_gbps, stream_gbps


def add_ceilings(result, ceilings, achieved):
    """Copy-ceiling figures into the JSON config (see copy_ceiling)."""
    if ceilings is None:
        return
    torch_gbps, stream_gbps = ceilings
    result["config"]["copy_ceiling_gbps"] = round(torch_gbps, 2)
    result["config"]["stream_copy_gbps"] = round(stream_gbps, 2)
    result["config"]["frac_of_stream_copy"] = round(achieved / stream_gbps, 4)


POISON = 0x5A  # byte written over every output before the timed region


def poison(bufs):
    """Overwrites every output with a byte pattern (outside the timed region),
    so outputs the timed calls did not write fail the parity check."""
    for b in bufs:
        b.view(-1).view(__import__("torch").uint8).fill_(POISON)


def host_threads() -> int:
    """Threads for the oracle's all-cores leg: the CPUs this process may run
    on, capped by OMP_NUM_THREADS when it is set (a host's share per GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def split_range(lo, hi, parts, align=4096):
    """[lo, hi) as at most `parts` disjoint blocks whose inner edges are
    multiples of `align` elements."""
    step = -(-(hi - lo) // max(1, parts))
    step = max(align, -(-step // align) * align)
    return [(a, min(hi, a + step)) for a in range(lo, hi, step)]


def run_blocks(fn, lo, hi, threads):
    """fn(a, b) over disjoint blocks of [lo, hi), one block per thread.  The
    oracle's ctypes calls release the GIL, so the blocks run in parallel; each
    element is still summed in rank order, so results are those of one call."""
    blocks = split_range(lo, hi, threads)
    if threads <= 1 or len(blocks) <= 1:
        for a, b in blocks:
            fn(a, b)
        return
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(blocks)) as ex:
        for f in [ex.submit(fn, a, b) for a, b in blocks]:
            f.result()


def oracle_legs(block_fn, elems_total, bytes_per_elem, sample_bytes, threads, what):
    """The CPU baseline: the oracle as it stands timed on one thread and on
    `threads` threads (disjoint element blocks), each over a bounded prefix of
    the workload -- sample_bytes of algorithmic bytes per thread -- with one
    warm-up run and the median of three timed runs.  block_fn(a, b) runs the
    oracle over elements [a, b) of every rank."""
    import statistics
    legs = []
    for th in (1, threads):
        elems = min(elems_total, max(4096, th * sample_bytes // bytes_per_elem))
        runs = []
        for i in range(4):  # 1 warm-up + 3 timed
            t0 = time.perf_counter()
            run_blocks(block_fn, 0, elems, th)
            if i:
                runs.append(time.perf_counter() - t0)
        med = statistics.median(runs)
        legs.append({"threads": th, "value": round(elems * bytes_per_elem / med / 1e9, 4),
                     "unit": "GB/s", "median_s": round(med, 3),
                     "runs_s": [round(r, 3) for r in runs], "elements_per_rank": elems,
                     "fraction_of_workload": round(elems / elems_total, 4)})
        if threads == 1:
            break
    best = legs[-1]
    return {"value": best["value"], "unit": "GB/s", "cores": best["threads"], "kind": "oracle",
            "host_cores": os.cpu_count(), "threads_available": threads,
            "sample": "%s; first %d elements of every rank (%.1f%% of the workload) on %d "
                      "threads, and the first %d on one thread; 1 warm-up + median of 3 runs "
                      "each" % (what, best["elements_per_rank"],
                                100.0 * best["fraction_of_workload"], best["threads"],
                                legs[0]["elements_per_rank"]),
            "legs": legs}


_NAN_TEST = {  # bit pattern -> NaN, on integer views of the element type
    "f32": lambda x: (x & 0x7FFFFFFF) > 0x7F800000,
    "f16": lambda x: (x & 0x7FFF) > 0x7C00,
    "bf16": lambda x: (x & 0x7FFF) > 0x7F80,
    "fp8": lambda x: (x & 0x7F) > 0x78,
    "fp8fn": lambda x: (x & 0x7F) == 0x7F,
}


def count_mismatches(torch, outs, want_bits, t, lo=0):
    """Elements of outs[k][lo : lo + len(want_bits)] whose bits differ from
    the oracle's (NaN against NaN counts as equal: only NaN-ness is
    specified), summed over every output k; compared on the outputs' device."""
    import numpy as np
    e = ESIZE[t]
    ints = {1: (np.uint8, torch.uint8), 2: (np.int16, torch.int16), 4: (np.int32, torch.int32)}[e]
    want = torch.from_numpy(np.ascontiguousarray(want_bits).view(ints[0])).to(outs[0].device)
    n = want.numel()
    bad = 0
    for o in outs:
        got = o.view(-1).view(torch.uint8)[lo * e:(lo + n) * e].view(ints[1])
        diff = got != want
        if bool(diff.any()):
            isnan = _NAN_TEST[t]
            diff &= ~(isnan(got) & isnan(want))
            bad += int(diff.sum())
    return bad


def verify_rsag(torch, orc, host_ins, outs, t, acc, tout, lo, hi, threads):
    """The oracle over elements [lo, hi) of every rank (all host threads, on
    disjoint blocks), compared with every output of the last timed call."""
    import numpy as np
    NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
          "fp8fn": np.uint8}
    want = np.empty(hi - lo, dtype=NP[tout])

    def block(a, b):
        orc.allreduce([x[a:b] for x in host_ins], t, acc, tout, out=want[a - lo:b - lo])

    t0 = time.perf_counter()
    run_blocks(block, lo, hi, threads)
    dt = time.perf_counter() - t0
    bad = count_mismatches(torch, outs, want, tout, lo)
    return {"mismatches": bad, "elements": len(outs) * (hi - lo), "outputs": len(outs),
            "oracle_s": round(dt, 2), "threads": threads,
            "checked": "every element of every output of the last timed call, bit for bit "
                       "against the oracle (outputs poisoned before the timed region)"}


def cpu_baseline_rsag(args, torch, ins_dev, outs, t, acc, tout, lo, hi):
    """The cpu_baseline leg: the oracle timed on this host (one thread and all
    threads), then run over the whole measured range to check the timed
    call's outputs."""
    import oracle
    import synth
    orc = oracle.default()  # build/load outside the timed runs
    threads = host_threads()
    host_ins = [synth.to_bits_numpy(x) for x in ins_dev]
    n = len(host_ins)
    per_elem = n * (ESIZE[t] + ESIZE[tout])

    def block(a, b):
        orc.allreduce_all([x[a:b] for x in host_ins], t, acc, tout)

    base = oracle_legs(block, host_ins[0].size, per_elem, args.cpu_sample_mib * MiB, threads,
                       "all %d outputs written" % n)
    parity = verify_rsag(torch, orc, host_ins, outs, t, acc, tout, lo, hi, threads)
    return base, parity


def bench_rsag(args, torch, mrr, synth):
    if args.config == "c1":
        n, t, per_rank = 2, "bf16", 1 * MiB
        tout, acc = t, "f32"
        kind = "normal"
    elif args.config == "c4":
        n, t, per_rank = 8, ("fp8fn" if args.fp8 == "e4m3fn" else "fp8"), 32 * MiB
        tout, acc = (t if args.out == "fp8" else args.out), "f32"
        kind = "fp8codes"
    elif args.config == "c5":
        n, t, per_rank = args.nranks, "bf16", 256 * MiB
        tout, acc = t, "f32"
        kind = "normal"
    elif args.config == "custom":
        n, t, per_rank = args.nranks, args.dtype, args.size * 1024
        fp8 = t in ("fp8", "fp8fn")
        tout, acc = ((t if args.out == "fp8" else args.out) if fp8 else t), "f32"
        kind = "fp8codes" if fp8 else "normal"
    else:
        n, t, per_rank = 8, "f16", 64 * MiB
        tout, acc = t, "f32"
        kind = "normal"
    count = per_rank // ESIZE[t]
    gen_dev = "cuda" if n * count > (1 << 26) else "cpu"
    log("config", args.config, "n", n, "type", t, "->", tout, "count", count, "inputs drawn on", gen_dev)
    ins_sep = [x.to("cuda") for x in synth.rank_inputs(kind, t, n, count, args.seed0, device=gen_dev)]
    outs_sep = [torch.empty(count * ESIZE[tout], dtype=torch.uint8, device="cuda") for _ in range(n)]
    if args.layout == "pitch":
        # The library's recommended HBM placement: each side's N rank buffers
        # in one allocation, mrr_rank_buffer_pitch() bytes apart.
        _, ins = mrr.alloc_rank_buffers(n, count, t)
        for dst, src in zip(ins, ins_sep):
            dst.view(torch.uint8).copy_(src.view(torch.uint8))
        _, outs = mrr.alloc_rank_buffers(n, count, tout)
        layout = ("one allocation per side, rank buffers %d B apart (mrr_rank_buffer_pitch)"
                  % mrr.mrr_rank_buffer_pitch(count * ESIZE[t], n))
    else:
        ins, outs = ins_sep, outs_sep
        layout = "one allocation per rank buffer"
    torch.cuda.synchronize()

    compiled = n in (2, 4, 8, 16, 32)
    if not compiled and tout != t:
        raise SystemExit("rank counts outside 2/4/8/16/32 run through mrr_allreduce, whose output "
                         "type is the input type: --out %s is not available at %d ranks" % (tout, n))

    rank = args.rank
    if rank >= 0 and (not compiled or rank >= n):
        raise SystemExit("--rank needs a compiled rank count (2, 4, 8, 16, 32) and 0 <= rank < N")

    def step():
        if compiled:
            st = mrr.mrr_allreduce_rsag_ex(ins, outs, count, t, acc, tout, n, rank)
        else:  # rank counts without a compiled kernel: the runtime-N RS/AG
            st = mrr.mrr_allreduce(ins, outs, count, t, acc, n)
        if st != mrr.MRR_OK:
            raise mrr.MrrError(st)

    if rank < 0:
        lo, hi = 0, count
    else:  # one rank's share: chunk `rank` of every input, written to every output
        gran = 256 // ESIZE[t]  # chunk widths are rounded to 256 bytes of input
        per = -(-count // n)
        chunk = -(-per // gran) * gran
        lo, hi = min(count, rank * chunk), min(count, (rank + 1) * chunk)
    alg_bytes = n * (hi - lo) * (ESIZE[t] + ESIZE[tout])
    graph = use_graph(args, alg_bytes)
    eager_us = None
    prime = lambda: poison(outs)  # noqa: E731
    if graph:
        eager_us = Timer(torch).run(step, args.steps, args.warmup)[1] * 1e3
        wall_ms, kern_ms = Timer(torch).run_graph(step, args.steps, args.warmup, prime)
    else:
        wall_ms, kern_ms = Timer(torch).run(step, args.steps, args.warmup, prime)
    # The parity check reads what the last timed call wrote: nothing before it
    # writes `outs` again (the layout comparison and the copy ceiling use
    # buffers of their own, and the per-call pass runs after the check).
    checked = outs
    sep_us = None
    if args.layout == "pitch" and args.layout_compare:
        def step_sep():
            st = mrr.mrr_allreduce_rsag_ex(ins_sep, outs_sep, count, t, acc, tout, n, rank) \
                if compiled else mrr.mrr_allreduce(ins_sep, outs_sep, count, t, acc, n)
            if st != mrr.MRR_OK:
                raise mrr.MrrError(st)
        # A short pass (at most 20 timed calls after 5 warm-up calls), so that
        # in a kernel trace of the default command these launches weigh
        # little against the 100 timed ones.
        timer = Timer(torch)
        sep_us = (timer.run_graph if graph else timer.run)(
            step_sep, min(args.steps, 20), min(args.warmup, 5))[1] * 1e3
    value = alg_bytes / (wall_ms * 1e-3) / 1e9
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    key = {"c1": "rsag_2x1MiB_bf16", "c2": "rsag_8x64MiB_f16",
           "c4": "rsag_8x32MiB_%s_to_%s" % (t, tout), "c5": "rsag_%dx256MiB_bf16" % n,
           "custom": "rsag_%dx%dKiB_%s%s" % (n, args.size, t,
                                              "" if tout == t else "_to_" + tout)}[args.config]
    traffic = measured_traffic(key)
    ceiling = copy_ceiling(torch, mrr, n * count * ESIZE[t]) if args.copy_ceiling else None
    workload = {"c1": "RS/AG allreduce, 2 ranks x 1 MiB bf16 ~N(0,1), fp32 accumulation",
                "c2": "RS/AG zero-copy allreduce, 8 ranks x 64 MiB f16 ~N(0,1), fp32 accumulation, "
                      "reduced chunks written to all 8 outputs",
                "c4": "RS/AG allreduce, 8 ranks x 32 MiB FP8 %s finite codes, fp32 "
                      "accumulation, %s outputs"
                      % ("E4M3B15" if t == "fp8" else "OCP E4M3FN", tout),
                "c5": "RS/AG allreduce, %d ranks x 256 MiB bf16 ~N(0,1), fp32 accumulation" % n,
                "custom": "RS/AG allreduce, %d ranks x %d KiB %s, fp32 accumulation, %s outputs"
                          % (n, args.size, t, tout)}[args.config]
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if acc == "f32" else acc,
        "data": "synthetic (seeded, rank r drawn with seed %d + r)" % args.seed0,
        "config": {"workload": workload, "nranks": n, "bytes_per_rank": count * ESIZE[t],
                   "count": count, "in": t, "accum": acc, "out": tout,
                   "algorithmic_bytes_per_call": alg_bytes, "kernel_us": round(kern_ms * 1e3, 2),
                   "pct_of_hbm_peak": round(100 * value / PEAK_GBPS, 2), "layout": layout},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic},
    }
    add_ceilings(result, ceiling, achieved)
    if sep_us is not None:
        # The same call on one allocation per rank buffer (N separate tensors,
        # the natural layout for callers that do not use alloc_rank_buffers).
        result["config"]["kernel_us_one_allocation_per_rank"] = round(sep_us, 2)
        result["config"]["frac_one_allocation_per_rank"] = round(
            alg_bytes / (sep_us * 1e-6) / 1e9 / PEAK_GBPS, 4)
    result["config"]["timing"] = TIMING_GRAPH if graph else TIMING_EAGER
    if eager_us is not None:
        result["config"]["eager_us_per_call"] = round(eager_us, 2)
    if rank >= 0:
        # One rank's share (the per-GPU work of the sharded layout); the
        # counter summaries cover whole calls only.
        result["config"]["workload"] += (", rank %d's share only (chunk %d of every input, "
                                         "written to all %d outputs)" % (rank, rank, n))
        result["config"]["rank"] = rank
        result["roofline"]["traffic"] = None
    if args.cpu_baseline:
        base, parity = cpu_baseline_rsag(args, torch, ins, checked, t, acc, tout, lo, hi)
        if rank < 0:
            result["cpu_baseline"] = base
        result["parity"] = parity
    if not graph:
        # K more calls on the same buffers, an event between consecutive ones.
        result["config"]["kernel_us_per_call"] = Timer(torch).per_call(step, args.steps)
    return result


def bench_packet(args, torch, mrr, synth):
    n, t = args.nranks, args.dtype
    if n not in (2, 4, 8, 16, 32) or t not in ("f32", "f16", "bf16"):
        raise SystemExit("c3 takes --nranks 2/4/8/16/32 and --dtype f32/f16/bf16")
    count = args.size * 1024 // ESIZE[t]
    ins = [x.to("cuda") for x in synth.rank_inputs("uniform", t, n, count, args.seed0)]
    outs = [torch.empty_like(x) for x in ins]
    two_phase = args.algo == "rsag"
    fullmesh = args.algo == "fullmesh"
    sbytes = {"allpair": mrr.mrr_packet_scratch_bytes, "rsag": mrr.mrr_packet_rsag_scratch_bytes,
              "fullmesh": mrr.mrr_fullmesh_scratch_bytes}[args.algo](count, t, n)
    scratch = torch.zeros(-(-sbytes // 8), dtype=torch.int64, device="cuda")
    flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    entry = {"allpair": mrr.mrr_allreduce_packet_ex, "rsag": mrr.mrr_allreduce_packet_rsag,
             "fullmesh": mrr.mrr_allreduce_fullmesh}[args.algo]

    def step():
        st = entry(ins, outs, scratch, sbytes, flags, count, t, "f32", n, 4_000_000, err,
                   args.blocks, args.threads)
        if st != mrr.MRR_OK:
            raise mrr.MrrError(st)

    S = count * ESIZE[t]
    graph = use_graph(args, n * S)
    eager_us = None
    prime = lambda: poison(outs)  # noqa: E731
    if graph:
        eager_us = Timer(torch).run(step, args.steps, args.warmup)[1] * 1e3
        wall_ms, kern_ms = Timer(torch).run_graph(step, args.steps, args.warmup, prime)
    else:
        wall_ms, kern_ms = Timer(torch).run(step, args.steps, args.warmup, prime)
    if int(err.item()) != 0:
        raise RuntimeError("packet poll timed out")
    # allpair: send reads NS, packets 2N(N-1)S written and read, own input NS, outputs NS.
    # two-phase: input NS; rs packets 2(N-1)S written and read; own chunk S; outputs NS;
    # ag packets 2(N-1)S written and read.
    # full-mesh: peers' chunks (N-1)S read, written to inboxes and read back; own
    # chunks S; outputs NS.
    alg_bytes = {"allpair": 3 * n * S + 4 * n * (n - 1) * S,
                 "rsag": 3 * n * S + 8 * (n - 1) * S,
                 "fullmesh": (4 * n - 2) * S}[args.algo]
    name = {"allpair": "LL-packet allpair", "rsag": "two-phase (RS + AG) packet",
            "fullmesh": "full-mesh (plain data + semaphores)"}[args.algo]
    result = {
        "metric": "%s allreduce latency" % name, "value": round(kern_ms * 1e3, 3),
        "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic ~U(-1,1)",
        "config": {"workload": "%s allreduce, %d ranks x %d KiB %s" % (name, n, args.size, t),
                   "nranks": n, "bytes_per_rank": S, "blocks_per_rank": args.blocks,
                   "threads": args.threads, "algorithmic_bytes_per_call": alg_bytes,
                   "algorithmic_gbps": round(alg_bytes / (kern_ms * 1e-3) / 1e9, 2),
                   "timing": TIMING_GRAPH if graph else TIMING_EAGER,
                   "eager_us_per_call": None if eager_us is None else round(eager_us, 3)},
    }
    if args.cpu_baseline:
        base, parity = cpu_baseline_rsag(args, torch, ins, outs, t, "f32", t, 0, count)
        base["sample"] += " (the RS/AG sum the packet path must equal)"
        result["cpu_baseline"] = base
        result["parity"] = parity
    return result


def bench_dual(args, torch, mrr, synth):
    """FP8 workload with both outputs from one pass: 8 ranks x 32 MiB codes,
    fp32 accumulation, f16 outputs and the FP8 re-encode (mrr_allreduce_rsag_dual)."""
    n, per_rank = 8, 32 * MiB
    t = "fp8fn" if args.fp8 == "e4m3fn" else "fp8"
    acc, count = "f32", per_rank
    gen_dev = "cuda"
    log("config c4 dual", "n", n, "type", t, "count", count)
    src = [x.to("cuda") for x in synth.rank_inputs("fp8codes", t, n, count, args.seed0, device=gen_dev)]
    _, ins = mrr.alloc_rank_buffers(n, count, t)
    for dst, x in zip(ins, src):
        dst.copy_(x)
    del src
    _, o16 = mrr.alloc_rank_buffers(n, count, "f16")
    _, o8 = mrr.alloc_rank_buffers(n, count, t)
    torch.cuda.synchronize()

    def step():
        st = mrr.mrr_allreduce_rsag_dual(ins, o16, o8, count, t, acc, n, -1)
        if st != mrr.MRR_OK:
            raise mrr.MrrError(st)

    wall_ms, kern_ms = Timer(torch).run(step, args.steps, args.warmup,
                                        lambda: poison(list(o16) + list(o8)))
    alg_bytes = n * count * (1 + 2 + 1)
    value = alg_bytes / (wall_ms * 1e-3) / 1e9
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    key = "rsag_dual_8x32MiB_%s" % t
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded, rank r drawn with seed %d + r)" % args.seed0,
        "config": {"workload": "RS/AG allreduce, 8 ranks x 32 MiB FP8 %s finite codes, fp32 "
                               "accumulation, f16 outputs and the FP8 re-encode from one pass"
                               % ("E4M3B15" if t == "fp8" else "OCP E4M3FN"),
                   "nranks": n, "bytes_per_rank": count, "count": count, "in": t, "accum": acc,
                   "out": "f16 + %s" % t, "algorithmic_bytes_per_call": alg_bytes,
                   "kernel_us": round(kern_ms * 1e3, 2),
                   "pct_of_hbm_peak": round(100 * value / PEAK_GBPS, 2),
                   "layout": "one allocation per side, rank buffers mrr_rank_buffer_pitch() apart",
                   "timing": TIMING_EAGER},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": measured_traffic(key)},
    }
    if args.copy_ceiling:
        add_ceilings(result, copy_ceiling(torch, mrr, n * count), achieved)
    if args.cpu_baseline:
        import oracle
        orc = oracle.default()
        threads = host_threads()
        host_ins = [synth.to_bits_numpy(x) for x in ins]

        def block(a, b):
            sub = [x[a:b] for x in host_ins]
            orc.allreduce_all(sub, t, acc, "f16")
            orc.allreduce_all(sub, t, acc, t)

        result["cpu_baseline"] = oracle_legs(block, count, n * 4, args.cpu_sample_mib * MiB,
                                             threads, "both output sets written")
        p16 = verify_rsag(torch, orc, host_ins, o16, t, acc, "f16", 0, count, threads)
        p8 = verify_rsag(torch, orc, host_ins, o8, t, acc, t, 0, count, threads)
        result["parity"] = {"mismatches": p16["mismatches"] + p8["mismatches"],
                            "elements": p16["elements"] + p8["elements"],
                            "outputs": p16["outputs"] + p8["outputs"],
                            "oracle_s": round(p16["oracle_s"] + p8["oracle_s"], 2),
                            "threads": threads, "checked": p16["checked"] + ", both output sets"}
    return result


CODEC = {  # --dir: (entry point, input type, output type)
    "dec16": ("mrr_fp8b15_to_f16", "fp8", "f16"), "dec32": ("mrr_fp8b15_to_f32", "fp8", "f32"),
    "enc16": ("mrr_f16_to_fp8b15", "f16", "fp8"), "enc32": ("mrr_f32_to_fp8b15", "f32", "fp8")}


def bench_codec(args, torch, mrr, synth):
    """Standalone FP8 E4M3B15 codec over the FP8 workload's volume: 8 x 32 MiB
    codes as one buffer of 268,435,456 elements, one launch per step."""
    fn_name, tin, tout = CODEC[args.dir]
    n = 8 * 32 * MiB
    if tin == "fp8":
        src = synth.fp8_finite_codes(n, args.seed0, device="cuda")
        kind = "uniform over the 240 finite E4M3B15 codes"
    else:
        src = synth.uniform(tin, n, args.seed0, device="cuda")
        kind = "%s ~U(-1,1)" % tin
    dst = torch.empty(n * ESIZE[tout], dtype=torch.uint8, device="cuda")
    fn = getattr(mrr, fn_name)
    torch.cuda.synchronize()

    def step():
        st = fn(src, dst, n)
        if st != mrr.MRR_OK:
            raise mrr.MrrError(st)

    wall_ms, kern_ms = Timer(torch).run(step, args.steps, args.warmup, lambda: poison([dst]))
    alg_bytes = n * (ESIZE[tin] + ESIZE[tout])
    value = alg_bytes / (wall_ms * 1e-3) / 1e9
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    key = "codec_%s_256Mi" % args.dir
    ceiling = copy_ceiling(torch, mrr, n * ESIZE[tin]) if args.copy_ceiling else None
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8" if tin == "fp8" and tout == "f16" else "f32",
        "data": "synthetic (seeded %d), %s" % (args.seed0, kind),
        "config": {"workload": "FP8 E4M3B15 codec %s, %s -> %s, 268,435,456 elements (8 x 32 MiB "
                               "codes)" % (fn_name, tin, tout),
                   "count": n, "in": tin, "out": tout, "algorithmic_bytes_per_call": alg_bytes,
                   "kernel_us": round(kern_ms * 1e3, 2),
                   "pct_of_hbm_peak": round(100 * value / PEAK_GBPS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": measured_traffic(key, CODEC_SOURCES)},
    }
    add_ceilings(result, ceiling, achieved)
    if args.cpu_baseline:
        import numpy as np
        import oracle
        orc = oracle.default()
        threads = host_threads()
        host = synth.to_bits_numpy(src)

        def block(a, b):
            orc.convert(host[a:b], tin, tout)

        result["cpu_baseline"] = oracle_legs(block, n, ESIZE[tin] + ESIZE[tout],
                                             args.cpu_sample_mib * MiB, threads, "conversion")
        NP = {"f32": np.float32, "f16": np.uint16, "fp8": np.uint8}
        want = np.empty(n, dtype=NP[tout])

        def full(a, b):
            orc.convert(host[a:b], tin, tout, out=want[a:b])

        t0 = time.perf_counter()
        run_blocks(full, 0, n, threads)
        dt = time.perf_counter() - t0
        out_t = {"f32": "f32", "f16": "f16", "fp8": "fp8"}[tout]
        result["parity"] = {"mismatches": count_mismatches(torch, [dst.view(torch.uint8)], want,
                                                           out_t),
                            "elements": n, "outputs": 1, "oracle_s": round(dt, 2),
                            "threads": threads,
                            "checked": "every element of the last timed call's output, bit for "
                                       "bit against the oracle (output poisoned before the "
                                       "timed region)"}
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5", "custom", "codec"])
    ap.add_argument("--dir", default="dec16", choices=sorted(CODEC),
                    help="codec: direction (dec16/dec32 = E4M3B15 -> f16/f32, enc16/enc32 = back)")
    ap.add_argument("--dtype", default="f16", choices=["f32", "f16", "bf16", "fp8", "fp8fn"],
                    help="custom / c3: type (fp8 = E4M3B15, fp8fn = OCP E4M3FN; c3 takes "
                         "f32, f16, bf16)")
    ap.add_argument("--nranks", type=int, default=8, help="c3 / c5 / custom: rank count")
    ap.add_argument("--out", default="f16", choices=["f16", "fp8", "f32", "dual"],
                    help="c4 / custom FP8: output type (fp8 = the input's FP8 format; c4 dual = "
                         "f16 outputs and the FP8 re-encode from one pass)")
    ap.add_argument("--fp8", default="e4m3b15", choices=["e4m3b15", "e4m3fn"],
                    help="c4: FP8 input format")
    ap.add_argument("--size", type=int, default=1024, help="c3 / custom: KiB per rank")
    ap.add_argument("--algo", default="allpair", choices=["allpair", "rsag", "fullmesh"],
                    help="c3: allpair packets, the two-phase (RS + AG) packet variant, or the "
                         "full-mesh allreduce (plain data + semaphores)")
    ap.add_argument("--blocks", type=int, default=0, help="c3: blocks per rank (0 = auto)")
    ap.add_argument("--threads", type=int, default=0, help="c3: threads (0 = auto)")
    ap.add_argument("--seed0", type=int, default=0)
    ap.add_argument("--layout", default="pitch", choices=["pitch", "separate"],
                    help="rank buffer placement: one allocation per side at mrr_rank_buffer_pitch() "
                         "spacing (default), or one allocation per buffer")
    ap.add_argument("--cpu-sample-mib", type=int, default=128,
                    help="CPU baseline: algorithmic MiB per thread in each timed oracle run "
                         "(the one-thread and all-threads legs each cover a prefix of the "
                         "workload of that many MiB per thread)")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-copy-ceiling", dest="copy_ceiling", action="store_false")
    ap.add_argument("--no-layout-compare", dest="layout_compare", action="store_false",
                    help="skip the short extra pass that times the same call on one allocation "
                         "per rank buffer (reported as kernel_us_one_allocation_per_rank)")
    ap.add_argument("--rank", type=int, default=-1,
                    help="RS/AG configs: time only this rank's share (chunk `rank`), -1 = all")
    ap.add_argument("--graph", default="auto", choices=["auto", "on", "off"],
                    help="time a HIP graph of the K calls (auto: when a call moves < 64 MiB)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the N rank buffers live in one MI355X's HBM, "
              "so --gpus %d (more than one GPU) is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import allreduce_reduction_nranks_amd as mrr
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mrr.load_library()
    if args.config == "c3":
        result = bench_packet(args, torch, mrr, synth)
    elif args.config == "codec":
        result = bench_codec(args, torch, mrr, synth)
    elif args.config == "c4" and args.out == "dual":
        result = bench_dual(args, torch, mrr, synth)
    else:
        result = bench_rsag(args, torch, mrr, synth)
    print(json.dumps(result), flush=True)
    parity = result.get("parity")
    if parity is not None and parity["mismatches"] != 0:
        print("bench.py: %d of %d output elements differ from the oracle"
              % (parity["mismatches"], parity["elements"]), file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
