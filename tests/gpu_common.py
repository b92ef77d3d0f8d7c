"""Helpers shared by the GPU parity tests: device buffers, bit-level
comparison against the oracle, and progress prints that name each case
before it touches the GPU."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import synth

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.uint8,
         "fp8fn": torch.uint8}
SIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "fp8fn": 1}


def announce(*what):
    print("[gpu case]", *what, file=sys.stderr, flush=True)


def bits(x: torch.Tensor) -> np.ndarray:
    return synth.to_bits_numpy(x)


def is_nan_bits(a: np.ndarray, t: str) -> np.ndarray:
    a = np.asarray(a)
    if t == "f32":
        u = a.view(np.uint32)
        return (u & 0x7FFFFFFF) > 0x7F800000
    if t == "f16":
        return (a.view(np.uint16) & 0x7FFF) > 0x7C00
    if t == "bf16":
        return (a.view(np.uint16) & 0x7FFF) > 0x7F80
    if t == "fp8fn":
        return (a.view(np.uint8) & 0x7F) == 0x7F
    return (a.view(np.uint8) & 0x7F) > 0x78


def assert_bits_equal(got: np.ndarray, want: np.ndarray, t: str, what: str = ""):
    """Bit-exact equality; NaN positions only need to be NaN on both sides."""
    g = np.ascontiguousarray(got)
    w = np.ascontiguousarray(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    view = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
            "fp8fn": np.uint8}[t]
    gn, wn = is_nan_bits(g, t), is_nan_bits(w, t)
    assert np.array_equal(gn, wn), "%s: NaN positions differ" % what
    bad = np.nonzero((g.view(view) != w.view(view)) & ~wn)[0]
    assert bad.size == 0, "%s: %d mismatches, first at %s: got %s want %s" % (
        what, bad.size, bad[:4], g.view(view)[bad[:4]], w.view(view)[bad[:4]])


def empty(t: str, count: int, fill=None) -> torch.Tensor:
    x = torch.empty(count, dtype=TORCH[t], device="cuda")
    if fill is not None:
        x.view(torch.uint8).fill_(fill)
    return x


def inputs_for(t: str, n: int, count: int, seed0: int, kind=None, device="cuda"):
    kind = kind or ("fp8codes" if t in ("fp8", "fp8fn") else "normal")
    return [x.to(device) for x in synth.rank_inputs(kind, t, n, count, seed0, device="cpu")] \
        if device == "cuda" and count * n <= (1 << 24) else \
        synth.rank_inputs(kind, t, n, count, seed0, device=device)


NP_BITS = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
           "fp8fn": np.uint8}


def host_threads() -> int:
    """Host threads for the oracle: the CPUs this process may use, at most
    OMP_NUM_THREADS when set, and at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(16, n))


def oracle_allreduce_threaded(host_ins, t, acc, tout, block=1 << 22):
    """oracle.allreduce over disjoint element blocks on host threads (its
    ctypes calls release the GIL).  Each element is still summed by one
    oracle call in rank order, so the result is the oracle's, whole."""
    count = host_ins[0].size
    want = np.empty(count, dtype=NP_BITS[tout])
    orc = oracle.default()

    def run(lo):
        hi = min(count, lo + block)
        orc.allreduce([x[lo:hi] for x in host_ins], t, acc, tout, out=want[lo:hi])

    with ThreadPoolExecutor(host_threads()) as ex:
        for f in [ex.submit(run, lo) for lo in range(0, count, block)]:
            f.result()
    return want


def assert_outputs_match(outs, want, t, what):
    """Every element of every output equals the oracle's bits (NaN against NaN
    counts as equal): compared on the GPU, with a host comparison for the
    message when something differs."""
    ints = {1: (np.uint8, torch.uint8), 2: (np.int16, torch.int16),
            4: (np.int32, torch.int32)}[SIZE[t]]
    w = torch.from_numpy(np.ascontiguousarray(want).view(ints[0])).to("cuda")
    for k, o in enumerate(outs):
        got = o.view(-1).view(torch.uint8).view(ints[1])
        assert got.numel() == w.numel(), (what, got.numel(), w.numel())
        if not torch.equal(got, w):
            assert_bits_equal(bits(o), want, t, "%s out[%d]" % (what, k))
