"""Element counts past 2^31 and 2^32: the 64-bit index paths of the compiled
and runtime-N RS/AG kernels and of the codec, at 4-16 GiB per buffer.

Each call runs twice, into outputs filled with 0x00 and with 0xFF first; the
two results must agree byte for byte over every output, which shows that
every output byte was written.  All N outputs must agree with each other in
full (compared on the device).  Against the oracle the check is sampled: the
reduced value at a position depends only on the N inputs at that position, so
the oracle runs on the inputs gathered at the sampled positions -- windows at
the start, around 2^31 and 2^32 elements, at every chunk edge and at the end,
plus 2^20 random positions."""
import gc

import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

CHUNK_ALIGN = {"f32": 64, "f16": 128, "bf16": 128, "fp8": 256, "fp8fn": 256}


def sample_positions(count, edges, seed):
    marks = [0, 1 << 31, 1 << 32, count] + list(edges)
    parts = [np.arange(max(0, p - 2048), min(count, p + 2048), dtype=np.int64) for p in marks]
    parts.append(np.random.default_rng(seed).integers(0, count, 1 << 20, dtype=np.int64))
    return np.unique(np.concatenate(parts))


def chunk_edges(count, n, t):
    per = -(-count // n)
    chunk = -(-per // CHUNK_ALIGN[t]) * CHUNK_ALIGN[t]
    return [min(count, r * chunk) for r in range(1, n)]


def gathered(x, idx):
    return bits(x[idx])


@pytest.fixture(autouse=True)
def free_device_memory():
    """These buffers take tens of GiB: hand them back after each test."""
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def run_twice(call, make_outs):
    """The call into 0x00-filled and into 0xFF-filled outputs; returns the
    first set after checking the second equals it byte for byte."""
    first = make_outs(0x00)
    assert call(first) == mrr.MRR_OK
    second = make_outs(0xFF)
    assert call(second) == mrr.MRR_OK
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "an output byte was not written"
    del second
    torch.cuda.empty_cache()
    return first


RSAG_CASES = [
    # (ranks, in, accumulator, out, count): the compiled kernels past 2^32
    # elements (FP8 outputs, and f32 outputs through the 16-codes-per-lane
    # kernel), bf16 past 2^31 elements, the runtime-N kernel at 3 ranks
    (2, "fp8", "f32", "fp8", (1 << 32) + 3 * 256 + 5),
    (2, "fp8", "f32", "f32", (1 << 32) + 1000),
    (2, "bf16", "f32", "bf16", (1 << 31) + 1003),
    (3, "f16", "f32", "f16", (1 << 31) + 7),
]


@pytest.mark.parametrize("n,t,acc,tout,count", RSAG_CASES,
                         ids=["%d-%s-%s-%s" % c[:4] for c in RSAG_CASES])
def test_rsag_past_32bit_counts(n, t, acc, tout, count):
    announce("large rsag", n, t, acc, tout, count)
    ins = inputs_for(t, n, count, seed0=4000 + n)

    def call(outs):
        if n in (2, 4, 8, 16, 32):
            return mrr.mrr_allreduce_rsag_ex(ins, outs, count, t, acc, tout, n)
        return mrr.mrr_allreduce(ins, outs, count, t, acc, n)

    outs = run_twice(call, lambda fill: [empty(tout, count, fill) for _ in range(n)])
    for k in range(1, n):
        assert torch.equal(outs[0].view(torch.uint8), outs[k].view(torch.uint8)), "out %d" % k
    pos = sample_positions(count, chunk_edges(count, n, t), seed=count % 1000)
    idx = torch.from_numpy(pos).cuda()
    want = oracle.allreduce([gathered(x, idx) for x in ins], t, acc, tout)
    assert_bits_equal(gathered(outs[0], idx), want, tout, "n=%d %s/%s/%s sampled" % (n, t, acc, tout))


CODEC_CASES = [("dec16", "fp8", "f16", mrr.mrr_fp8b15_to_f16),
               ("enc32", "f32", "fp8", mrr.mrr_f32_to_fp8b15)]


@pytest.mark.parametrize("name,tin,tout,fn", CODEC_CASES, ids=[c[0] for c in CODEC_CASES])
def test_codec_past_2_to_32(name, tin, tout, fn):
    count = (1 << 32) + 5
    announce("large codec", name, count)
    src = inputs_for(tin, 1, count, seed0=77, kind="fp8codes" if tin == "fp8" else "normal")[0]
    out = run_twice(lambda o: fn(src, o[0], count), lambda fill: [empty(tout, count, fill)])[0]
    pos = sample_positions(count, [], seed=5)
    idx = torch.from_numpy(pos).cuda()
    want = oracle.convert(gathered(src, idx), tin, tout)
    assert_bits_equal(gathered(out, idx), want, tout, "%s sampled" % name)
