"""Two ranks, every pair of 16-bit inputs: the N=2 RS/AG reduction of f16 and
bf16 buffers run over all 2^32 pairs (x_0, x_1) of bit patterns -- signed
zeros, subnormals, infinities, NaNs, overflow to infinity and every rounding
case of the narrowing -- and compared with the oracle, bit for bit.  With f32
accumulation every pair is covered; with native accumulation a quarter of
them (x_0 among the smallest and the largest patterns of both signs).

Pair i of the 2^32 is x_0 = i >> 16, x_1 = i & 0xFFFF; each launch covers
2^28 consecutive pairs (4096 values of x_0 against all 65,536 of x_1).

FP8 inputs (both formats, every code including inf and NaN codes) are
covered the same way: every pair at two ranks for each accumulator and
output type, and every triple at three ranks."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import TORCH, announce, assert_bits_equal

pytestmark = pytest.mark.gpu

SLICE = 1 << 28  # pairs per launch
SUB = 1 << 24    # pairs per oracle call on the host


def patterns16():
    """The 65,536 16-bit patterns 0..0xFFFF in order, as an int16 tensor."""
    v = torch.arange(65536, dtype=torch.int32, device="cuda")
    return torch.where(v >= 32768, v - 65536, v).to(torch.int16)


def oracle_pairs(t, acc, lo):
    i = np.arange(lo, lo + SUB, dtype=np.uint64)
    x0 = (i >> np.uint64(16)).astype(np.uint16)
    x1 = (i & np.uint64(0xFFFF)).astype(np.uint16)
    return oracle.allreduce([x0, x1], t, acc, t)


@pytest.mark.parametrize("t,acc,slices", [
    ("f16", "f32", range(16)), ("bf16", "f32", range(16)),
    ("f16", "f16", (0, 7, 8, 15)), ("bf16", "bf16", (0, 7, 8, 15)),
], ids=["f16-f32", "bf16-f32", "f16-native", "bf16-native"])
def test_n2_every_pair(t, acc, slices):
    pat = patterns16()
    x1 = pat.repeat(SLICE // 65536).view(TORCH[t])
    outs = [torch.empty(SLICE, dtype=TORCH[t], device="cuda") for _ in range(2)]
    workers = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for s in slices:
            announce("n=2 every pair", t, acc, "slice", s)
            x0 = pat[s * 4096:(s + 1) * 4096].repeat_interleave(65536).view(TORCH[t])
            st = mrr.mrr_allreduce_rsag_ex([x0, x1], outs, SLICE, t, acc, t, 2)
            assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
            want = list(pool.map(lambda lo: oracle_pairs(t, acc, lo),
                                 range(s * SLICE, (s + 1) * SLICE, SUB)))
            torch.cuda.synchronize()
            assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
            got = outs[0].view(torch.int16).cpu().numpy().view(np.uint16)
            for j, w in enumerate(want):
                k = s * SLICE + j * SUB
                assert_bits_equal(got[j * SUB:(j + 1) * SUB], w, t,
                                  "pairs from x0=%04x x1=%04x" % (k >> 16, k & 0xFFFF))


FP8_TRIPLES = [(t, a, o) for t in ("fp8", "fp8fn") for a in ("f32", "f16", t) for o in (t, "f16", "f32")]


@pytest.mark.parametrize("t,acc,tout", FP8_TRIPLES, ids=["-".join(x) for x in FP8_TRIPLES])
def test_fp8_n2_every_pair_of_codes(t, acc, tout):
    """All 65,536 pairs of FP8 codes (inf and NaN codes included) through the
    two-rank kernel, for every accumulator and output type."""
    announce("fp8 every pair", t, acc, tout)
    i = np.arange(65536, dtype=np.uint32)
    x = [(i >> 8).astype(np.uint8), (i & 0xFF).astype(np.uint8)]
    ins = [torch.from_numpy(v).cuda() for v in x]
    outs = [torch.empty(65536, dtype=TORCH[tout], device="cuda") for _ in range(2)]
    st = mrr.mrr_allreduce_rsag_ex(ins, outs, 65536, t, acc, tout, 2)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    want = oracle.allreduce(x, t, acc, tout)
    for k in range(2):
        got = outs[k].cpu().numpy()
        assert_bits_equal(got.view(want.dtype), want, tout, "out[%d]" % k)


@pytest.mark.parametrize("t", ["fp8", "fp8fn"])
@pytest.mark.parametrize("acc", ["f32", "f16", "native"])
def test_fp8_n3_every_triple_of_codes(t, acc):
    """All 2^24 triples of FP8 codes at three ranks, a rank count with no
    compiled kernel (the size-based dispatcher runs the runtime-N kernel);
    native accumulation rounds to FP8 after each of the two adds."""
    acc = t if acc == "native" else acc
    announce("fp8 every triple", t, acc)
    i = np.arange(1 << 24, dtype=np.uint32)
    x = [(i >> 16).astype(np.uint8), ((i >> 8) & 0xFF).astype(np.uint8), (i & 0xFF).astype(np.uint8)]
    ins = [torch.from_numpy(v).cuda() for v in x]
    outs = [torch.empty(1 << 24, dtype=torch.uint8, device="cuda") for _ in range(3)]
    st = mrr.mrr_allreduce(ins, outs, 1 << 24, t, acc, 3)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    sub = 1 << 20
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        want = np.concatenate(list(pool.map(
            lambda lo: oracle.allreduce([v[lo:lo + sub] for v in x], t, acc, t), range(0, 1 << 24, sub))))
    torch.cuda.synchronize()
    for k in range(3):
        assert_bits_equal(outs[k].cpu().numpy(), want, t, "out[%d]" % k)
