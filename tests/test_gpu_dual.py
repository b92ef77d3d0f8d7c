"""GPU parity of the dual-output RS/AG allreduce (FP8 inputs; f16 outputs and
the FP8 re-encode of the same sums from one pass) against the CPU oracle,
bit-exact, and against two single-output calls."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

RANKS = [2, 4, 8, 16, 32]
PAIRS = [("fp8", "f32"), ("fp8", "f16"), ("fp8", "fp8"), ("fp8fn", "f32"), ("fp8fn", "f16"),
         ("fp8fn", "fp8fn")]


def with_specials(ins, t, seed):
    """Plants every exponent-15 code of type t (inf / NaN for E4M3B15; the
    largest finite values and NaN for E4M3FN), signed zeros and the
    smallest subnormals."""
    rng = np.random.default_rng(seed)
    special = np.array([0x78, 0xF8, 0x79, 0xFF, 0x00, 0x80, 0x01, 0x81] if t == "fp8" else
                       [0x7F, 0xFF, 0x7E, 0xFE, 0x00, 0x80, 0x01, 0x81], np.uint8)
    out = []
    for x in ins:
        h = x.cpu().numpy().copy()
        pos = rng.integers(0, h.size, max(1, h.size // 64))
        h[pos] = rng.choice(special, pos.size)
        out.append(torch.from_numpy(h).cuda())
    return out


def dual(ins, t, acc, rank=-1, o16=None, o8=None):
    n, count = len(ins), ins[0].numel()
    o16 = o16 if o16 is not None else [empty("f16", count, 0xA5) for _ in range(n)]
    o8 = o8 if o8 is not None else [empty(t, count, 0xA5) for _ in range(n)]
    st = mrr.mrr_allreduce_rsag_dual(ins, o16, o8, count, t, acc, n, rank)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    return o16, o8


def check(ins, o16, o8, t, acc, what):
    src = [bits(x) for x in ins]
    w16 = oracle.allreduce(src, t, acc, "f16")
    w8 = oracle.allreduce(src, t, acc, t)
    for k in range(len(ins)):
        assert_bits_equal(bits(o16[k]).view(np.uint16), w16, "f16", "%s f16 out[%d]" % (what, k))
        assert_bits_equal(bits(o8[k]), w8, t, "%s fp8 out[%d]" % (what, k))


@pytest.mark.parametrize("n", RANKS)
@pytest.mark.parametrize("t,acc", PAIRS, ids=["-".join(p) for p in PAIRS])
def test_dual_parity(n, t, acc):
    count = 3 * 64 * 16 * n + 13  # several tiles per chunk and a ragged tail
    announce("dual", n, t, acc, count)
    ins = inputs_for(t, n, count, seed0=9000 + n)
    o16, o8 = dual(ins, t, acc)
    check(ins, o16, o8, t, acc, "n=%d" % n)


@pytest.mark.parametrize("n", [2, 8, 32])
@pytest.mark.parametrize("t,acc", PAIRS, ids=["-".join(p) for p in PAIRS])
def test_dual_special_codes(n, t, acc):
    count = 2 * 64 * 16 * n + 7
    announce("dual specials", n, t, acc)
    ins = with_specials(inputs_for(t, n, count, seed0=9100 + n), t, seed=n)
    o16, o8 = dual(ins, t, acc)
    check(ins, o16, o8, t, acc, "specials n=%d" % n)


@pytest.mark.parametrize("t", ["fp8", "fp8fn"])
def test_dual_matches_two_single_calls(t):
    n, count = 8, 300007
    announce("dual vs two calls", t)
    ins = inputs_for(t, n, count, seed0=9200)
    o16, o8 = dual(ins, t, "f32")
    for tout, got in (("f16", o16), (t, o8)):
        outs = [empty(tout, count, 0x11) for _ in range(n)]
        assert mrr.mrr_allreduce_rsag_ex(ins, outs, count, t, "f32", tout, n) == mrr.MRR_OK
        torch.cuda.synchronize()
        for k in range(n):
            assert torch.equal(outs[k].view(torch.uint8), got[k].view(torch.uint8)), (tout, k)


@pytest.mark.parametrize("n", [2, 8, 32])
def test_dual_rank_share_and_in_place(n):
    """rank=r writes only chunk r of both output sets; outputs2 may be the
    inputs themselves (in place)."""
    t, count = "fp8", n * 3000 + 5
    announce("dual rank share", n)
    ins = inputs_for(t, n, count, seed0=9300)
    src = [bits(x) for x in ins]
    w16 = oracle.allreduce(src, t, "f32", "f16")
    w8 = oracle.allreduce(src, t, "f32", t)
    per = -(-count // n)
    chunk = -(-per // 256) * 256
    for r in (0, n - 1):
        o16, o8 = dual(ins, t, "f32", rank=r)
        lo, hi = min(r * chunk, count), min((r + 1) * chunk, count)
        for k in range(n):
            b16 = bits(o16[k]).view(np.uint16)
            b8 = bits(o8[k])
            assert_bits_equal(b16[lo:hi], w16[lo:hi], "f16", "rank %d f16 %d" % (r, k))
            assert_bits_equal(b8[lo:hi], w8[lo:hi], t, "rank %d fp8 %d" % (r, k))
            assert np.all(np.concatenate([b16[:lo], b16[hi:]]) == 0xA5A5)
            assert np.all(np.concatenate([b8[:lo], b8[hi:]]) == 0xA5)
    copies = [x.clone() for x in ins]
    o16, o8 = dual(ins, t, "f32", o8=ins)  # re-encode written over the inputs
    check(copies, o16, o8, t, "f32", "in place")


@pytest.mark.parametrize("t", ["fp8", "fp8fn"])
def test_dual_full_size(t):
    """8 ranks x 32 MiB of FP8 codes, pooled layout: every element of output
    0 of each set against the oracle, all outputs of a set identical."""
    n, count = 8, 32 << 20
    announce("dual 8 x 32 MiB", t)
    pool_in, ins = mrr.alloc_rank_buffers(n, count, t)
    for r, x in enumerate(inputs_for(t, n, count, seed0=9400, device="cuda")):
        ins[r].copy_(x)
    _, o16 = mrr.alloc_rank_buffers(n, count, "f16")
    _, o8 = mrr.alloc_rank_buffers(n, count, t)
    dual(ins, t, "f32", o16=o16, o8=o8)
    src = [bits(x) for x in ins]
    assert_bits_equal(bits(o16[0]).view(np.uint16), oracle.allreduce(src, t, "f32", "f16"), "f16",
                      "f16 out[0]")
    assert_bits_equal(bits(o8[0]), oracle.allreduce(src, t, "f32", t), t, "fp8 out[0]")
    for k in range(1, n):
        assert torch.equal(o16[k].view(torch.uint8), o16[0].view(torch.uint8)), k
        assert torch.equal(o8[k], o8[0]), k
