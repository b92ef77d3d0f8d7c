"""GPU parity of the one-call dispatcher mrr_allreduce: the runtime-N RS/AG
kernel for rank counts without a compiled kernel, and the packet / RS-AG
choice by message size, against the CPU oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

ODD_RANKS = [1, 3, 5, 6, 7, 9, 12, 17, 24, 31]
TRIPLES = [("f32", "f32"), ("f16", "f32"), ("bf16", "bf16"), ("fp8", "f32"), ("fp8", "fp8")]


@pytest.mark.parametrize("n", ODD_RANKS)
@pytest.mark.parametrize("t,acc", TRIPLES, ids=["-".join(x) for x in TRIPLES])
def test_runtime_rank_count(n, t, acc):
    count = 3 * 64 * 16 * n + 11  # several tiles per chunk and a ragged tail
    announce("dispatch runtime-N", n, t, acc, count)
    ins = inputs_for(t, n, count, seed0=900 + n)
    outs = [empty(t, count, 0xA5) for _ in range(n)]
    assert mrr.mrr_allreduce(ins, outs, count, t, acc, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], t, acc, t)
    for k, o in enumerate(outs):
        assert_bits_equal(bits(o), want, t, "n=%d out[%d]" % (n, k))


def test_runtime_rank_count_full_size():
    """12 ranks x 64 MiB of f16 through the runtime-N kernel, sampled."""
    n, count, t = 12, 32 << 20, "f16"
    announce("dispatch runtime-N 12 x 64 MiB")
    ins = inputs_for(t, n, count, seed0=1200, device="cuda")
    outs = [empty(t, count) for _ in range(n)]
    assert mrr.mrr_allreduce(ins, outs, count, t, "f32", n) == mrr.MRR_OK
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.unique(np.concatenate([
        np.random.default_rng(12).integers(0, count, 1 << 17), [0, count - 1]]))).cuda()
    want = oracle.allreduce([bits(x[idx]) for x in ins], t, "f32")
    for k in range(n):
        assert_bits_equal(bits(outs[k][idx]), want, t, "out[%d]" % k)


@pytest.mark.parametrize("threshold,expect_packets", [(0, False), (1 << 20, True)])
def test_packet_or_rsag_by_size(threshold, expect_packets):
    n, t, count = 8, "f16", 10000
    announce("dispatch threshold", threshold)
    ins = inputs_for(t, n, count, seed0=5, kind="uniform")
    outs = [empty(t, count) for _ in range(n)]
    sbytes = mrr.mrr_packet_scratch_bytes(count, t, n)
    scratch = torch.zeros(sbytes // 8, dtype=torch.int64, device="cuda")
    flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = mrr.mrr_allreduce(ins, outs, count, t, "f32", n, scratch, sbytes, flags, threshold,
                           1_000_000, err)
    assert st == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want = oracle.allreduce([bits(x) for x in ins], t, "f32")
    for k in range(n):
        assert_bits_equal(bits(outs[k]), want, t, "out[%d]" % k)
    f = flags.cpu().numpy().view(np.uint32)
    assert np.all(f == (1 if expect_packets else 0))
