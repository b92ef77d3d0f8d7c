"""MRR_COOPERATIVE=1: the kernels whose workgroups wait for each other (allpair
and two-phase packets, full mesh) launch through hipLaunchCooperativeKernel,
eagerly and under HIP-graph capture.  Normal path only: every call fits on
the GPU and must give the oracle's sum; every wait is bounded."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

SPINS = 2_000_000
ALGS = {"allpair": (mrr.mrr_packet_scratch_bytes, mrr.mrr_allreduce_packet_ex),
        "two-phase": (mrr.mrr_packet_rsag_scratch_bytes, mrr.mrr_allreduce_packet_rsag),
        "fullmesh": (mrr.mrr_fullmesh_scratch_bytes, mrr.mrr_allreduce_fullmesh)}


@pytest.mark.parametrize("alg", sorted(ALGS))
@pytest.mark.parametrize("n,count", [(8, 8192), (2, 200003), (32, 4099)])
def test_cooperative_launch_eager_and_captured(alg, n, count, mrr_env):
    t = "f16"
    announce("cooperative", alg, n, count)
    mrr_env("MRR_COOPERATIVE", "1")
    size_fn, entry = ALGS[alg]
    sbytes = size_fn(count, t, n)
    scratch = torch.zeros(-(-sbytes // 8), dtype=torch.int64, device="cuda")
    flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ins = inputs_for(t, n, count, seed0=n + count, kind="uniform")
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    want = oracle.allreduce([bits(x) for x in ins], t, "f32")

    def call(stream=None):
        return entry(ins, outs, scratch, sbytes, flags, count, t, "f32", n, SPINS, err, 0, 0,
                     stream=stream)

    for it in (1, 2):
        assert call() == mrr.MRR_OK
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for k in range(n):
            assert_bits_equal(bits(outs[k]), want, t, "%s eager %d out[%d]" % (alg, it, k))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert call(stream=s) == mrr.MRR_OK
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.all(flags.cpu().numpy().view(np.uint32) == 3 + rep)
        for k in range(n):
            assert_bits_equal(bits(outs[k]), want, t, "%s replay %d out[%d]" % (alg, rep, k))
