"""FP8 inputs reduced with a wider accumulator are at least as accurate as
with native FP8 accumulation, on every algorithm variant's GPU output.

The MSCCL++ commit log (entry adding the fp8_e4m3b15 datatype and mixed
precision accumulation) states this for all allreduce algorithm variants;
here it is checked on the outputs of the RS/AG kernel, the runtime-N kernel,
the allpair packet kernel and the two-phase packet kernel, against the exact
sum of the decoded inputs.  With f32 accumulation the sum of at most 32 FP8
values is exact before the one final rounding, so that output wins element
by element; f16 accumulation is compared on the mean error."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, bits, inputs_for

pytestmark = pytest.mark.gpu

SPINS = 2_000_000


def run_variant(variant, ins, t, acc):
    n, count = len(ins), ins[0].numel()
    outs = [torch.empty_like(x) for x in ins]
    if variant == "rsag":
        st = mrr.mrr_allreduce_rsag_ex(ins, outs, count, t, acc, t, n)
    elif variant == "runtime_n":
        st = mrr.mrr_allreduce(ins, outs, count, t, acc, n)
    else:
        flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if variant == "packet_allpair":
            sb = mrr.mrr_packet_scratch_bytes(count, t, n)
            sc = torch.zeros(sb // 8, dtype=torch.int64, device="cuda")
            st = mrr.mrr_allreduce_packet(ins, outs, sc, sb, flags, count, t, acc, n, SPINS, err)
        else:
            sb = mrr.mrr_packet_rsag_scratch_bytes(count, t, n)
            sc = torch.zeros(sb // 8, dtype=torch.int64, device="cuda")
            st = mrr.mrr_allreduce_packet_rsag(ins, outs, sc, sb, flags, count, t, acc, n, SPINS, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, "%s: device error" % variant
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "%s: outputs differ between ranks" % variant
    return bits(outs[0])


@pytest.mark.parametrize("variant,n", [("rsag", 8), ("runtime_n", 6), ("packet_allpair", 8),
                                       ("packet_rsag", 4)])
@pytest.mark.parametrize("t", ["fp8", "fp8fn"])
def test_wider_accumulation_at_least_as_accurate(variant, n, t):
    count = 20000 + 3
    announce("fp8 accuracy", variant, n, t, count)
    ins = inputs_for(t, n, count, seed0=800 + n)
    exact = sum(oracle.widen_f64(bits(x), t) for x in ins)
    err = {}
    for acc in ("f32", "f16", t):
        got = run_variant(variant, ins, t, acc)
        assert np.array_equal(got, oracle.allreduce([bits(x) for x in ins], t, acc, t)), \
            "%s acc %s: differs from the oracle" % (variant, acc)
        err[acc] = np.abs(oracle.widen_f64(got, t) - exact)
    assert np.all(err["f32"] <= err[t]), "%s: f32 accumulation less accurate somewhere" % variant
    assert err["f32"].max() <= err[t].max()
    assert err["f16"].mean() <= err[t].mean()
    assert err["f32"].mean() < err[t].mean()  # the inputs make native FP8 sums round
