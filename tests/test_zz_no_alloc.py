"""GPU checks of mrr_allreduce_packet_noalloc, the LL-packet allpair allreduce
whose scratch and flag slots live in the library's own static device
workspace: outputs equal those of mrr_allreduce_packet (caller-owned scratch
and flags) bit for bit, and the oracle's sum, over consecutive calls that
shrink, grow and change rank count and type on the one shared workspace.
Every poll is bounded by max_spins, so a protocol fault ends in an error word,
not a hang."""
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

SPINS = 2_000_000
KiB = 1 << 10
ESZ = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "fp8fn": 1}


def with_own_buffers(ins, t, acc):
    """The existing entry point, on fresh caller-owned scratch and flags."""
    n, count = len(ins), ins[0].numel()
    sbytes = mrr.mrr_packet_scratch_bytes(count, t, n)
    scratch = torch.zeros(sbytes // 8, dtype=torch.int64, device="cuda")
    flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    assert mrr.mrr_allreduce_packet(ins, outs, scratch, sbytes, flags, count, t, acc, n, SPINS,
                                    err) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return outs


def no_alloc(ins, t, acc):
    n, count = len(ins), ins[0].numel()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = [empty(t, count, 0xDD) for _ in range(n)]
    st = mrr.mrr_allreduce_packet_noalloc(ins, outs, count, t, acc, n, SPINS, err)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "device error word %d" % err.item()
    return outs


def check(n, t, acc, count, seed, what):
    announce("packet no-alloc", what, n, t, acc, count)
    kind = "uniform" if t in ("f32", "f16", "bf16") else None
    ins = inputs_for(t, n, count, seed0=seed, kind=kind)
    copies = [x.clone() for x in ins]
    got = no_alloc(ins, t, acc)
    ref = with_own_buffers(ins, t, acc)
    want = oracle.allreduce([bits(x) for x in copies], t, acc)
    for k in range(n):
        assert torch.equal(got[k].view(torch.uint8), ref[k].view(torch.uint8)), \
            "%s: output %d differs from mrr_allreduce_packet" % (what, k)
        assert_bits_equal(bits(got[k]), want, t, "%s out[%d]" % (what, k))
        assert torch.equal(ins[k].view(torch.uint8), copies[k].view(torch.uint8)), \
            "%s: input %d was written" % (what, k)


def test_two_calls_second_smaller():
    """Two calls in a row on the shared workspace, the second smaller, each
    against the caller-owned entry point."""
    check(8, "f16", "f32", 128 * KiB // 2, 11, "first (128 KiB per rank)")
    check(8, "f16", "f32", 4 * KiB // 2 + 3, 12, "second (4 KiB + 6 B per rank)")


def test_calls_change_rank_count_type_and_size():
    """One flag sequence across rank counts: a call at N sets the flag slots
    of all 32 ranks, so a later call at a larger N finds them equal."""
    cases = [(4, "bf16", "f32", 20000), (32, "f32", "f32", 4096), (2, "fp8", "f16", 1 << 20),
             (16, "f16", "f16", 7001), (8, "fp8fn", "f32", 65536), (32, "bf16", "bf16", 8192),
             (8, "f16", "f32", 5), (2, "f32", "f32", 1)]
    for i, (n, t, acc, count) in enumerate(cases):
        check(n, t, acc, count, 100 + i, "sequence step %d" % i)


def test_largest_size_and_refusal():
    """The largest call that fits the workspace runs; one element more is
    refused with MRR_ESCRATCH and launches nothing."""
    n, t = 8, "f16"
    cap = mrr.MRR_NOALLOC_SCRATCH_BYTES
    count = cap // (n * n * 8) * 4 // ESZ[t]  # packets of 4 payload bytes
    assert mrr.mrr_packet_scratch_bytes(count, t, n) == cap
    check(n, t, "f32", count, 300, "largest")
    ins = inputs_for(t, n, count + 2, seed0=301, kind="uniform")
    outs = [empty(t, count + 2, 0x11) for _ in range(n)]
    st = mrr.mrr_allreduce_packet_noalloc(ins, outs, count + 2, t, "f32", n, SPINS, None)
    assert st == mrr.MRR_ESCRATCH
    torch.cuda.synchronize()
    assert all(bool((o.view(torch.uint8) == 0x11).all()) for o in outs), "refused call wrote"
    check(n, t, "f32", 1000, 302, "after a refused call")
