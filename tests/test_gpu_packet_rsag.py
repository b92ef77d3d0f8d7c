"""GPU parity of the two-phase (reduce-scatter + all-gather) packet allreduce
against the CPU oracle: outputs, both scratch regions, flag slots and
untouched inputs, over consecutive flags, every type pair and rank count,
ragged and near-empty chunk layouts, in place, a flag buffer shared with the
allpair variant, a host-forced time-out, and HIP graph replays."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

SPINS = 2_000_000
KiB = 1 << 10


class State:
    def __init__(self, n, count, t, flags=None):
        self.sbytes = max(mrr.mrr_packet_rsag_scratch_bytes(count, t, n), 8)
        self.scratch = torch.zeros(self.sbytes // 8, dtype=torch.int64, device="cuda")
        self.flags = flags if flags is not None else \
            torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")


def call(ins, outs, st, t, acc, spins=SPINS, blocks=0, threads=0, stream=None):
    n, count = len(ins), ins[0].numel()
    return mrr.mrr_allreduce_packet_rsag(ins, outs, st.scratch, st.sbytes, st.flags, count, t, acc,
                                         n, spins, st.err, blocks, threads, stream=stream)


def check(ins, outs, st, t, acc, flag, copies, what):
    n = len(ins)
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0, "%s: device error" % what
    rs, ag, want = oracle.allreduce_packet_rsag([bits(x) for x in copies], t, acc, flag)
    for k in range(n):
        assert_bits_equal(bits(outs[k]), want, t, "%s out[%d]" % (what, k))
        assert torch.equal(ins[k].view(torch.uint8), copies[k].view(torch.uint8)), \
            "%s: input %d written" % (what, k)
    cw = rs.shape[2]
    sc = st.scratch.cpu().numpy().view(np.uint64)[:2 * n * n * cw].reshape(2, n, n, cw)
    for d in range(n):
        for s in range(n):
            if d == s:
                continue
            written = rs[d, s] != 0
            assert np.array_equal(sc[0, d, s][written], rs[d, s][written]), "%s rs[%d][%d]" % (what, d, s)
            written = ag[d, s] != 0
            assert np.array_equal(sc[1, d, s][written], ag[d, s][written]), "%s ag[%d][%d]" % (what, d, s)
    assert np.all(st.flags.cpu().numpy().view(np.uint32) == flag), what


@pytest.mark.parametrize("size", [16 * KiB, 64 * KiB, 256 * KiB, 1024 * KiB])
def test_eight_ranks_twenty_flags(size):
    n, t = 8, "f16"
    count = size // 2
    announce("packet rsag 8 ranks", size)
    st = State(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in range(1, 21):
        ins = inputs_for(t, n, count, seed0=3000 * it, kind="uniform")
        copies = [x.clone() for x in ins]
        assert call(ins, outs, st, t, "f32") == mrr.MRR_OK
        if it in (1, 2, 13, 20) or size <= 64 * KiB:
            check(ins, outs, st, t, "f32", it, copies, "size %d it %d" % (size, it))
        else:
            torch.cuda.synchronize()
            assert int(st.err.item()) == 0


PAIRS = [("f32", "f32"), ("f16", "f32"), ("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16"),
         ("fp8", "f32"), ("fp8", "f16"), ("fp8", "fp8")]


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("t,acc", PAIRS, ids=["-".join(p) for p in PAIRS])
def test_types_ragged(n, t, acc):
    count = {"f32": 3001, "f16": 4099, "bf16": 4099, "fp8": 8195}[t]
    announce("packet rsag types", n, t, acc)
    st = State(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in (1, 2):
        ins = inputs_for(t, n, count, seed0=70 * it + n, kind="fp8codes" if t == "fp8" else "uniform")
        copies = [x.clone() for x in ins]
        assert call(ins, outs, st, t, acc) == mrr.MRR_OK
        check(ins, outs, st, t, acc, it, copies, "n=%d %s/%s" % (n, t, acc))


@pytest.mark.parametrize("count", [1, 3, 5, 9, 17, 100, 257])
def test_small_counts_leave_chunks_empty(count):
    n, t = 8, "f16"
    announce("packet rsag small", count)
    st = State(n, count, t)
    ins = inputs_for(t, n, count, seed0=count, kind="uniform")
    copies = [x.clone() for x in ins]
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    assert call(ins, outs, st, t, "f32") == mrr.MRR_OK
    check(ins, outs, st, t, "f32", 1, copies, "count %d" % count)


def test_geometry_and_shared_flags_with_allpair():
    """Geometry changes between calls, and the same flag buffer serves the
    allpair and the two-phase variant alternately."""
    n, t, count = 8, "bf16", 30000
    flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    st = State(n, count, t, flags)
    ap_bytes = mrr.mrr_packet_scratch_bytes(count, t, n)
    ap_scratch = torch.zeros(ap_bytes // 8, dtype=torch.int64, device="cuda")
    outs = [empty(t, count) for _ in range(n)]
    geoms = [(0, 0), (1, 64), (5, 192), (60, 64), (2, 512), (0, 128)]
    for it, (b, th) in enumerate(geoms, start=1):
        announce("packet rsag geometry", b, th)
        ins = inputs_for(t, n, count, seed0=it, kind="uniform")
        copies = [x.clone() for x in ins]
        if it % 2:
            assert call(ins, outs, st, t, "f32", blocks=b, threads=th) == mrr.MRR_OK
            check(ins, outs, st, t, "f32", it, copies, "rsag geometry %s" % ((b, th),))
        else:
            assert mrr.mrr_allreduce_packet_ex(ins, outs, ap_scratch, ap_bytes, flags, count, t, "f32",
                                               n, SPINS, st.err, b, th) == mrr.MRR_OK
            torch.cuda.synchronize()
            assert int(st.err.item()) == 0
            want = oracle.allreduce([bits(x) for x in copies], t, "f32")
            for k in range(n):
                assert_bits_equal(bits(outs[k]), want, t, "allpair out[%d]" % k)
            assert np.all(flags.cpu().numpy().view(np.uint32) == it)


def test_in_place_and_matches_rsag():
    n, t, count = 8, "f16", 262144 + 3
    announce("packet rsag in place")
    ins = inputs_for(t, n, count, seed0=8, kind="uniform")
    ref = [empty(t, count) for _ in range(n)]
    assert mrr.mrr_allreduce_rsag(ins, ref, count, t, n) == mrr.MRR_OK
    st = State(n, count, t)
    assert call(ins, ins, st, t, "f32") == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0
    for k in range(n):
        assert torch.equal(ins[k].view(torch.int16), ref[k].view(torch.int16))


def test_stale_flags_time_out():
    n, t, count = 4, "f16", 8192
    announce("packet rsag forced timeout")
    st = State(n, count, t)
    st.flags[2 * mrr.PKT_FLAG_SLOTS:3 * mrr.PKT_FLAG_SLOTS] = 9
    ins = inputs_for(t, n, count, seed0=1, kind="uniform")
    outs = [empty(t, count) for _ in range(n)]
    assert call(ins, outs, st, t, "f32", spins=200) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(st.err.item()) == mrr.MRR_ETIMEDOUT


def test_graph_replays():
    n, t, count = 8, "f16", 50000
    announce("packet rsag graph")
    st = State(n, count, t)
    ins = inputs_for(t, n, count, seed0=12, kind="uniform")
    outs = [empty(t, count) for _ in range(n)]
    want = oracle.allreduce([bits(x) for x in ins], t, "f32")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert call(ins, outs, st, t, "f32", stream=s) == mrr.MRR_OK
    torch.cuda.synchronize()
    for rep in range(1, 6):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.err.item()) == 0
        assert np.all(st.flags.cpu().numpy().view(np.uint32) == rep)
        for k in range(n):
            assert_bits_equal(bits(outs[k]), want, t, "replay %d out %d" % (rep, k))
