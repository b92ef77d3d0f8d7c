"""GPU parity of the full-mesh allreduce (plain-data inboxes signalled by
semaphores) against the CPU oracle: outputs, the whole scratch image
(semaphores and inboxes, chained from call to call through the oracle alone),
flag slots and untouched inputs, over consecutive flags, every type pair and
rank count, ragged and near-empty chunk layouts, geometry changes, a flag
buffer and scratch shared with the allpair packet variant, in place, a
host-forced time-out and HIP graph replays.  Every wait is bounded by
max_spins, so a protocol fault ends in an error word, not a hang."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

SPINS = 2_000_000
KiB = 1 << 10
ESZ = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "fp8fn": 1}


def blocks_for(n, count, t):
    """An explicit blocks-per-rank choice: one 16-byte vector per lane of a
    256-lane workgroup (the default width), at most 512 workgroups in all
    (they all fit at once)."""
    chunk, _, _ = oracle.default().fullmesh_layout(count, t, n)
    cvec = chunk * ESZ[t] // 16
    return max(1, min(-(-cvec // 256), 512 // n, 1024))


class State:
    def __init__(self, n, count, t, flags=None, scratch_bytes=None):
        self.sbytes = scratch_bytes or mrr.mrr_fullmesh_scratch_bytes(count, t, n)
        self.scratch = torch.zeros(self.sbytes, dtype=torch.uint8, device="cuda")
        self.flags = flags if flags is not None else \
            torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.image = None  # the oracle's expected scratch image after the last call


def call(ins, outs, st, t, acc, spins=SPINS, blocks=0, threads=0, stream=None):
    n, count = len(ins), ins[0].numel()
    return mrr.mrr_allreduce_fullmesh(ins, outs, st.scratch, st.sbytes, st.flags, count, t, acc,
                                      n, spins, st.err, blocks, threads, stream=stream)


def check(ins, outs, st, t, acc, flag, copies, blocks, what):
    """Outputs and inputs; with blocks > 0 also the whole scratch image the
    oracle expects from the previous expected image."""
    n = len(ins)
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0, "%s: device error" % what
    host_ins = [bits(x) for x in copies]
    if blocks > 0:
        st.image, want = oracle.allreduce_fullmesh(host_ins, t, acc, flag, blocks, st.image)
        got = st.scratch.cpu().numpy()[:st.image.size]
        if not np.array_equal(got, st.image):
            bad = np.nonzero(got != st.image)[0]
            raise AssertionError("%s: scratch image differs at %d bytes, first %s" %
                                 (what, bad.size, bad[:6]))
    else:
        want = oracle.allreduce(host_ins, t, acc)
    for k in range(n):
        assert_bits_equal(bits(outs[k]), want, t, "%s out[%d]" % (what, k))
        assert torch.equal(ins[k].view(torch.uint8), copies[k].view(torch.uint8)), \
            "%s: input %d written" % (what, k)
    assert np.all(st.flags.cpu().numpy().view(np.uint32) == flag), what


@pytest.mark.parametrize("size", [16 * KiB, 64 * KiB, 256 * KiB, 1024 * KiB])
def test_eight_ranks_twenty_flags(size):
    n, t = 8, "f16"
    count = size // 2
    blocks = blocks_for(n, count, t)
    announce("fullmesh 8 ranks", size, "blocks", blocks)
    st = State(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in range(1, 21):
        ins = inputs_for(t, n, count, seed0=5000 * it, kind="uniform")
        copies = [x.clone() for x in ins]
        assert call(ins, outs, st, t, "f32", blocks=blocks) == mrr.MRR_OK
        check(ins, outs, st, t, "f32", it, copies, blocks, "size %d it %d" % (size, it))


PAIRS = [("f32", "f32"), ("f16", "f32"), ("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16"),
         ("fp8", "f32"), ("fp8", "f16"), ("fp8", "fp8"), ("fp8fn", "f32"), ("fp8fn", "f16"),
         ("fp8fn", "fp8fn")]


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("t,acc", PAIRS, ids=["-".join(p) for p in PAIRS])
def test_types_ragged(n, t, acc):
    count = {"f32": 3001, "f16": 4099, "bf16": 4099, "fp8": 8195, "fp8fn": 8195}[t]
    blocks = blocks_for(n, count, t)
    announce("fullmesh types", n, t, acc, "blocks", blocks)
    st = State(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in (1, 2):
        kind = "uniform" if t in ("f32", "f16", "bf16") else None
        ins = inputs_for(t, n, count, seed0=90 * it + n, kind=kind)
        copies = [x.clone() for x in ins]
        assert call(ins, outs, st, t, acc, blocks=blocks) == mrr.MRR_OK
        check(ins, outs, st, t, acc, it, copies, blocks, "n=%d %s/%s it %d" % (n, t, acc, it))


@pytest.mark.parametrize("count", [1, 3, 5, 9, 17, 100, 257])
def test_small_counts_leave_chunks_empty(count):
    n, t = 8, "f16"
    announce("fullmesh small", count)
    st = State(n, count, t)
    ins = inputs_for(t, n, count, seed0=count, kind="uniform")
    copies = [x.clone() for x in ins]
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    assert call(ins, outs, st, t, "f32", blocks=1) == mrr.MRR_OK
    check(ins, outs, st, t, "f32", 1, copies, 1, "count %d" % count)


def test_geometry_changes_between_calls():
    """Blocks per rank and workgroup width change from call to call on one
    scratch; slots of blocks a call does not use keep their older flags."""
    n, t, count = 8, "bf16", 30000
    st = State(n, count, t)
    outs = [empty(t, count) for _ in range(n)]
    for it, (b, th) in enumerate([(3, 64), (1, 128), (40, 64), (7, 512), (2, 256)], start=1):
        announce("fullmesh geometry", b, th)
        ins = inputs_for(t, n, count, seed0=40 + it, kind="uniform")
        copies = [x.clone() for x in ins]
        assert call(ins, outs, st, t, "f32", blocks=b, threads=th) == mrr.MRR_OK
        check(ins, outs, st, t, "f32", it, copies, b, "geometry %s" % ((b, th),))


@pytest.mark.parametrize("n,t,count", [(8, "f16", 1 << 20), (32, "bf16", 65536 + 24),
                                       (2, "fp8", 5 << 20)])
def test_auto_geometry(n, t, count):
    announce("fullmesh auto geometry", n, t, count)
    st = State(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in (1, 2, 3):
        kind = "uniform" if t in ("f32", "f16", "bf16") else None
        ins = inputs_for(t, n, count, seed0=7 * it, kind=kind)
        copies = [x.clone() for x in ins]
        assert call(ins, outs, st, t, "f32") == mrr.MRR_OK
        check(ins, outs, st, t, "f32", it, copies, 0, "auto n=%d %s it %d" % (n, t, it))


def test_shares_flags_and_scratch_with_allpair():
    """One flag buffer and one scratch buffer serve the full-mesh and the
    allpair packet variants alternately: the packets the allpair calls leave
    in the scratch carry older flags, which no semaphore wait accepts."""
    n, t, count = 8, "f16", 20000
    size = max(mrr.mrr_fullmesh_scratch_bytes(count, t, n), mrr.mrr_packet_scratch_bytes(count, t, n))
    st = State(n, count, t, scratch_bytes=size)
    outs = [empty(t, count) for _ in range(n)]
    for it in range(1, 9):
        announce("fullmesh / allpair alternation", it)
        ins = inputs_for(t, n, count, seed0=600 + it, kind="uniform")
        copies = [x.clone() for x in ins]
        if it % 2:
            assert call(ins, outs, st, t, "f32") == mrr.MRR_OK
        else:
            assert mrr.mrr_allreduce_packet(ins, outs, st.scratch, size, st.flags, count, t, "f32",
                                            n, SPINS, st.err) == mrr.MRR_OK
        check(ins, outs, st, t, "f32", it, copies, 0, "alternation it %d" % it)


def test_in_place_matches_rsag():
    n, t, count = 8, "f16", 262144 + 3
    announce("fullmesh in place")
    ins = inputs_for(t, n, count, seed0=8, kind="uniform")
    ref = [empty(t, count) for _ in range(n)]
    assert mrr.mrr_allreduce_rsag(ins, ref, count, t, n) == mrr.MRR_OK
    st = State(n, count, t)
    assert call(ins, ins, st, t, "f32") == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0
    for k in range(n):
        assert torch.equal(ins[k].view(torch.int16), ref[k].view(torch.int16))


def test_four_mib_bf16_whole_outputs():
    n, t, count = 8, "bf16", 2 << 20
    announce("fullmesh 8 x 4 MiB bf16")
    ins = inputs_for(t, n, count, seed0=31)
    st = State(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    assert call(ins, outs, st, t, "f32") == mrr.MRR_OK
    check(ins, outs, st, t, "f32", 1, ins, 0, "8 x 4 MiB")


def test_stale_flags_time_out():
    """Rank 2's flag slots disagree with the others: every wait ends at
    max_spins with MRR_ETIMEDOUT in the error word, and the kernel finishes."""
    n, t, count = 4, "f16", 8192
    announce("fullmesh forced timeout")
    st = State(n, count, t)
    st.flags[2 * mrr.PKT_FLAG_SLOTS:3 * mrr.PKT_FLAG_SLOTS] = 9
    ins = inputs_for(t, n, count, seed0=1, kind="uniform")
    outs = [empty(t, count) for _ in range(n)]
    assert call(ins, outs, st, t, "f32", spins=200) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(st.err.item()) == mrr.MRR_ETIMEDOUT


def test_graph_replays():
    n, t, count = 8, "f16", 50000
    announce("fullmesh graph")
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
