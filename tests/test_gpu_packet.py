"""GPU parity of the LL-packet paths against the CPU oracle: allpair packet
allreduce (outputs, scratch contents, flag slots, inputs untouched) over 20
consecutive flags on one scratch, geometry changes between calls, the
receive-only packet reduce, pack/unpack, host-forced poll timeouts, and HIP
graph replays.  Every wait is bounded by max_spins, so a protocol fault ends
in an error word rather than a hang."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import TORCH, announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu

SPINS = 2_000_000  # generous bound for calls that must succeed
KiB = 1 << 10


class PacketState:
    """Scratch + flags + error word for one rank count and size."""

    def __init__(self, n, count, t):
        self.sbytes = mrr.mrr_packet_scratch_bytes(count, t, n)
        self.scratch = torch.zeros(self.sbytes // 8, dtype=torch.int64, device="cuda")
        self.flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")


def allpair(ins, outs, st, t, acc, spins=SPINS, blocks=0, threads=0, stream=None):
    n, count = len(ins), ins[0].numel()
    return mrr.mrr_allreduce_packet_ex(ins, outs, st.scratch, st.sbytes, st.flags, count, t, acc,
                                       n, spins, st.err, blocks, threads, stream=stream)


def check_call(ins, outs, st, t, acc, flag, in_copies, what):
    n = len(ins)
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0, "%s: device error %d" % (what, st.err.item())
    want_scratch, want = oracle.allreduce_packet([bits(x) for x in in_copies], t, acc, flag)
    for k in range(n):
        assert_bits_equal(bits(outs[k]), want, t, "%s out[%d]" % (what, k))
        assert torch.equal(ins[k].view(torch.uint8), in_copies[k].view(torch.uint8)), \
            "%s: input %d was written" % (what, k)
    sc = st.scratch.cpu().numpy().view(np.uint64).reshape(n, n, -1)
    npkt = want_scratch.shape[2]
    for d in range(n):
        for s in range(n):
            if d != s:
                assert np.array_equal(sc[d, s, :npkt], want_scratch[d, s]), \
                    "%s: scratch[%d][%d]" % (what, d, s)
    f = st.flags.cpu().numpy().view(np.uint32)
    assert np.all(f == flag), "%s: flag slots %s" % (what, np.unique(f))


@pytest.mark.parametrize("size", [16 * KiB, 64 * KiB, 256 * KiB, 1024 * KiB])
def test_allpair_eight_ranks_twenty_flags(size):
    """8 ranks, f16 ~U(-1,1); 20 calls on one scratch and flag buffer, the
    flag advancing 1..20; every call checked."""
    n, t = 8, "f16"
    count = size // 2
    announce("packet allpair 8 ranks", size)
    st = PacketState(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in range(1, 21):
        ins = inputs_for(t, n, count, seed0=1000 * it, kind="uniform")
        copies = [x.clone() for x in ins]
        assert allpair(ins, outs, st, t, "f32") == mrr.MRR_OK
        if it in (1, 2, 7, 20) or size <= 64 * KiB:
            check_call(ins, outs, st, t, "f32", it, copies, "size %d iter %d" % (size, it))
        else:
            torch.cuda.synchronize()
            assert int(st.err.item()) == 0
            assert np.all(st.flags.cpu().numpy().view(np.uint32) == it)


PAIRS = [("f32", "f32"), ("f16", "f32"), ("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16"),
         ("fp8", "f32"), ("fp8", "f16"), ("fp8", "fp8")]


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("t,acc", PAIRS, ids=["-".join(p) for p in PAIRS])
def test_allpair_types_ragged(n, t, acc):
    count = {"f32": 3001, "f16": 4099, "bf16": 4099, "fp8": 8195}[t]
    announce("packet allpair types", n, t, acc, count)
    st = PacketState(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in (1, 2):
        ins = inputs_for(t, n, count, seed0=7 * it + n, kind="fp8codes" if t == "fp8" else "uniform")
        copies = [x.clone() for x in ins]
        assert allpair(ins, outs, st, t, acc) == mrr.MRR_OK
        check_call(ins, outs, st, t, acc, it, copies, "n=%d %s/%s it %d" % (n, t, acc, it))


# The allpair kernel polls two packets per lane from 32768 packets per rank up
# (at most 8 ranks), one below: sizes on both sides of that switch, ragged
# past it, and 16 ranks at the same size (one per lane).
@pytest.mark.parametrize("n,npkt", [(2, 32767), (2, 32768), (4, 32768 + 129), (8, 32767),
                                    (8, 32768), (8, 65536 + 3), (16, 32768 + 1)])
@pytest.mark.parametrize("t,acc", [("f16", "f32"), ("fp8", "f16")])
def test_allpair_packets_per_lane_switch(n, npkt, t, acc):
    count = npkt * 4 // {"f16": 2, "fp8": 1}[t] - 1  # last word half (f16) or 3/4 (fp8) full
    announce("packet allpair batch switch", n, npkt, t, acc, count)
    st = PacketState(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for it in (1, 2):
        ins = inputs_for(t, n, count, seed0=11 * it + n, kind="fp8codes" if t == "fp8" else "uniform")
        copies = [x.clone() for x in ins]
        assert allpair(ins, outs, st, t, acc) == mrr.MRR_OK
        check_call(ins, outs, st, t, acc, it, copies, "n=%d npkt=%d %s it %d" % (n, npkt, t, it))


def test_geometry_changes_between_calls():
    """Blocks per rank and threads change every call; the shared flag slots
    keep every call consistent (no hang, flags advance by one per call)."""
    n, t, count = 8, "f16", 40000
    st = PacketState(n, count, t)
    outs = [empty(t, count) for _ in range(n)]
    geoms = [(1, 64), (3, 128), (64, 256), (7, 512), (0, 0), (200, 64), (1, 512), (16, 448)]
    for it, (b, th) in enumerate(geoms, start=1):
        announce("packet geometry", b, th)
        ins = inputs_for(t, n, count, seed0=50 + it, kind="uniform")
        copies = [x.clone() for x in ins]
        assert allpair(ins, outs, st, t, "f32", blocks=b, threads=th) == mrr.MRR_OK
        check_call(ins, outs, st, t, "f32", it, copies, "geometry %s" % ((b, th),))


def test_sizes_change_on_one_scratch():
    """One scratch sized for the largest call serves smaller and larger-count
    calls in any order (stale packets always carry older flags)."""
    n, t = 4, "bf16"
    big = 100000
    st = PacketState(n, big, t)
    for it, count in enumerate([big, 17, 5000, 1, big // 3, 4096], start=1):
        announce("packet size change", count)
        ins = inputs_for(t, n, count, seed0=it, kind="uniform")
        copies = [x.clone() for x in ins]
        outs = [empty(t, count) for _ in range(n)]
        assert allpair(ins, outs, st, t, "f32") == mrr.MRR_OK
        torch.cuda.synchronize()
        assert int(st.err.item()) == 0
        want = oracle.allreduce([bits(x) for x in copies], t, "f32")
        for k in range(n):
            assert_bits_equal(bits(outs[k]), want, t, "count %d out %d" % (count, k))
        assert np.all(st.flags.cpu().numpy().view(np.uint32) == it)


def test_packet_matches_rsag_bitwise():
    n, t, count = 8, "f16", 262144
    announce("packet == rsag")
    ins = inputs_for(t, n, count, seed0=31, kind="uniform")
    st = PacketState(n, count, t)
    a = [empty(t, count) for _ in range(n)]
    b = [empty(t, count) for _ in range(n)]
    assert allpair(ins, a, st, t, "f32") == mrr.MRR_OK
    assert mrr.mrr_allreduce_rsag(ins, b, count, t, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    for k in range(n):
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))


def test_in_place_allpair():
    n, t, count = 4, "f32", 10001
    announce("packet in place")
    ins = inputs_for(t, n, count, seed0=3, kind="uniform")
    want = oracle.allreduce([bits(x) for x in ins], t, "f32")
    st = PacketState(n, count, t)
    assert allpair(ins, ins, st, t, "f32") == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0
    for k in range(n):
        assert_bits_equal(bits(ins[k]), want, t, "in place %d" % k)


def test_allpair_stale_flags_time_out():
    """Host-forced: rank 1's flag slots disagree with the others, so no
    receiver ever sees its flag; every wait ends at max_spins, the error word
    says MRR_ETIMEDOUT and the kernel completes."""
    n, t, count = 4, "f16", 8192
    announce("packet forced timeout (allpair)")
    st = PacketState(n, count, t)
    st.flags[mrr.PKT_FLAG_SLOTS:2 * mrr.PKT_FLAG_SLOTS] = 5
    ins = inputs_for(t, n, count, seed0=1, kind="uniform")
    outs = [empty(t, count) for _ in range(n)]
    assert allpair(ins, outs, st, t, "f32", spins=200) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(st.err.item()) == mrr.MRR_ETIMEDOUT


def packets_of(xs, t, flag):
    return [torch.from_numpy(oracle.pack(bits(x), flag).view(np.int64)).cuda() for x in xs]


@pytest.mark.parametrize("n", [2, 8, 32])
@pytest.mark.parametrize("t,acc", PAIRS, ids=["-".join(p) for p in PAIRS])
def test_packet_reduce_parity(n, t, acc):
    count = {"f32": 5001, "f16": 10002, "bf16": 10002, "fp8": 20004}[t]
    announce("packet reduce", n, t, acc)
    xs = inputs_for(t, n, count, seed0=n, kind="fp8codes" if t == "fp8" else "uniform")
    pk = packets_of(xs, t, 41)
    npk = pk[0].numel()
    out = torch.zeros(npk, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert mrr.mrr_packet_reduce(pk, out, npk, t, acc, n, 41, 42, SPINS, err) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want = oracle.packet_reduce([p.cpu().numpy().view(np.uint64) for p in pk], t, acc, 41, 42)
    got = out.cpu().numpy().view(np.uint64)
    assert np.all((got >> np.uint64(32)) == 42)
    pay = (got & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(oracle.NP_BITS[t] if t != "f32" else np.float32)
    wpay = (want & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(oracle.NP_BITS[t] if t != "f32" else np.float32)
    assert_bits_equal(pay, wpay, t, "packet reduce")


def test_packet_reduce_stale_packet_times_out():
    n, t = 4, "f16"
    announce("packet forced timeout (reduce)")
    xs = inputs_for(t, n, 4096, seed0=2, kind="uniform")
    pk = packets_of(xs, t, 9)
    bad = pk[2].cpu().numpy().view(np.uint64).copy()
    bad[100] = (bad[100] & np.uint64(0xFFFFFFFF)) | (np.uint64(8) << np.uint64(32))
    pk[2] = torch.from_numpy(bad.view(np.int64)).cuda()
    out = torch.zeros(pk[0].numel(), dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert mrr.mrr_packet_reduce(pk, out, pk[0].numel(), t, "f32", n, 9, 10, 100, err) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(err.item()) == mrr.MRR_ETIMEDOUT


@pytest.mark.parametrize("nbytes", [0, 1, 2, 3, 4, 5, 1023, 4096, 1 << 20, (1 << 20) + 3])
def test_pack_unpack(nbytes):
    announce("pack/unpack", nbytes)
    rng = np.random.default_rng(nbytes)
    src_np = rng.integers(0, 256, max(nbytes, 1), dtype=np.uint8)
    src = torch.from_numpy(src_np).cuda()
    npk = (nbytes + 3) // 4
    pk = torch.zeros(max(npk, 1), dtype=torch.int64, device="cuda")
    assert mrr.mrr_pack(src, pk, nbytes, 0xABCD1234) == mrr.MRR_OK
    back = torch.full((max(nbytes, 1),), 0x77, dtype=torch.uint8, device="cuda")
    assert mrr.mrr_unpack(pk, back, nbytes) == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.pack(src_np[:nbytes], 0xABCD1234)
    assert np.array_equal(pk.cpu().numpy().view(np.uint64)[:npk], want)
    assert np.array_equal(back.cpu().numpy()[:nbytes], src_np[:nbytes])


def test_allpair_graph_replays_advance_flags():
    """A captured allpair call replayed 5 times: the flag advances on the
    device each replay and every replay's outputs are correct."""
    n, t, count = 8, "f16", 65536
    announce("packet graph")
    st = PacketState(n, count, t)
    ins = inputs_for(t, n, count, seed0=12, kind="uniform")
    outs = [empty(t, count) for _ in range(n)]
    want = oracle.allreduce([bits(x) for x in ins], t, "f32")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert allpair(ins, outs, st, t, "f32", stream=s) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert np.all(st.flags.cpu().numpy() == 0)  # capture does not run the kernel
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


def test_flag_buffer_save_restore_and_recycle():
    """The caller-owned flag buffer is the packet protocol's only persistent
    state.  Saved to the host after three calls and restored into a fresh
    buffer (with fresh zeroed scratch), the next call continues at flag 4;
    a recycled buffer zeroed together with its scratch restarts at flag 1."""
    n, t, count = 8, "f16", 6001
    announce("packet flags save / restore")
    st = PacketState(n, count, t)
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for flag in (1, 2, 3):
        ins = inputs_for(t, n, count, seed0=4000 + flag, kind="uniform")
        copies = [x.clone() for x in ins]
        assert allpair(ins, outs, st, t, "f32") == mrr.MRR_OK
        check_call(ins, outs, st, t, "f32", flag, copies, "call %d" % flag)
    saved = st.flags.cpu().clone()
    fresh = PacketState(n, count, t)
    fresh.flags.copy_(saved.cuda())
    ins = inputs_for(t, n, count, seed0=4100, kind="uniform")
    copies = [x.clone() for x in ins]
    assert allpair(ins, outs, fresh, t, "f32") == mrr.MRR_OK
    check_call(ins, outs, fresh, t, "f32", 4, copies, "restored")
    fresh.flags.zero_()
    fresh.scratch.zero_()
    torch.cuda.synchronize()
    ins = inputs_for(t, n, count, seed0=4200, kind="uniform")
    copies = [x.clone() for x in ins]
    assert allpair(ins, outs, fresh, t, "f32") == mrr.MRR_OK
    check_call(ins, outs, fresh, t, "f32", 1, copies, "recycled")


def test_flag_wrap_skips_zero():
    """Flag slots preset near the top of the 32-bit range (scratch zeroed):
    the calls stamp 2^32 - 1 and then 1, skipping 0, and every output,
    scratch packet and flag slot is the oracle's -- the documented wrap, on
    a buffer re-zeroed as the wrap contract asks."""
    n, t, count = 4, "bf16", 5000
    announce("packet flag wrap")
    st = PacketState(n, count, t)
    st.flags.fill_(-2)  # every slot 0xFFFFFFFE
    outs = [empty(t, count, 0xEE) for _ in range(n)]
    for flag in (0xFFFFFFFF, 1, 2):
        ins = inputs_for(t, n, count, seed0=4300 + (flag & 0xFF), kind="uniform")
        copies = [x.clone() for x in ins]
        assert allpair(ins, outs, st, t, "f32") == mrr.MRR_OK
        check_call(ins, outs, st, t, "f32", flag, copies, "flag %#x" % flag)
