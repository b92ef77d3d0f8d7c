"""Randomized differential parity (seeded): a few hundred calls drawn across
every allreduce entry point -- RS/AG (all chunks or one rank's share, in
place, element-wise path on unaligned buffers), the size-based dispatcher
(any rank count 1..32), the allpair and two-phase packet variants and the
full mesh, the
one-pass FP8 reduction and the codec -- with random rank counts, sizes
(weighted toward edges), types and accumulators, each compared bit for bit
with the CPU oracle.  Every case prints its parameters before it runs."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import SIZE, TORCH, announce, assert_bits_equal, bits, inputs_for

pytestmark = pytest.mark.gpu

COMPILED = [2, 4, 8, 16, 32]
TRIPLES = [("f32", "f32", "f32"), ("f16", "f32", "f16"), ("f16", "f16", "f16"),
           ("bf16", "f32", "bf16"), ("bf16", "bf16", "bf16")] + \
          [(t, a, o) for t in ("fp8", "fp8fn") for a in ("f32", "f16", t) for o in (t, "f16", "f32")]
PKT_PAIRS = [("f32", "f32"), ("f16", "f32"), ("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16"),
             ("fp8", "f32"), ("fp8", "f16"), ("fp8", "fp8"), ("fp8fn", "f32"), ("fp8fn", "f16"),
             ("fp8fn", "fp8fn")]
CASES = 150  # per entry-point family


def rand_count(rng, hi):
    r = rng.random()
    if r < 0.15:
        return int(rng.integers(0, 33))
    if r < 0.3:
        base = int(rng.choice([64, 128, 256, 512, 1024, 4096]))
        return max(0, base * int(rng.integers(1, 9)) + int(rng.integers(-3, 4)))
    return int(rng.integers(33, hi))


def empty_bytes(t, count, fill, offset=0):
    raw = torch.empty(count * SIZE[t] + offset + 16, dtype=torch.uint8, device="cuda")
    raw.fill_(fill)
    return raw[offset:offset + count * SIZE[t]].view(TORCH[t])


def kind_for(t):
    return "fp8codes" if t in ("fp8", "fp8fn") else "normal"


@pytest.mark.parametrize("case", range(CASES))
def test_random_rsag(case):
    rng = np.random.default_rng(10_000 + case)
    n = int(rng.choice(COMPILED))
    t, acc, tout = TRIPLES[int(rng.integers(len(TRIPLES)))]
    count = rand_count(rng, 40_000 // n + 64)
    rank = -1 if rng.random() < 0.7 else int(rng.integers(n))
    mode = rng.choice(["plain", "unaligned", "in_place"]) if SIZE[t] == SIZE[tout] else "plain"
    announce("random rsag", case, n, t, acc, tout, count, rank, mode)
    ins = inputs_for(t, n, count, seed0=20_000 + 37 * case, kind=kind_for(t))
    if mode == "unaligned":  # element-aligned, not 16-byte aligned
        off = SIZE[t] * int(rng.integers(1, 16 // SIZE[t])) if SIZE[t] < 16 else 0
        moved = []
        for x in ins:
            y = empty_bytes(t, count, 0, off)
            y.copy_(x)
            moved.append(y)
        ins = moved
        outs = [empty_bytes(tout, count, 0x5A, SIZE[tout]) for _ in range(n)]
    elif mode == "in_place":
        outs = ins
    else:
        outs = [empty_bytes(tout, count, 0x5A) for _ in range(n)]
    src = [bits(x) for x in ins]
    want = oracle.allreduce(src, t, acc, tout)
    st = mrr.mrr_allreduce_rsag_ex(ins, outs, count, t, acc, tout, n, rank)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    if rank < 0:
        lo, hi = 0, count
    else:
        gran = 256 // SIZE[t]
        per = -(-count // n)
        chunk = -(-per // gran) * gran
        lo, hi = min(rank * chunk, count), min((rank + 1) * chunk, count)
    for k in range(n):
        got = bits(outs[k])
        assert_bits_equal(got[lo:hi], want[lo:hi], tout, "case %d out[%d]" % (case, k))
        if mode != "in_place":
            rest = np.concatenate([got[:lo], got[hi:]]).view(np.uint8)
            assert np.all(rest == 0x5A), "case %d: out[%d] written outside its share" % (case, k)


@pytest.mark.parametrize("case", range(CASES))
def test_random_dispatch(case):
    rng = np.random.default_rng(30_000 + case)
    n = int(rng.integers(1, 33))
    same = [x for x in TRIPLES if x[0] == x[2]]
    t, acc, _ = same[int(rng.integers(len(same)))]
    count = rand_count(rng, 60_000 // n + 64)
    announce("random dispatch", case, n, t, acc, count)
    ins = inputs_for(t, n, count, seed0=40_000 + 31 * case, kind=kind_for(t))
    outs = [empty_bytes(t, count, 0x5A) for _ in range(n)]
    st = mrr.mrr_allreduce(ins, outs, count, t, acc, n)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], t, acc, t)
    for k in range(n):
        assert_bits_equal(bits(outs[k]), want, t, "case %d out[%d]" % (case, k))


@pytest.mark.parametrize("case", range(CASES))
def test_random_packets(case):
    rng = np.random.default_rng(50_000 + case)
    n = int(rng.choice(COMPILED))
    t, acc = PKT_PAIRS[int(rng.integers(len(PKT_PAIRS)))]
    algo = ["allpair", "two-phase", "fullmesh"][min(2, int(rng.random() * 3))]
    count = max(1, rand_count(rng, 20_000 // n + 64))
    calls = int(rng.integers(1, 4))
    announce("random packets", case, n, t, acc, count, algo, calls)
    size_fn = {"allpair": mrr.mrr_packet_scratch_bytes, "two-phase": mrr.mrr_packet_rsag_scratch_bytes,
               "fullmesh": mrr.mrr_fullmesh_scratch_bytes}[algo]
    sbytes = max(8, size_fn(count, t, n))
    scratch = torch.zeros(sbytes // 8 + 1, dtype=torch.int64, device="cuda")
    flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = [empty_bytes(t, count, 0x5A) for _ in range(n)]
    entry = {"allpair": mrr.mrr_allreduce_packet_ex, "two-phase": mrr.mrr_allreduce_packet_rsag,
             "fullmesh": mrr.mrr_allreduce_fullmesh}[algo]
    for call in range(calls):
        ins = inputs_for(t, n, count, seed0=60_000 + 97 * case + 7 * call, kind=kind_for(t))
        st = entry(ins, outs, scratch, sbytes, flags, count, t, acc, n, 2_000_000, err)
        assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, "case %d call %d: device time-out" % (case, call)
        want = oracle.allreduce([bits(x) for x in ins], t, acc, t)
        for k in range(n):
            assert_bits_equal(bits(outs[k]), want, t, "case %d call %d out[%d]" % (case, call, k))
        assert np.all(flags.cpu().numpy().view(np.uint32) == call + 1)


@pytest.mark.parametrize("case", range(CASES // 2))
def test_random_dual_and_codec(case):
    rng = np.random.default_rng(70_000 + case)
    n = int(rng.choice(COMPILED))
    t = "fp8" if rng.random() < 0.5 else "fp8fn"
    acc = ["f32", "f16", t][int(rng.integers(3))]
    count = rand_count(rng, 40_000 // n + 64)
    announce("random dual", case, n, t, acc, count)
    ins = inputs_for(t, n, count, seed0=80_000 + 13 * case, kind="fp8codes")
    o16 = [empty_bytes("f16", count, 0x5A) for _ in range(n)]
    o8 = [empty_bytes(t, count, 0x5A) for _ in range(n)]
    st = mrr.mrr_allreduce_rsag_dual(ins, o16, o8, count, t, acc, n)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    src = [bits(x) for x in ins]
    w16 = oracle.allreduce(src, t, acc, "f16")
    w8 = oracle.allreduce(src, t, acc, t)
    for k in range(n):
        assert_bits_equal(bits(o16[k]).view(np.uint16), w16, "f16", "case %d f16[%d]" % (case, k))
        assert_bits_equal(bits(o8[k]), w8, t, "case %d fp8[%d]" % (case, k))
    # codec on random bytes of random length and alignment
    m = rand_count(rng, 100_000)
    off = int(rng.integers(0, 4))
    announce("random codec", case, m, off)
    codes = torch.from_numpy(rng.integers(0, 256, m + off, dtype=np.uint8)).cuda()[off:]
    h = empty_bytes("f16", m, 0, 2 * off)
    assert mrr.mrr_fp8b15_to_f16(codes, h, m) == mrr.MRR_OK
    back = empty_bytes("fp8", m, 0, off)
    assert mrr.mrr_f16_to_fp8b15(h, back, m) == mrr.MRR_OK
    torch.cuda.synchronize()
    src = bits(codes)
    assert_bits_equal(bits(h).view(np.uint16), oracle.convert(src, "fp8", "f16"), "f16", "case %d dec" % case)
    assert_bits_equal(bits(back), oracle.convert(bits(h).view(np.uint16), "f16", "fp8"), "fp8",
                      "case %d enc" % case)
