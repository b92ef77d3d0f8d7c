"""GPU parity of OCP FP8 E4M3FN inputs (bias 7, largest finite 448, no
infinity, S.1111.111 NaN) on every allreduce path -- the RS/AG kernels for
compiled and runtime rank counts, the allpair and two-phase packet variants --
against the CPU oracle, bit-exact, including NaN inputs, saturation at +-448
and signed zeros."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import (announce, assert_bits_equal, assert_outputs_match, bits, empty, inputs_for,
                        oracle_allreduce_threaded)

pytestmark = pytest.mark.gpu

T = "fp8fn"
SPINS = 2_000_000
ACC_OUT = [("f32", "fp8fn"), ("f32", "f16"), ("f32", "f32"), ("f16", "fp8fn"), ("f16", "f16"),
           ("f16", "f32"), ("fp8fn", "fp8fn"), ("fp8fn", "f16"), ("fp8fn", "f32")]
OUT_TORCH = {"fp8fn": torch.uint8, "f16": torch.float16, "f32": torch.float32}


def out_buf(t, count):
    x = torch.empty(count, dtype=OUT_TORCH[t], device="cuda")
    x.view(torch.uint8).fill_(0xA5)
    return x


def with_specials(ins, seed):
    """Plants NaN codes, the saturating extremes +-448, signed zeros and the
    smallest subnormals at random positions of every rank."""
    rng = np.random.default_rng(seed)
    special = np.array([0x7F, 0xFF, 0x7E, 0xFE, 0x00, 0x80, 0x01, 0x81], np.uint8)
    out = []
    for x in ins:
        h = x.cpu().numpy().copy()
        pos = rng.integers(0, h.size, max(1, h.size // 50))
        h[pos] = rng.choice(special, pos.size)
        out.append(torch.from_numpy(h).cuda())
    return out


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("acc,tout", ACC_OUT, ids=["-".join(x) for x in ACC_OUT])
def test_rsag_fn(n, acc, tout):
    count = 3 * 64 * 16 * n + 13  # several tiles per chunk and a ragged tail
    announce("fn rsag", n, acc, tout, count)
    ins = inputs_for(T, n, count, seed0=7000 + n)
    outs = [out_buf(tout, count) for _ in range(n)]
    assert mrr.mrr_allreduce_rsag_ex(ins, outs, count, T, acc, tout, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], T, acc, tout)
    for k, o in enumerate(outs):
        assert_bits_equal(bits(o), want, tout, "n=%d out[%d]" % (n, k))


@pytest.mark.parametrize("n", [2, 8, 32])
@pytest.mark.parametrize("acc,tout", ACC_OUT, ids=["-".join(x) for x in ACC_OUT])
def test_rsag_fn_specials(n, acc, tout):
    count = 2 * 64 * 16 * n + 5
    announce("fn rsag specials", n, acc, tout, count)
    ins = with_specials(inputs_for(T, n, count, seed0=7100 + n), seed=n)
    outs = [out_buf(tout, count) for _ in range(n)]
    assert mrr.mrr_allreduce_rsag_ex(ins, outs, count, T, acc, tout, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], T, acc, tout)
    for k, o in enumerate(outs):
        assert_bits_equal(bits(o), want, tout, "n=%d out[%d]" % (n, k))


def test_rsag_fn_unaligned_buffers():
    """Buffers off 16-byte alignment take the element-wise kernel."""
    n, count = 4, 5003
    announce("fn rsag unaligned")
    base = [x for x in inputs_for(T, n, count + 3, seed0=7200)]
    ins = [x[3:] for x in base]
    outs = [out_buf("fp8fn", count + 1)[1:] for _ in range(n)]
    assert mrr.mrr_allreduce_rsag_ex(ins, outs, count, T, "f32", T, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], T, "f32", T)
    for k, o in enumerate(outs):
        assert_bits_equal(bits(o), want, T, "out[%d]" % k)


@pytest.mark.parametrize("tout", [T, "f32"])
def test_rsag_fn_full_size_whole(tout):
    """8 ranks x 64 MiB of E4M3FN, f32 accumulation, pooled layout; E4M3FN
    outputs, and f32 outputs (the 128-lane-tile kernel).  A sampled pre-check,
    then every element of every output against the oracle (host threads)."""
    n, count = 8, 64 << 20
    announce("fn rsag 8 x 64 MiB ->", tout)
    pool_in, ins = mrr.alloc_rank_buffers(n, count, T)
    for r, x in enumerate(inputs_for(T, n, count, seed0=7300, device="cuda")):
        ins[r].copy_(x)
    pool_out, outs = mrr.alloc_rank_buffers(n, count, tout)
    assert mrr.mrr_allreduce_rsag_ex(ins, outs, count, T, "f32", tout, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.unique(np.concatenate([
        np.random.default_rng(8).integers(0, count, 1 << 17), [0, count - 1]]))).cuda()
    want = oracle.allreduce([bits(x[idx]) for x in ins], T, "f32", tout)
    for k in range(n):
        assert_bits_equal(bits(outs[k][idx]), want, tout, "out[%d] sampled" % k)
    want = oracle_allreduce_threaded([bits(x) for x in ins], T, "f32", tout)
    assert_outputs_match(outs, want, tout, "8 x 64 MiB -> %s whole" % tout)


@pytest.mark.parametrize("n", [3, 5, 12, 31])
@pytest.mark.parametrize("acc", ["f32", "fp8fn"])
def test_dispatch_runtime_rank_count_fn(n, acc):
    count = 3 * 64 * 16 * n + 9
    announce("fn dispatch runtime-N", n, acc)
    ins = with_specials(inputs_for(T, n, count, seed0=7400 + n), seed=100 + n)
    outs = [out_buf(T, count) for _ in range(n)]
    assert mrr.mrr_allreduce(ins, outs, count, T, acc, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], T, acc, T)
    for k, o in enumerate(outs):
        assert_bits_equal(bits(o), want, T, "n=%d out[%d]" % (n, k))


def _packet_state(nbytes_scratch, n):
    scratch = torch.zeros(max(nbytes_scratch, 8) // 8, dtype=torch.int64, device="cuda")
    flags = torch.zeros(n * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    return scratch, flags, err


@pytest.mark.parametrize("n", [2, 8, 32])
@pytest.mark.parametrize("acc", ["f32", "f16", "fp8fn"])
def test_packet_allpair_fn(n, acc):
    count = 4099
    announce("fn packet allpair", n, acc)
    sbytes = mrr.mrr_packet_scratch_bytes(count, T, n)
    scratch, flags, err = _packet_state(sbytes, n)
    outs = [out_buf(T, count) for _ in range(n)]
    for flag in (1, 2, 3):
        ins = with_specials(inputs_for(T, n, count, seed0=7500 + 10 * flag + n), seed=flag)
        copies = [x.clone() for x in ins]
        st = mrr.mrr_allreduce_packet(ins, outs, scratch, sbytes, flags, count, T, acc, n, SPINS,
                                      err)
        assert st == mrr.MRR_OK
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        want_scratch, want = oracle.allreduce_packet([bits(x) for x in copies], T, acc, flag)
        for k in range(n):
            assert_bits_equal(bits(outs[k]), want, T, "flag %d out[%d]" % (flag, k))
        assert np.all(flags.cpu().numpy().view(np.uint32) == flag)


@pytest.mark.parametrize("n", [2, 8, 16])
@pytest.mark.parametrize("acc", ["f32", "fp8fn"])
def test_packet_rsag_fn(n, acc):
    count = 96 * 1024 + 7
    announce("fn packet rsag", n, acc)
    sbytes = mrr.mrr_packet_rsag_scratch_bytes(count, T, n)
    scratch, flags, err = _packet_state(sbytes, n)
    outs = [out_buf(T, count) for _ in range(n)]
    for flag in (1, 2):
        ins = with_specials(inputs_for(T, n, count, seed0=7600 + 10 * flag + n), seed=50 + flag)
        copies = [x.clone() for x in ins]
        st = mrr.mrr_allreduce_packet_rsag(ins, outs, scratch, sbytes, flags, count, T, acc, n,
                                           SPINS, err)
        assert st == mrr.MRR_OK
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        _, _, want = oracle.allreduce_packet_rsag([bits(x) for x in copies], T, acc, flag)
        for k in range(n):
            assert_bits_equal(bits(outs[k]), want, T, "flag %d out[%d]" % (flag, k))


def test_packet_reduce_fn():
    n, npk = 8, 3001
    announce("fn packet reduce")
    ins = with_specials(inputs_for(T, n, npk * 4, seed0=7700), seed=7)
    pk = [torch.from_numpy(oracle.pack(bits(x), 41).view(np.int64)).cuda() for x in ins]
    out = torch.zeros(npk, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert mrr.mrr_packet_reduce(pk, out, npk, T, "f32", n, 41, 42, SPINS, err) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want = oracle.packet_reduce([p.cpu().numpy().view(np.uint64) for p in pk], T, "f32", 41, 42)
    got = out.cpu().numpy().view(np.uint64)
    assert np.array_equal(got >> np.uint64(32), want >> np.uint64(32))
    gp = (got & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.uint8)
    wp = (want & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.uint8)
    assert_bits_equal(gp, wp, T, "packet payload")
