"""GPU parity of the RS/AG zero-copy reduction against the CPU oracle.

Every comparison is bit-exact (0 mismatches); NaN positions only need to be
NaN on both sides.  Small cases span several workgroup tiles per chunk and a
ragged tail; the full-size cases run the exact launch bench.py times."""
import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import (TORCH, announce, assert_bits_equal, assert_outputs_match, bits, empty,
                        inputs_for, oracle_allreduce_threaded)

pytestmark = pytest.mark.gpu

RANKS = [2, 4, 8, 16, 32]
TRIPLES = [("f32", "f32", "f32"), ("f16", "f32", "f16"), ("f16", "f16", "f16"),
           ("bf16", "f32", "bf16"), ("bf16", "bf16", "bf16"),
           ("fp8", "f32", "fp8"), ("fp8", "f32", "f16"), ("fp8", "f32", "f32"),
           ("fp8", "f16", "fp8"), ("fp8", "f16", "f16"), ("fp8", "f16", "f32"),
           ("fp8", "fp8", "fp8"), ("fp8", "fp8", "f16"), ("fp8", "fp8", "f32")]
VW = {"f32": 4, "f16": 8, "bf16": 8, "fp8": 16}
# RS/AG chunk granularity in elements: 256 bytes of input.
CHUNK_ALIGN = {"f32": 64, "f16": 128, "bf16": 128, "fp8": 256, "fp8fn": 256}


def run(ins, t, acc, tout, rank=-1, outs=None, fill=0xA5):
    n, count = len(ins), ins[0].numel()
    outs = outs if outs is not None else [empty(tout, count, fill) for _ in range(n)]
    st = mrr.mrr_allreduce_rsag_ex(ins, outs, count, t, acc, tout, n, rank)
    assert st == mrr.MRR_OK, mrr.mrr_status_string(st)
    torch.cuda.synchronize()
    return outs


def check_all(outs, want, tout, what):
    for k, o in enumerate(outs):
        assert_bits_equal(bits(o), want, tout, "%s out[%d]" % (what, k))


@pytest.mark.parametrize("n", RANKS)
@pytest.mark.parametrize("t,acc,tout", TRIPLES, ids=["-".join(x) for x in TRIPLES])
def test_parity_small(n, t, acc, tout):
    # several tiles of 256 lanes x up to 4 vectors per chunk, plus a ragged tail
    count = n * 3 * 256 * 2 * VW[t] + 13
    announce("rsag small", n, t, acc, tout, count)
    ins = inputs_for(t, n, count, seed0=10 * n)
    outs = run(ins, t, acc, tout)
    want = oracle.allreduce([bits(x) for x in ins], t, acc, tout)
    check_all(outs, want, tout, "n=%d %s/%s/%s" % (n, t, acc, tout))


# Calls whose compiled kernel would have fewer than 2 tiles per CU run the
# runtime-N kernel instead (N = 2 for 16/32-bit and FP8 data), so
# test_parity_small covers that route for them.  These sizes put the same
# rank counts well above that threshold (3x, on 256 CUs) so the compiled
# kernels, at the units per lane of their launch table, are covered too.
FN_TRIPLES = [("fp8fn", a, o) for a in ("f32", "f16", "fp8fn") for o in ("fp8fn", "f16", "f32")]
OUT_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "fp8fn": 1}


def table_unroll(n, t, tout):
    # units per lane of the compiled kernels' launch table (rsag.hip)
    if t in ("fp8", "fp8fn"):
        if n == 2:
            return 4 * {"f32": 4, "f16": 2}.get(tout, 1)
        if n == 4 and t == "fp8" and tout != "f32":
            return 2
        return 2 if tout == "f32" else 1
    return 2 if n == 2 else 1


VEC_CASES = [(n, t, a, o) for (t, a, o) in TRIPLES + FN_TRIPLES
             for n in ((2,) if t in ("fp8", "fp8fn") else (2, 4, 16))]


@pytest.mark.parametrize("n,t,acc,tout", VEC_CASES, ids=["%d-%s-%s-%s" % c for c in VEC_CASES])
def test_parity_compiled_kernel_sizes(n, t, acc, tout):
    u = table_unroll(n, t, tout)
    ue = 16 // OUT_SIZE[tout]
    count = n * 64 * u * (3 * 512 // n + 1) * ue + 13
    announce("rsag compiled-kernel size", n, t, acc, tout, count)
    ins = inputs_for(t, n, count, seed0=30 * n + 1)
    outs = run(ins, t, acc, tout)
    want = oracle.allreduce([bits(x) for x in ins], t, acc, tout)
    check_all(outs, want, tout, "n=%d %s/%s/%s" % (n, t, acc, tout))


# FP8 inputs to f32 outputs run a kernel of their own at most rank counts
# (16 codes per lane, stores transposed through LDS).  count = N (1024 m + 512)
# - 1000: from 4 ranks up every chunk is m whole 1024-element tiles and a half
# tile, and the last chunk is 1000 elements short, so its last tile is partial
# (33 of 64 lanes store), the tile after it starts past the buffer's last whole
# 16-element unit, and 8 elements form the scalar tail (2 ranks: chunks of
# 1024 m + 256, the last one 16 lanes into its last tile plus the same tail).
# m keeps N <= 8 well above the small-call switch, so the compiled kernels run.
WIDE_CASES = [(n, t, acc) for n in (2, 4, 8, 16, 32) for t in ("fp8", "fp8fn")
              for acc in ("f32", "f16", t)]


@pytest.mark.parametrize("n,t,acc", WIDE_CASES, ids=["%d-%s-%s" % c for c in WIDE_CASES])
def test_parity_fp8_to_f32_tiles(n, t, acc):
    m = {2: 2048, 4: 2048, 8: 512}.get(n, 16)
    count = n * (1024 * m + 512) - 1000
    per = -(-count // n)
    chunk = -(-per // CHUNK_ALIGN[t]) * CHUNK_ALIGN[t]
    announce("rsag fp8 -> f32 tiles", n, t, acc, count)
    ins = inputs_for(t, n, count, seed0=700 + n)
    host = [bits(x) for x in ins]
    want = oracle_allreduce_threaded(host, t, acc, "f32")
    check_all(run(ins, t, acc, "f32"), want, "f32", "n=%d %s/%s" % (n, t, acc))
    # The last rank's share alone: its chunk is the short one.
    r = n - 1
    outs = run(ins, t, acc, "f32", rank=r, fill=0x5A)
    lo = r * chunk
    for k, o in enumerate(outs):
        b = bits(o)
        assert_bits_equal(b[lo:], want[lo:], "f32", "rank %d out %d" % (r, k))
        assert np.all(b[:lo].view(np.uint8) == 0x5A), "rank %d wrote outside its chunk" % r


def plant_fp8_specials(ins, t, seed):
    """Every exponent-15 code of E4M3B15 (inf, NaN) or the NaNs and largest
    finite values of E4M3FN, signed zeros and the smallest subnormals, at
    1/64 of the positions of each rank."""
    rng = np.random.default_rng(seed)
    special = np.array(list(range(0x78, 0x80)) + list(range(0xF8, 0x100)) + [0x00, 0x80, 0x01, 0x81]
                       if t == "fp8" else [0x7F, 0xFF, 0x7E, 0xFE, 0x00, 0x80, 0x01, 0x81], np.uint8)
    out = []
    for x in ins:
        h = bits(x).copy()
        pos = rng.integers(0, h.size, max(1, h.size // 64))
        h[pos] = rng.choice(special, pos.size)
        out.append(torch.from_numpy(h).cuda())
    return out


# FP8 inputs holding inf / NaN codes at sizes that run the compiled kernels
# (the general kernel, the 16-codes-per-lane kernel for f32 outputs) and the
# runtime-N kernel well above the small-call switch: a unit holding such a
# code is reduced again with the exact decode, so this covers that path in
# every kernel, every output type and every accumulator.
SPECIAL_CASES = [(n, t, acc, o) for n in (2, 4, 8, 16, 32) for t in ("fp8", "fp8fn")
                 for acc in ("f32", "f16", t) for o in (t, "f16", "f32")] + \
                [(n, t, acc, t) for n in (3, 12) for t in ("fp8", "fp8fn") for acc in ("f32", "f16", t)]


@pytest.mark.parametrize("n,t,acc,tout", SPECIAL_CASES, ids=["%d-%s-%s-%s" % c for c in SPECIAL_CASES])
def test_fp8_special_codes_at_kernel_sizes(n, t, acc, tout):
    # 2 ranks: over 512 tiles of 4096 codes, above the small-call switch
    count = (1 << 21) + (1 << 16) + 1031 if n == 2 else (600 * 1024 + 7 if n <= 12 else n * 16896 - 1000)
    announce("rsag fp8 specials", n, t, acc, tout, count)
    ins = plant_fp8_specials(inputs_for(t, n, count, seed0=1300 + n), t, seed=n)
    if n in (2, 4, 8, 16, 32):
        outs = run(ins, t, acc, tout)
    else:
        outs = [empty(tout, count, 0xA5) for _ in range(n)]
        assert mrr.mrr_allreduce(ins, outs, count, t, acc, n) == mrr.MRR_OK
        torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], t, acc, tout)
    check_all(outs, want, tout, "specials n=%d %s/%s/%s" % (n, t, acc, tout))


@pytest.mark.parametrize("t", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("count", [1, 3, 7, 8, 9, 15, 16, 17, 31, 33, 127, 129, 4095, 4097])
def test_edge_counts(t, count):
    n = 8
    announce("rsag edge", t, count)
    ins = inputs_for(t, n, count, seed0=count)
    outs = run(ins, t, "f32", t)
    want = oracle.allreduce([bits(x) for x in ins], t, "f32", t)
    check_all(outs, want, t, "count=%d" % count)


def test_two_rank_bf16_one_mib():
    """2 ranks, 1 MiB of bf16 each (524288 elements) ~N(0,1), seeds 0 and 1."""
    announce("rsag 2x1MiB bf16")
    ins = inputs_for("bf16", 2, 524288, seed0=0)
    outs = [empty("bf16", 524288) for _ in range(2)]
    assert mrr.mrr_allreduce_rsag(ins, outs, 524288, "bf16", 2) == mrr.MRR_OK
    torch.cuda.synchronize()
    check_all(outs, oracle.allreduce([bits(x) for x in ins], "bf16", "f32"), "bf16", "2x1MiB")


@pytest.mark.parametrize("n,count", [(2, 2005), (8, 8005), (32, 32005), (32, 1000), (16, 100003)])
def test_rank_share_writes_only_its_chunk(n, count):
    """rank=r writes exactly chunk r (256-byte rounded widths; with 32 ranks
    of 1000 elements, ranks 8..31 own empty chunks and write nothing)."""
    t = "f16"
    announce("rsag rank share", n, count)
    ins = inputs_for(t, n, count, seed0=77)
    want = oracle.allreduce([bits(x) for x in ins], t, "f32", t)
    per = -(-count // n)
    chunk = -(-per // CHUNK_ALIGN[t]) * CHUNK_ALIGN[t]
    for r in range(n):
        outs = run(ins, t, "f32", t, rank=r, fill=0x5A)
        lo, hi = min(r * chunk, count), min((r + 1) * chunk, count)
        for k, o in enumerate(outs):
            b = bits(o)
            assert_bits_equal(b[lo:hi], want[lo:hi], t, "rank %d out %d" % (r, k))
            untouched = np.concatenate([b[:lo], b[hi:]]).view(np.uint8)
            assert np.all(untouched == 0x5A), "rank %d wrote outside its chunk" % r


@pytest.mark.parametrize("t", ["f16", "bf16", "f32", "fp8"])
def test_in_place(t):
    n, count = 8, 50021
    announce("rsag in place", t)
    ins = inputs_for(t, n, count, seed0=5)
    want = oracle.allreduce([bits(x) for x in ins], t, "f32", t)
    run(ins, t, "f32", t, outs=ins)
    check_all(ins, want, t, "in place")


def views_at_offsets(t, n, count, fill, step):
    # rank buffer r starts (r + 1) * step bytes into its own allocation:
    # 16-byte aligned (the vector kernels run) but off the 256-byte grid
    out = []
    for r in range(n):
        off = (r + 1) * step
        raw = torch.empty(count * OUT_SIZE[t] + off + 64, dtype=torch.uint8, device="cuda")
        raw.fill_(fill)
        out.append(raw[off:off + count * OUT_SIZE[t]].view(TORCH[t]))
    return out


# Shapes whose output stores are device-scope buffer stores (4, 16 and 32
# ranks of 16/32-bit data, FP8 to FP8 / f16 at 2, 8, 16 and 32 ranks, FP8 to
# f32 in the 128-lane and the wide kernel) and two with plain streaming
# stores (8 ranks of f16, 4 ranks of E4M3B15 at two units per lane).
OFFSET_CASES = [(4, "bf16", "f32", "bf16"), (16, "f16", "f32", "f16"), (32, "bf16", "f32", "bf16"),
                (16, "f32", "f32", "f32"), (2, "fp8", "f32", "fp8"), (8, "fp8fn", "f32", "f16"),
                (8, "fp8", "f32", "f32"), (16, "fp8", "f32", "f32"), (4, "fp8fn", "f32", "f32"),
                (32, "fp8", "f32", "f16"), (8, "f16", "f32", "f16"), (4, "fp8", "f32", "fp8")]


@pytest.mark.parametrize("n,t,acc,tout", OFFSET_CASES, ids=["%d-%s-%s-%s" % c for c in OFFSET_CASES])
@pytest.mark.parametrize("step", [16, 48])
def test_vector_kernels_at_16_byte_offsets(n, t, acc, tout, step):
    u = table_unroll(n, t, tout)
    ue = 16 // OUT_SIZE[tout]
    count = n * 64 * u * (3 * 512 // n + 1) * ue + 13
    announce("rsag 16-byte offsets", n, t, acc, tout, step, count)
    base = inputs_for(t, n, count, seed0=700 + n)
    ins = views_at_offsets(t, n, count, 0, step)
    for dst, src in zip(ins, base):
        dst.copy_(src)
    outs = views_at_offsets(tout, n, count, 0xA5, step + 16)
    run(ins, t, acc, tout, outs=outs)
    want = oracle.allreduce([bits(x) for x in base], t, acc, tout)
    check_all(outs, want, tout, "offset %d n=%d %s/%s/%s" % (step, n, t, acc, tout))


@pytest.mark.parametrize("t,off", [("f16", 1), ("bf16", 3), ("f32", 1), ("fp8", 5)])
def test_unaligned_buffers_use_elementwise_path(t, off):
    n, count = 4, 20000
    announce("rsag unaligned", t, off)
    base = inputs_for(t, n, count + off, seed0=9)
    ins = [x[off:] for x in base]
    outs = [empty(t, count + off)[off:] for _ in range(n)]
    run(ins, t, "f32", t, outs=outs)
    want = oracle.allreduce([bits(x) for x in ins], t, "f32", t)
    check_all(outs, want, t, "unaligned")


def test_special_values():
    n = 4
    # -0, +0, inf, -inf, NaN, subnormals, overflow, cancellation
    f16 = np.array([0x8000, 0x0000, 0x7C00, 0xFC00, 0x7E00, 0x0001, 0x03FF, 0x7BFF, 0x3C00,
                    0xBC00, 0x8001, 0x0200] * 37, np.uint16)
    rng = np.random.default_rng(3)
    cols = [np.roll(f16, s) if s else f16 for s in range(n)]
    cols[3] = rng.permutation(cols[3])
    for t in ("f16", "bf16"):
        announce("rsag special", t)
        ins = [torch.from_numpy(c.view(np.int16).copy()).view(TORCH[t]).cuda() for c in cols]
        for acc in ("f32", t):
            outs = run(ins, t, acc, t)
            check_all(outs, oracle.allreduce(cols, t, acc, t), t, "special %s/%s" % (t, acc))
    f32 = np.array([-0.0, 0.0, np.inf, -np.inf, np.nan, 1e-45, 3e38, 3e38, -1e-40, 1.0],
                   np.float32)
    cols = [np.roll(f32, s) for s in range(n)]
    ins = [torch.from_numpy(c.copy()).cuda() for c in cols]
    outs = run(ins, "f32", "f32", "f32")
    check_all(outs, oracle.allreduce(cols, "f32", "f32"), "f32", "special f32")
    codes = [np.arange(256, dtype=np.uint8)[np.random.default_rng(s).permutation(256)]
             for s in range(n)]
    ins = [torch.from_numpy(c).cuda() for c in codes]
    for acc in ("f32", "f16", "fp8"):
        for tout in ("fp8", "f16", "f32"):
            outs = run(ins, "fp8", acc, tout)
            check_all(outs, oracle.allreduce(codes, "fp8", acc, tout), tout,
                      "special fp8 %s/%s" % (acc, tout))


@pytest.mark.parametrize("t,tout", [("f16", "f16"), ("fp8", "fp8"), ("fp8", "f16")])
def test_pooled_rank_buffers(t, tout):
    """Rank buffers carved from one allocation at mrr_rank_buffer_pitch()."""
    n, count = 8, 3 * 65536 + 7
    announce("rsag pooled", t, tout)
    src = inputs_for(t, n, count, seed0=44)
    _, ins = mrr.alloc_rank_buffers(n, count, t)
    for d, x in zip(ins, src):
        d.copy_(x)
    _, outs = mrr.alloc_rank_buffers(n, count, tout)
    run(ins, t, "f32", tout, outs=outs)
    check_all(outs, oracle.allreduce([bits(x) for x in src], t, "f32", tout), tout, "pooled")


def test_rank_order_pin():
    """x_0 = 1, x_1..7 = 2^-24 in f32: only the sequential rank order gives 1.0."""
    announce("rsag order pin")
    count = 4096
    ins = [torch.full((count,), 1.0, device="cuda")] + \
          [torch.full((count,), 2.0 ** -24, device="cuda") for _ in range(7)]
    outs = run(ins, "f32", "f32", "f32")
    for o in outs:
        assert torch.all(o == 1.0).item()


def test_graph_replays_match_eager():
    n, count, t = 8, 1 << 20, "f16"
    announce("rsag graph")
    ins = inputs_for(t, n, count, seed0=21)
    eager = run(ins, t, "f32", t)
    outs = [empty(t, count, 0) for _ in range(n)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert mrr.mrr_allreduce_rsag(ins, outs, count, t, n, stream=s) == mrr.MRR_OK
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(n):
            assert torch.equal(outs[k], eager[k]), "replay %d out %d" % (rep, k)


# ---------------------------------------------------------------------------
# Full sizes, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

def sample_indices(count, n, vw, rng, k=1 << 18):
    per = -(-count // n)
    chunk = -(-per // vw) * vw
    edges = []
    for r in range(n + 1):
        for d in (-2, -1, 0, 1):
            i = r * chunk + d
            if 0 <= i < count:
                edges.append(i)
    idx = np.concatenate([rng.integers(0, count, k), np.array(edges + [count - 1], np.int64)])
    return torch.from_numpy(np.unique(idx)).cuda()


def test_full_size_eight_ranks_64mib_f16():
    """8 ranks x 64 MiB of f16 ~N(0,1): whole output 0 against the oracle, and
    all eight outputs identical."""
    n, count, t = 8, 64 * (1 << 20) // 2, "f16"
    announce("rsag 8x64MiB f16 full")
    ins = inputs_for(t, n, count, seed0=0)
    outs = [empty(t, count) for _ in range(n)]
    assert mrr.mrr_allreduce_rsag(ins, outs, count, t, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], t, "f32")
    assert_bits_equal(bits(outs[0]), want, t, "8x64MiB out[0]")
    for k in range(1, n):
        assert torch.equal(outs[k].view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("tout", ["f16", "fp8", "f32"])
def test_full_size_fp8_eight_ranks_32mib(tout):
    n, count = 8, 32 * (1 << 20)
    announce("rsag 8x32MiB fp8 ->", tout)
    ins = inputs_for("fp8", n, count, seed0=100)
    outs = [empty(tout, count) for _ in range(n)]
    st = mrr.mrr_allreduce_rsag_ex(ins, outs, count, "fp8", "f32", tout, n, -1)
    assert st == mrr.MRR_OK
    torch.cuda.synchronize()
    want = oracle.allreduce([bits(x) for x in ins], "fp8", "f32", tout)
    assert_bits_equal(bits(outs[0]), want, tout, "fp8 out[0]")
    for k in range(1, n):
        assert torch.equal(outs[k].view(torch.uint8), outs[0].view(torch.uint8))


@pytest.mark.parametrize("n", RANKS)
def test_rank_sweep_256mib_bf16_whole(n):
    """N x 256 MiB of bf16 ~N(0,1) (inputs drawn on the device): a sampled
    pre-check (chunk edges included), then every element of every output
    against the oracle, run over the whole inputs on host threads."""
    count, t = 256 * (1 << 20) // 2, "bf16"
    announce("rsag sweep 256MiB bf16 n=%d" % n)
    ins = inputs_for(t, n, count, seed0=1000, device="cuda")
    outs = [empty(t, count) for _ in range(n)]
    assert mrr.mrr_allreduce_rsag(ins, outs, count, t, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    idx = sample_indices(count, n, CHUNK_ALIGN[t], np.random.default_rng(n))
    want = oracle.allreduce([bits(x[idx]) for x in ins], t, "f32")
    for k in range(n):
        assert_bits_equal(bits(outs[k][idx]), want, t, "n=%d out[%d] sampled" % (n, k))
    host = [bits(x) for x in ins]
    del ins
    want = oracle_allreduce_threaded(host, t, "f32", t)
    del host
    assert_outputs_match(outs, want, t, "n=%d whole" % n)
    del outs
    torch.cuda.empty_cache()


# 8 ranks with at least 128 MiB of input per rank, and 2 ranks with at least
# 256 MiB, run a second instance of the compiled kernel (device-scope
# stores, fewer workgroups per CU).  Sizes just above those thresholds with
# a ragged tail, every element of every output, and one rank's share
# written only into its chunk.
LARGE_CASES = [(8, "f16", "f32", "f16", (64 << 20) + 4099), (8, "f32", "f32", "f32", (32 << 20) + 13),
               (8, "bf16", "bf16", "bf16", (64 << 20) + 1), (2, "f16", "f32", "f16", (128 << 20) + 4099),
               (2, "f32", "f32", "f32", (64 << 20) + 13)]


@pytest.mark.parametrize("n,t,acc,tout,count", LARGE_CASES, ids=["%d-%s-%s-%s" % c[:4] for c in LARGE_CASES])
def test_large_buffer_instances(n, t, acc, tout, count):
    announce("rsag large buffers", n, t, acc, tout, count)
    ins = inputs_for(t, n, count, seed0=1200 + n, device="cuda")
    outs = [empty(tout, count, 0xA5) for _ in range(n)]
    run(ins, t, acc, tout, outs=outs)
    host = [bits(x) for x in ins]
    want = oracle_allreduce_threaded(host, t, acc, tout)
    assert_outputs_match(outs, want, tout, "%d ranks large %s/%s/%s" % (n, t, acc, tout))
    # one rank's share: its chunk equals the oracle, everything else keeps the fill
    r = min(5, n - 1)
    share = [empty(tout, count, 0x5A) for _ in range(n)]
    run(ins, t, acc, tout, rank=r, outs=share)
    per = -(-count // n)
    chunk = -(-per // CHUNK_ALIGN[t]) * CHUNK_ALIGN[t]
    lo, hi = min(count, r * chunk), min(count, (r + 1) * chunk)
    for k in range(n):
        b = bits(share[k])
        assert_bits_equal(b[lo:hi], want[lo:hi], tout, "rank %d share out[%d]" % (r, k))
        untouched = np.concatenate([b[:lo], b[hi:]]).view(np.uint8)
        assert np.all(untouched == 0x5A), "rank %d wrote outside its chunk (out[%d])" % (r, k)
    del ins, outs, share, host
    torch.cuda.empty_cache()


# Launches of more tiles than MRR_MAX_GRID workgroups: each workgroup walks
# several tiles (the path calls above 2^24 tiles take), including partial
# tiles at chunk ends and the element tail (the mrr_env fixture sets the override).
WALK_CASES = [(2, "bf16", "f32", "bf16"), (8, "f16", "f32", "f16"), (16, "f32", "f32", "f32"),
              (32, "bf16", "f32", "bf16"), (8, "fp8", "f32", "fp8"), (8, "fp8fn", "f32", "f32"),
              (4, "fp8", "f32", "f16")]


@pytest.mark.parametrize("n,t,acc,tout", WALK_CASES, ids=["%d-%s-%s-%s" % c for c in WALK_CASES])
@pytest.mark.parametrize("grid", [1, 7, 300])
def test_parity_workgroups_walk_tiles(n, t, acc, tout, grid, mrr_env):
    count = n * 64 * 2 * (3 * 512 // n + 1) * (16 // OUT_SIZE[tout]) + 13
    announce("rsag tile walk", n, t, acc, tout, count, "grid", grid)
    ins = inputs_for(t, n, count, seed0=70 * n + grid)
    mrr_env("MRR_MAX_GRID", str(grid))
    outs = run(ins, t, acc, tout)
    for r in (0, n - 1):
        share = run(ins, t, acc, tout, rank=r, outs=[empty(tout, count, 0x5A) for _ in range(n)])
        chunk = -(-(-(-count // n)) // CHUNK_ALIGN[t]) * CHUNK_ALIGN[t]
        lo, hi = min(count, r * chunk), min(count, (r + 1) * chunk)
        want_share = oracle.allreduce([bits(x)[lo:hi] for x in ins], t, acc, tout)
        for k, o in enumerate(share):
            assert_bits_equal(bits(o)[lo:hi], want_share, tout, "rank %d share out[%d]" % (r, k))
            raw = o.view(torch.uint8).cpu().numpy()
            esz = OUT_SIZE[tout]
            assert np.all(raw[:lo * esz] == 0x5A) and np.all(raw[hi * esz:] == 0x5A), \
                "rank %d share wrote outside its chunk" % r
    mrr_env("MRR_MAX_GRID", None)
    want = oracle.allreduce([bits(x) for x in ins], t, acc, tout)
    check_all(outs, want, tout, "walk n=%d %s/%s/%s grid %d" % (n, t, acc, tout, grid))


@pytest.mark.parametrize("n,t,acc,tout", WALK_CASES, ids=["%d-%s-%s-%s" % c for c in WALK_CASES])
def test_parity_persistent_grid(n, t, acc, tout, mrr_env):
    """MRR_LDS_CAP=0 (re-read through mrr_reload_env): no LDS reservation, a persistent grid of
    the table's workgroups per CU striding over the tiles."""
    count = n * 64 * 2 * (3 * 512 // n + 1) * (16 // OUT_SIZE[tout]) + 13
    announce("rsag persistent grid", n, t, acc, tout, count)
    ins = inputs_for(t, n, count, seed0=90 * n + 1)
    mrr_env("MRR_LDS_CAP", "0")
    outs = run(ins, t, acc, tout)
    mrr_env("MRR_LDS_CAP", None)
    want = oracle.allreduce([bits(x) for x in ins], t, acc, tout)
    check_all(outs, want, tout, "persistent n=%d %s/%s/%s" % (n, t, acc, tout))
