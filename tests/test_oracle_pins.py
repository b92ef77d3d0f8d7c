"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- values the pages state, library routines (numpy / torch CPU casts and
adds), exact integer arithmetic, closed forms and brute force over every input
of a small format.  A plausible slip anywhere in the oracle (a dropped term, a
wrong sign, exponent or bias, a reversed rank order, a wrong tie rule, a moved
packet flag) fails at least one of these.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    facts = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            facts[k] = v
    return facts


# ---------------------------------------------------------------------------
# Independent helpers (numpy / torch library routines, no oracle code)
# ---------------------------------------------------------------------------

def np_f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16)


def fp8_values_via_f16():
    """FP8 E4M3B15 values by the route the pages name: place the code's
    exponent and mantissa into an fp16's fields (same bias, 15) and let numpy
    decode the fp16.  Exponent field 15 is inf (m = 0) or NaN (m != 0)."""
    c = np.arange(256, dtype=np.uint16)
    h = ((c & 0x80) << 8) | ((c & 0x7F) << 7)
    v = np_f16(h).astype(np.float64)
    e15 = (c & 0x78) == 0x78
    m = c & 7
    sign = np.where(c & 0x80, -1.0, 1.0)
    v = np.where(e15 & (m == 0), sign * np.inf, v)
    v = np.where(e15 & (m != 0), np.nan, v)
    return v


FP8_VALUES = fp8_values_via_f16()
FP8_MAGS = FP8_VALUES[:0x78]  # codes 0x00..0x77, the finite non-negative ones


def brute_fp8_encode(x):
    """Nearest finite FP8 E4M3B15 value by exhaustive search over all 120
    magnitudes, ties to the even code; NaN -> 0x7F|s; +-inf saturate.

    Distances are float64 differences.  Wherever x is close enough to a
    midpoint for the choice to depend on rounding (2^-18 <= |x| <= 2) x has
    an ulp of at least 2^-41, so those differences are exact."""
    x = np.asarray(x, dtype=np.float64).ravel()
    out = np.empty(x.size, dtype=np.uint8)
    for lo in range(0, x.size, 1 << 16):
        xs = x[lo:lo + (1 << 16)]
        a = np.abs(xs)
        # above 2 every distance keeps its order but float64 can no longer
        # resolve it; the nearest finite value there is the largest one anyway
        a_fin = np.where(np.isfinite(a), np.minimum(a, 2.0), 2.0)
        d = np.abs(a_fin[:, None] - FP8_MAGS[None, :])
        i = np.argmin(d, axis=1)
        nxt = np.minimum(i + 1, 0x77)
        tie = (nxt != i) & (d[np.arange(len(i)), nxt] == d[np.arange(len(i)), i])
        i = np.where(tie & (i % 2 == 1), nxt, i)
        code = i.astype(np.uint8) | np.where(np.signbit(xs), 0x80, 0).astype(np.uint8)
        nan_code = np.where(np.signbit(xs), 0x80, 0) | 0x7F
        out[lo:lo + len(xs)] = np.where(np.isnan(xs), nan_code, code).astype(np.uint8)
    return out


def torch_bf16_bits(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def torch_bf16_value(bits):
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def same_bits_or_both_nan(got_vals, want_vals):
    got_vals = np.asarray(got_vals, dtype=np.float64)
    want_vals = np.asarray(want_vals, dtype=np.float64)
    nan_ok = np.isnan(got_vals) == np.isnan(want_vals)
    eq = (got_vals == want_vals) & (np.signbit(got_vals) == np.signbit(want_vals))
    return bool(np.all(nan_ok & (eq | np.isnan(want_vals))))


def assert_codes_equal(got, want, is_nan=None):
    got = np.asarray(got)
    want = np.asarray(want)
    mask = np.ones(got.shape, bool) if is_nan is None else ~is_nan
    bad = np.nonzero((got != want) & mask)[0]
    assert bad.size == 0, "mismatch at %s: got %s want %s" % (
        bad[:5], got[bad[:5]], want[bad[:5]])


# ---------------------------------------------------------------------------
# Format facts from the pages
# ---------------------------------------------------------------------------

def test_fp8_format_facts_from_pages(orc):
    facts = read_golden("fp8_e4m3b15_format.txt")
    assert facts["exponent_bits"] == ["4"] and facts["mantissa_bits"] == ["3"]
    bias = int(facts["bias"][0])
    max_finite = float(facts["max_finite"][0])
    v = orc.widen_f64(np.arange(256, dtype=np.uint8), "fp8")
    finite = v[np.isfinite(v)]
    assert finite.max() == max_finite
    assert finite.min() == -max_finite
    # 240 finite codes; +0 and -0 coincide -> 239 distinct finite values
    assert np.isfinite(v).sum() == 240
    assert len(np.unique(finite)) == 239
    # the smallest normal is 2^(1 - bias); with bias 15 that is the f16 one too
    assert v[0x08] == 2.0 ** (1 - bias)
    assert v[0x01] == 2.0 ** (1 - bias) / 8


def test_fp8_decode_matches_fp16_route(orc):
    v = orc.widen_f64(np.arange(256, dtype=np.uint8), "fp8")
    assert same_bits_or_both_nan(v, FP8_VALUES)
    # e = 15: inf for m = 0, NaN otherwise (the reading that keeps 0.9375 max)
    assert v[0x78] == np.inf and v[0xF8] == -np.inf
    assert np.all(np.isnan(v[0x79:0x80])) and np.all(np.isnan(v[0xF9:0x100]))
    assert v[0x80] == 0.0 and np.signbit(v[0x80])


def test_fp8_decode_to_f16_and_f32_bits(orc):
    codes = np.arange(256, dtype=np.uint8)
    h = orc.convert(codes, "fp8", "f16")
    f = orc.convert(codes, "fp8", "f32")
    finite = np.isfinite(FP8_VALUES)
    want_h = (((codes.astype(np.uint16) & 0x80) << 8) | ((codes.astype(np.uint16) & 0x7F) << 7))
    assert_codes_equal(h[finite], want_h[finite])
    assert np.all(f[finite].astype(np.float64) == FP8_VALUES[finite])
    # NaN bits are canonical; inf keeps its sign
    assert h[0x78] == 0x7C00 and h[0xF8] == 0xFC00
    assert h[0x79] == 0x7E00 and h[0xF9] == 0xFE00
    assert f.view(np.uint32)[0x7A] == 0x7FC00000


def test_fp8_worked_values(orc):
    v = orc.widen_f64(np.array([0x01, 0x07, 0x08, 0x38, 0x70, 0x77, 0x80, 0xF7], np.uint8), "fp8")
    assert list(v) == [2.0 ** -17, 7 * 2.0 ** -17, 2.0 ** -14, 2.0 ** -8, 0.5, 0.9375, -0.0, -0.9375]


def test_fp8_encode_all_f16_inputs_brute_force(orc):
    h = np.arange(65536, dtype=np.uint16)
    got = orc.convert(h, "f16", "fp8")
    want = brute_fp8_encode(np_f16(h).astype(np.float64))
    assert_codes_equal(got, want)


def test_fp8_encode_ties_and_saturation(orc):
    x = np.array([0.53125, 0.59375, 2.0 ** -18, 3 * 2.0 ** -18, 1.0, 0.96875, 100.0,
                  -2.0 ** -20, np.inf, -np.inf, np.nan, -0.0], np.float64)
    got = orc.narrow_f64(x, "fp8")
    assert list(got) == [0x70, 0x72, 0x00, 0x02, 0x77, 0x77, 0x77, 0x80, 0x77, 0xF7, 0x7F, 0x80]


def test_fp8_encode_f32_midpoints_and_random(orc):
    mags = FP8_MAGS
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (mags[:-1] + mags[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(1234)
    rnd = rng.uniform(-1.1, 1.1, 100000).astype(np.float32)
    tiny = (rng.uniform(-1, 1, 20000) * 2.0 ** -12).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([mids, up, dn, -mids, -up, -dn, rnd, tiny, bits,
                        np.array([1e-45, -1e-45, 3.4e38, np.inf, -np.inf, 0, -0.0], np.float32)])
    got = orc.convert(x, "f32", "fp8")
    want = brute_fp8_encode(x.astype(np.float64))
    assert_codes_equal(got, want)


def test_fp8_roundtrip_and_monotone(orc):
    codes = np.array([c for c in range(256) if (c & 0x78) != 0x78], np.uint8)
    assert_codes_equal(orc.convert(orc.convert(codes, "fp8", "f32"), "f32", "fp8"), codes)
    assert_codes_equal(orc.convert(orc.convert(codes, "fp8", "f16"), "f16", "fp8"), codes)
    x = np.linspace(-1.2, 1.2, 200001)
    v = orc.widen_f64(orc.narrow_f64(x, "fp8"), "fp8")
    assert np.all(np.diff(v) >= 0)


# ---------------------------------------------------------------------------
# f16 / bf16 / f32 conversions against library casts
# ---------------------------------------------------------------------------

def test_f16_decode_all_codes(orc):
    h = np.arange(65536, dtype=np.uint16)
    assert same_bits_or_both_nan(orc.widen_f64(h, "f16"), np_f16(h).astype(np.float64))


def test_bf16_decode_all_codes(orc):
    b = np.arange(65536, dtype=np.uint16)
    assert same_bits_or_both_nan(orc.widen_f64(b, "bf16"), torch_bf16_value(b))


def test_f32_decode_random_bits(orc):
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    u[:6] = [0, 0x80000000, 1, 0x7F7FFFFF, 0x7F800000, 0xFF800000]
    assert same_bits_or_both_nan(orc.widen_f64(u.view(np.float32), "f32"),
                                 u.view(np.float32).astype(np.float64))


def _f16_midpoints():
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = np_f16(h).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2
    return np.concatenate([mids, [65520.0, 65519.99, 65520.01]])


def test_f16_narrow_from_f64_vs_numpy(orc):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        _f16_midpoints(), -_f16_midpoints(),
        rng.normal(0, 1, 1 << 20), rng.normal(0, 3e4, 1 << 18),
        rng.uniform(-1, 1, 1 << 18) * 2.0 ** -20,
        [np.inf, -np.inf, np.nan, 0.0, -0.0, 1e300, -1e-300]])
    got = orc.narrow_f64(x, "f16")
    want = x.astype(np.float16).view(np.uint16)
    assert_codes_equal(got, want, is_nan=np.isnan(x))
    assert np.all(np.isnan(np_f16(got[np.isnan(x)])))


def test_f16_narrow_from_f32_bits_vs_numpy(orc):
    rng = np.random.default_rng(12)
    u = rng.integers(0, 2 ** 32, 1 << 21, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    got = orc.convert(x, "f32", "f16")
    want = x.astype(np.float16).view(np.uint16)
    assert_codes_equal(got, want, is_nan=np.isnan(x))


def test_bf16_narrow_from_f32_vs_torch(orc):
    rng = np.random.default_rng(13)
    u = rng.integers(0, 2 ** 32, 1 << 21, dtype=np.uint64).astype(np.uint32)
    # exact bf16 midpoints (low half 0x8000) exercise the tie rule on both parities
    u[: 1 << 16] = (np.arange(1 << 16, dtype=np.uint32) << 16) | 0x8000
    x = u.view(np.float32)
    got = orc.convert(x, "f32", "bf16")
    want = torch_bf16_bits(x)
    assert_codes_equal(got, want, is_nan=np.isnan(x))
    assert np.all((got[np.isnan(x)] & 0x7FFF) > 0x7F80)


def test_f32_narrow_from_f64_vs_numpy(orc):
    rng = np.random.default_rng(14)
    x = np.concatenate([rng.normal(0, 1, 1 << 18), rng.normal(0, 1e38, 1 << 12),
                        rng.normal(0, 1e-40, 1 << 12), [1e300, -1e300, np.inf]])
    got = orc.narrow_f64(x, "f32")
    want = x.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# The reduction
# ---------------------------------------------------------------------------

def _randn_bits(t, n, seed):
    import synth
    return synth.to_bits_numpy(synth.normal(t, n, seed))


def test_two_rank_closed_form_bf16(orc):
    """N=2 with f32 accumulation: out = RNE_bf16(x0 + x1), the exact sum
    rounded once (f32 then bf16 is an innocuous double rounding)."""
    n = 524288
    x0, x1 = _randn_bits("bf16", n, 0), _randn_bits("bf16", n, 1)
    got = orc.allreduce([x0, x1], "bf16", "f32")
    exact = torch_bf16_value(x0) + torch_bf16_value(x1)  # exact in float64 for this data
    assert np.all(np.abs(exact) < 64)
    want = torch_bf16_bits(exact.astype(np.float32))
    assert_codes_equal(got, want)


def test_two_rank_closed_form_f16(orc):
    n = 524288
    x0, x1 = _randn_bits("f16", n, 0), _randn_bits("f16", n, 1)
    got = orc.allreduce([x0, x1], "f16", "f32")
    exact = np_f16(x0).astype(np.float64) + np_f16(x1).astype(np.float64)
    assert_codes_equal(got, exact.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("nranks", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("t,c", [("f32", -3.0), ("f16", 0.5), ("bf16", 1.25)])
def test_constant_buffers_sum_to_n_times_c(orc, nranks, t, c):
    x = torch.full((1000,), c, dtype={"f32": torch.float32, "f16": torch.float16,
                                      "bf16": torch.bfloat16}[t])
    import synth
    bits = synth.to_bits_numpy(x)
    outs = orc.allreduce_all([bits] * nranks, t, "f32")
    want = synth.to_bits_numpy(torch.full((1000,), nranks * c, dtype=x.dtype))
    for o in outs:
        assert np.array_equal(o.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("nranks", [2, 8, 32])
def test_constant_fp8_buffers(orc, nranks):
    c = np.full(64, 0x50, np.uint8)  # e=10, m=0: 2^-5 = 0.03125
    assert orc.widen_f64(c[:1], "fp8")[0] == 0.03125
    f16 = orc.allreduce([c] * nranks, "fp8", "f32", "f16")
    assert np.all(np_f16(f16) == nranks * 0.03125)
    f8 = orc.allreduce([c] * nranks, "fp8", "f32", "fp8")
    # 32 * 2^-5 = 1.0 lies above the largest finite value: saturates
    assert np.all(orc.widen_f64(f8, "fp8") == min(nranks * 0.03125, 0.9375))


def test_rank_order_pin_f32(orc):
    """x_0 = 1, x_1..7 = 2^-24: each add of 2^-24 to 1.0 is a tie that rounds
    back to 1.0, so only the sequential order 0..N-1 gives exactly 1.0."""
    n = 16
    xs = [np.full(n, 1.0, np.float32)] + [np.full(n, 2.0 ** -24, np.float32)] * 7
    got = orc.allreduce(xs, "f32", "f32")
    assert np.all(got.view(np.uint32) == 0x3F800000)
    # the pin discriminates: reversed order and a pairwise tree differ
    acc = np.float32(0)
    for x in reversed([np.float32(v[0]) for v in xs]):
        acc = np.float32(acc + x)
    assert acc != np.float32(1.0)
    pair = [np.float32(v[0]) for v in xs]
    while len(pair) > 1:
        pair = [np.float32(pair[i] + pair[i + 1]) for i in range(0, len(pair), 2)]
    assert pair[0] != np.float32(1.0)


def test_signed_zero_and_cancellation(orc):
    a = np.array([0.0, -0.0, 1.5, -2.0, -0.0], np.float32)
    b = np.array([-0.0, -0.0, -1.5, 2.0, 0.0], np.float32)
    got = orc.allreduce([a, b], "f32", "f32").view(np.uint32)
    assert list(got) == [0x00000000, 0x80000000, 0x00000000, 0x00000000, 0x00000000]
    h = np.array([0x8000, 0x8000], np.uint16)
    assert list(orc.allreduce([h, h, h, h], "f16", "f32")) == [0x8000, 0x8000]


def test_overflow_and_nan(orc):
    big = np.array([0x7BFF, 0xFBFF, 0x7E00, 0x7C00], np.uint16)  # 65504, -65504, NaN, inf
    got = orc.allreduce([big, big], "f16", "f32")
    assert list(got[:2]) == [0x7C00, 0xFC00]
    assert np.isnan(np_f16(got[2:3]))[0] and got[3] == 0x7C00
    inf_minus_inf = orc.allreduce([np.array([0x7C00], np.uint16), np.array([0xFC00], np.uint16)],
                                  "f16", "f32")
    assert np.isnan(np_f16(inf_minus_inf))[0]


@pytest.mark.parametrize("nranks", [4, 8])
def test_f32_sum_vs_numpy_sequential(orc, nranks):
    rng = np.random.default_rng(nranks)
    xs = [rng.normal(0, 1, 200000).astype(np.float32) for _ in range(nranks)]
    acc = xs[0].copy()
    for x in xs[1:]:
        acc = (acc + x).astype(np.float32)
    got = orc.allreduce(xs, "f32", "f32")
    assert np.array_equal(got.view(np.uint32), acc.view(np.uint32))


@pytest.mark.parametrize("nranks", [4, 8])
def test_f16_sum_vs_numpy(orc, nranks):
    xs = [_randn_bits("f16", 200000, 100 + r) for r in range(nranks)]
    acc32 = np_f16(xs[0]).astype(np.float32)
    for x in xs[1:]:
        acc32 = acc32 + np_f16(x).astype(np.float32)
    got = orc.allreduce(xs, "f16", "f32")
    assert_codes_equal(got, acc32.astype(np.float16).view(np.uint16))
    # native f16 accumulation: numpy's float16 add is correctly rounded
    acc16 = np_f16(xs[0]).copy()
    for x in xs[1:]:
        acc16 = (acc16 + np_f16(x)).astype(np.float16)
    assert_codes_equal(orc.allreduce(xs, "f16", "f16"), acc16.view(np.uint16))
    assert_codes_equal(orc.allreduce(xs, "f16", "auto"), acc16.view(np.uint16))


@pytest.mark.parametrize("nranks", [4, 8])
def test_bf16_sum_vs_torch(orc, nranks):
    import synth
    ts = [synth.normal("bf16", 200000, 200 + r) for r in range(nranks)]
    xs = [synth.to_bits_numpy(t) for t in ts]
    acc = ts[0].float()
    for t in ts[1:]:
        acc = acc + t.float()
    got = orc.allreduce(xs, "bf16", "f32")
    assert_codes_equal(got, synth.to_bits_numpy(acc.to(torch.bfloat16)))
    accb = ts[0].clone()
    for t in ts[1:]:
        accb = accb + t  # torch CPU bf16 add: float add, one RNE
    assert_codes_equal(orc.allreduce(xs, "bf16", "bf16"), synth.to_bits_numpy(accb))


def _fp8_codes(n, seed):
    import synth
    return synth.fp8_finite_codes(n, seed).numpy()


@pytest.mark.parametrize("nranks", [2, 8, 32])
def test_fp8_f32_accumulation_is_exact(orc, nranks):
    """Every finite FP8 E4M3B15 value is k * 2^-17 with |k| <= 122880, so a sum
    of <= 32 of them is exact in f32: the oracle's sum must equal the integer
    sum, and every output type is that exact value rounded once."""
    n = 100000
    xs = [_fp8_codes(n, 300 + r) for r in range(nranks)]
    k = sum(np.rint(FP8_VALUES[x] * 2.0 ** 17).astype(np.int64) for x in xs)
    exact = k.astype(np.float64) * 2.0 ** -17
    # IEEE round-to-nearest: a zero sum is -0 only when every term is -0
    all_neg_zero = np.logical_and.reduce([x == 0x80 for x in xs])
    exact = np.where(all_neg_zero, -0.0, exact)
    got32 = orc.allreduce(xs, "fp8", "f32", "f32")
    assert np.array_equal(got32.view(np.uint32), exact.astype(np.float32).view(np.uint32))
    got16 = orc.allreduce(xs, "fp8", "f32", "f16")
    assert_codes_equal(got16, exact.astype(np.float16).view(np.uint16))
    got8 = orc.allreduce(xs, "fp8", "f32", "fp8")
    assert_codes_equal(got8, brute_fp8_encode(exact))


def test_fp8_native_and_f16_accumulation(orc):
    n, nranks = 20000, 8
    xs = [_fp8_codes(n, 400 + r) for r in range(nranks)]
    acc = brute_fp8_encode(FP8_VALUES[xs[0]])
    for x in xs[1:]:
        acc = brute_fp8_encode(FP8_VALUES[acc] + FP8_VALUES[x])
    assert_codes_equal(orc.allreduce(xs, "fp8", "fp8", "fp8"), acc)
    assert_codes_equal(orc.allreduce(xs, "fp8", "auto", "fp8"), acc)
    acc16 = FP8_VALUES[xs[0]].astype(np.float16)
    for x in xs[1:]:
        acc16 = (acc16 + FP8_VALUES[x].astype(np.float16)).astype(np.float16)
    assert_codes_equal(orc.allreduce(xs, "fp8", "f16", "f16"), acc16.view(np.uint16))


def test_fp8_higher_precision_at_least_as_accurate(orc):
    """The pages claim higher-precision accumulation of FP8 data is at least
    as accurate as native FP8 accumulation.  With f32 accumulation the FP8
    output is the exact sum rounded once, so it wins element by element."""
    n, nranks = 50000, 8
    xs = [_fp8_codes(n, 500 + r) for r in range(nranks)]
    exact = sum(FP8_VALUES[x] for x in xs)
    err = {}
    for acc in ("f32", "f16", "fp8"):
        v = orc.widen_f64(orc.allreduce(xs, "fp8", acc, "fp8"), "fp8")
        err[acc] = np.abs(v - exact)
    assert np.all(err["f32"] <= err["fp8"])
    assert err["f32"].max() <= err["fp8"].max() and err["f16"].mean() <= err["fp8"].mean()


def test_all_outputs_identical(orc):
    xs = [_randn_bits("bf16", 4099, 600 + r) for r in range(8)]
    outs = orc.allreduce_all(xs, "bf16", "f32")
    assert len(outs) == 8
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ---------------------------------------------------------------------------
# LL packets
# ---------------------------------------------------------------------------

def test_pack_layout_worked_example(orc):
    """Payload in the low 32 bits (little-endian bytes), flag in the high 32."""
    pk = orc.pack(bytes([0, 1, 2, 3, 4, 5]), 7)
    assert [int(p) for p in pk] == [0x0000000703020100, 0x0000000700000504]
    h = np.array([0x1234, 0xABCD, 0x0F0F], np.uint16)  # f16 element 2k in the low half
    pk = orc.pack(h, 0xDEADBEEF)
    assert [int(p) for p in pk] == [0xDEADBEEFABCD1234, 0xDEADBEEF00000F0F]


def test_pack_unpack_roundtrip(orc):
    rng = np.random.default_rng(5)
    for nb in list(range(0, 34)) + [4096, 4097]:
        b = rng.integers(0, 256, nb, dtype=np.uint8)
        pk = orc.pack(b, 42)
        assert pk.size == (nb + 3) // 4
        assert np.all((pk >> np.uint64(32)) == 42)
        assert np.array_equal(orc.unpack(pk, nb), b)


def test_next_flag(orc):
    assert orc.next_flag(0) == 1 and orc.next_flag(5) == 6 and orc.next_flag(0xFFFFFFFF) == 1


def test_flag_sequence_wraps_past_zero(orc):
    """The flag a call stamps is one more than the slots hold and never 0 (0
    marks a slot no call has written): across the 32-bit wrap the sequence
    runs ..., 2^32 - 2, 2^32 - 1, 1, 2, ..., so it repeats every 2^32 - 1
    calls -- the period after which stale packets could carry a current
    flag again, which is why the flag buffer and scratch are re-zeroed before
    then."""
    seq, f = [], 0xFFFFFFFC
    for _ in range(5):
        f = orc.next_flag(f)
        seq.append(f)
    assert seq == [0xFFFFFFFD, 0xFFFFFFFE, 0xFFFFFFFF, 1, 2]
    # a packet stamped just after the wrap carries flag 1 in its high word
    pk = orc.pack(np.arange(8, dtype=np.uint8), orc.next_flag(0xFFFFFFFF))
    assert np.all((pk >> np.uint64(32)) == 1)


@pytest.mark.parametrize("t,count", [("f16", 1001), ("f32", 64), ("bf16", 7), ("fp8", 1023)])
def test_allreduce_packet_expectation(orc, t, count):
    nranks = 4
    import synth
    if t == "fp8":
        xs = [_fp8_codes(count, 700 + r) for r in range(nranks)]
    else:
        xs = [synth.to_bits_numpy(synth.uniform(t, count, 700 + r)) for r in range(nranks)]
    scratch, out = orc.allreduce_packet(xs, t, "f32", 9)
    for d in range(nranks):
        for s in range(nranks):
            if d != s:
                assert np.array_equal(scratch[d, s], orc.pack(xs[s], 9))
    assert np.array_equal(out, orc.allreduce(xs, t, "f32"))


def test_packet_reduce(orc):
    nranks, count = 8, 1000  # 500 words of f16
    import synth
    xs = [synth.to_bits_numpy(synth.uniform("f16", count, 800 + r)) for r in range(nranks)]
    pk = [orc.pack(x, 3) for x in xs]
    out = orc.packet_reduce(pk, "f16", "f32", 3, 4)
    assert np.all((out >> np.uint64(32)) == 4)
    assert np.array_equal(orc.unpack(out, 2 * count).view(np.uint16),
                          orc.allreduce(xs, "f16", "f32"))
    pk[3] = pk[3].copy()
    pk[3][17] = (pk[3][17] & np.uint64(0xFFFFFFFF)) | (np.uint64(2) << np.uint64(32))
    assert orc.packet_reduce(pk, "f16", "f32", 3, 4) is None


@pytest.mark.parametrize("t,count,nranks", [("f16", 1001, 4), ("fp8", 1023, 8), ("f32", 5, 8),
                                            ("bf16", 64, 2)])
def test_packet_rsag_expectation(orc, t, count, nranks):
    """Two-phase packet allreduce: chunk c of rank d's input goes to rank c
    (reduce-scatter), chunk c of the sum goes from rank c to everyone
    (all-gather).  Built here from numpy slicing and the pinned pack()."""
    import synth
    if t == "fp8":
        xs = [_fp8_codes(count, 750 + r) for r in range(nranks)]
    else:
        xs = [synth.to_bits_numpy(synth.uniform(t, count, 750 + r)) for r in range(nranks)]
    rs, ag, out = orc.allreduce_packet_rsag(xs, t, "f32", 5)
    assert np.array_equal(out, orc.allreduce(xs, t, "f32"))
    e = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[t]
    cw = rs.shape[2]
    chunk_bytes = cw * 4
    assert chunk_bytes % 16 == 0 and chunk_bytes >= -(-count // nranks) * e
    for c in range(nranks):
        lo = c * chunk_bytes
        for d in range(nranks):
            if c == d:
                assert not rs[c, d].any() and not ag[d, c].any()
                continue
            src = xs[d].view(np.uint8)[lo:lo + chunk_bytes]
            want = orc.pack(src, 5) if src.size else np.zeros(0, np.uint64)
            assert np.array_equal(rs[c, d, :want.size], want)
            assert not rs[c, d, want.size:].any()
            red = out.view(np.uint8)[lo:lo + chunk_bytes]
            want = orc.pack(red, 5) if red.size else np.zeros(0, np.uint64)
            assert np.array_equal(ag[d, c, :want.size], want)


@pytest.mark.parametrize("t,count,nranks,nblocks", [("f16", 1001, 4, 3), ("fp8", 1023, 8, 1),
                                                    ("f32", 5, 8, 2), ("bf16", 64, 2, 1024)])
def test_fullmesh_expectation(orc, t, count, nranks, nblocks):
    """Full-mesh allreduce: inbox [c][d] holds chunk c of rank d's input
    (c != d), semaphores [c][d][b < B] hold the flag in their high word, the
    rest of the image is untouched, and the output is the plain sum.  The
    expected image is rebuilt here from numpy slicing of the inputs."""
    import synth
    if t == "fp8":
        xs = [_fp8_codes(count, 760 + r) for r in range(nranks)]
    else:
        xs = [synth.to_bits_numpy(synth.uniform(t, count, 760 + r)) for r in range(nranks)]
    e = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[t]
    chunk, sem_b, box_b = orc.fullmesh_layout(count, t, nranks)
    assert chunk * e % 16 == 0 and chunk >= -(-count // nranks) and chunk * e - 16 < \
        -(-count // nranks) * e
    rng = np.random.default_rng(count)
    before = rng.integers(0, 256, sem_b + box_b, dtype=np.uint8)  # any prior scratch state
    img, out = orc.allreduce_fullmesh(xs, t, "f32", 0xABCD0123, nblocks, before)
    assert np.array_equal(out, orc.allreduce(xs, t, "f32"))
    want = before.copy()
    sem = want[:sem_b].view(np.uint64).reshape(nranks, nranks, 1024)
    box = want[sem_b:].reshape(nranks, nranks, chunk * e)
    for c in range(nranks):
        for d in range(nranks):
            if c == d:
                continue
            sem[c, d, :nblocks] = np.uint64(0xABCD0123) << np.uint64(32)
            part = xs[d].view(np.uint8)[c * chunk * e:(c + 1) * chunk * e]
            box[c, d, :part.size] = part
    assert np.array_equal(img, want)


# ---------------------------------------------------------------------------
# OCP FP8 E4M3FN
# ---------------------------------------------------------------------------

def torch_fn_values():
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


FN_VALUES = torch_fn_values()
FN_MAGS = FN_VALUES[:0x7F]


def brute_fn_encode(x):
    """Nearest finite E4M3FN magnitude (exhaustive), ties to the even code,
    saturating at 448; NaN -> 0x7F|s.  float64 distances are exact wherever
    the choice depends on them (|x| <= 512, ulp >= 2^-41 near midpoints)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    a = np.abs(x)
    a_fin = np.where(np.isfinite(a), np.minimum(a, 512.0), 512.0)
    d = np.abs(a_fin[:, None] - FN_MAGS[None, :])
    i = np.argmin(d, axis=1)
    nxt = np.minimum(i + 1, 0x7E)
    tie = (nxt != i) & (d[np.arange(len(i)), nxt] == d[np.arange(len(i)), i])
    i = np.where(tie & (i % 2 == 1), nxt, i)
    sign = np.where(np.signbit(x), 0x80, 0)
    return np.where(np.isnan(x), sign | 0x7F, i | sign).astype(np.uint8)


def test_fp8fn_decode_vs_torch(orc):
    v = orc.widen_f64(np.arange(256, dtype=np.uint8), "fp8fn")
    assert same_bits_or_both_nan(v, FN_VALUES)
    assert np.nanmax(v) == 448.0 and v[1] == 2.0 ** -9 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254


def test_fp8fn_encode_all_f16_brute_force_and_torch(orc):
    h = np.arange(65536, dtype=np.uint16)
    x = np_f16(h).astype(np.float64)
    got = orc.convert(h, "f16", "fp8fn")
    assert_codes_equal(got, brute_fn_encode(x))
    # torch's own cast agrees wherever it does not overflow (it gives NaN there)
    ok = np.abs(x) < 464
    want = torch.from_numpy(x[ok].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert_codes_equal(got[ok], want)
    assert list(orc.narrow_f64(np.array([464.0, 480.0, 1e9, np.inf, -np.inf, -500.0]), "fp8fn")) == \
        [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


@pytest.mark.parametrize("nranks", [2, 8, 32])
def test_fp8fn_f32_accumulation_is_exact(orc, nranks):
    """E4M3FN values are k * 2^-9 with |k| <= 229376, so <= 32 of them sum
    exactly in f32; every output is the exact sum rounded once."""
    import synth
    n = 50000
    xs = [synth.fp8fn_finite_codes(n, 1300 + r).numpy() for r in range(nranks)]
    k = sum(np.rint(FN_VALUES[x] * 2.0 ** 9).astype(np.int64) for x in xs)
    exact = k.astype(np.float64) * 2.0 ** -9
    exact = np.where(np.logical_and.reduce([x == 0x80 for x in xs]), -0.0, exact)
    got32 = orc.allreduce(xs, "fp8fn", "f32", "f32")
    assert np.array_equal(got32.view(np.uint32), exact.astype(np.float32).view(np.uint32))
    assert_codes_equal(orc.allreduce(xs, "fp8fn", "f32", "f16"), exact.astype(np.float16).view(np.uint16))
    assert_codes_equal(orc.allreduce(xs, "fp8fn", "f32", "fp8fn"), brute_fn_encode(exact))


def test_fp8fn_native_accumulation_and_accuracy(orc):
    import synth
    n, nranks = 20000, 8
    xs = [synth.fp8fn_finite_codes(n, 1400 + r).numpy() for r in range(nranks)]
    acc = brute_fn_encode(FN_VALUES[xs[0]])
    for x in xs[1:]:
        acc = brute_fn_encode(FN_VALUES[acc] + FN_VALUES[x])
    assert_codes_equal(orc.allreduce(xs, "fp8fn", "fp8fn", "fp8fn"), acc)
    exact = sum(FN_VALUES[x] for x in xs)
    e32 = np.abs(orc.widen_f64(orc.allreduce(xs, "fp8fn", "f32", "fp8fn"), "fp8fn") - exact)
    e8 = np.abs(FN_VALUES[acc] - exact)
    assert np.all(e32 <= e8)


# ---------------------------------------------------------------------------
# f32 -> FP8 over every f32 bit pattern
# ---------------------------------------------------------------------------

def f32_encode_steps(mags, nan_code):
    """The correct f32 -> FP8 encoder on the non-negative half of the bit
    patterns, as a step function of the pattern u (patterns of one sign are
    ordered like their values): code j on [starts[j], starts[j+1]).

    The step from code i to i+1 sits at the midpoint of the two magnitudes;
    the midpoint itself belongs to whichever of the two codes is even.  The
    largest code runs on through +inf (saturation), then the NaN patterns."""
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (mags[:-1] + mags[1:]) / 2)  # exact in f32
    mb = mids.view(np.uint32).astype(np.int64)
    code_above = np.arange(1, len(mags))
    starts = np.concatenate([[0], np.where(code_above % 2 == 0, mb, mb + 1), [0x7F800001]])
    codes = np.concatenate([np.arange(len(mags)), [nan_code]]).astype(np.uint8)
    assert np.all(np.diff(starts) > 0)
    return starts, codes


def step_values(starts, codes, lo, hi):
    out = np.empty(hi - lo, np.uint8)
    j = int(np.searchsorted(starts, lo, side="right")) - 1
    pos = lo
    while pos < hi:
        end = min(hi, int(starts[j + 1])) if j + 1 < len(starts) else hi
        out[pos - lo:end - lo] = codes[j]
        pos, j = end, j + 1
    return out


@pytest.mark.parametrize("t", ["fp8", "fp8fn"])
def test_f32_encode_every_bit_pattern(orc, t):
    """All 2^32 f32 inputs of the oracle's single-rounding f32 -> FP8 encoder
    against the step function above, built from magnitudes decoded by
    library routines (numpy's f16 for E4M3B15, torch's float8_e4m3fn for
    E4M3FN); negative patterns must give the same code with the sign bit."""
    from concurrent.futures import ThreadPoolExecutor
    mags = FP8_MAGS if t == "fp8" else FN_MAGS
    starts, codes = f32_encode_steps(mags, 0x7F)
    chunk = 1 << 24

    def run(job):
        sign, lo = job
        u = np.arange(lo, lo + chunk, dtype=np.uint32) | np.uint32(sign << 31)
        got = orc.convert(u.view(np.float32), "f32", t)
        want = step_values(starts, codes, lo, lo + chunk) | np.uint8(sign << 7)
        if np.array_equal(got, want):
            return None
        i = int(np.flatnonzero(got != want)[0])
        return "pattern %08x: %02x, want %02x" % (int(u[i]), int(got[i]), int(want[i]))

    jobs = [(s, lo) for s in (0, 1) for lo in range(0, 1 << 31, chunk)]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        bad = [r for r in pool.map(run, jobs) if r]
    assert not bad, bad[:4]


# ---------------------------------------------------------------------------
# Two ranks, every pair of 16-bit inputs
# ---------------------------------------------------------------------------

def library_pair_sum(t, x0, x1):
    """RNE_t(x0 + x1) from library arithmetic: numpy's binary16 add, or
    torch's float32 add then bfloat16 cast (one f32 rounding before the
    16-bit one is innocuous: 24 >= 2 * 11 + 2 and 24 >= 2 * 8 + 2)."""
    if t == "f16":
        with np.errstate(invalid="ignore", over="ignore"):  # inf - inf, overflow
            return (np_f16(x0) + np_f16(x1)).view(np.uint16)
    a = torch.from_numpy(x0.view(np.int16)).view(torch.bfloat16).float()
    b = torch.from_numpy(x1.view(np.int16)).view(torch.bfloat16).float()
    return (a + b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("t", ["f16", "bf16"])
def test_two_rank_every_pair(orc, t):
    """All 2^32 pairs (x0, x1) of f16 or bf16 bit patterns -- zeros of both
    signs, subnormals, infinities, NaNs, overflow -- through the oracle's
    two-rank reduction with f32 accumulation, against library arithmetic;
    NaN results need only be NaN on both sides."""
    from concurrent.futures import ThreadPoolExecutor
    nan_lo = 0x7C00 if t == "f16" else 0x7F80
    chunk = 1 << 24

    def run(lo):
        i = np.arange(lo, lo + chunk, dtype=np.uint64)
        x0 = (i >> np.uint64(16)).astype(np.uint16)
        x1 = (i & np.uint64(0xFFFF)).astype(np.uint16)
        got = orc.allreduce([x0, x1], t, "f32")
        want = library_pair_sum(t, x0, x1)
        nan_g, nan_w = (got & 0x7FFF) > nan_lo, (want & 0x7FFF) > nan_lo
        bad = np.flatnonzero((nan_g != nan_w) | ((got != want) & ~nan_w))
        if bad.size == 0:
            return None
        k = bad[0]
        return "x0=%04x x1=%04x: %04x, want %04x" % (x0[k], x1[k], got[k], want[k])

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        bad = [r for r in pool.map(run, range(0, 1 << 32, chunk)) if r]
    assert not bad, bad[:4]
