"""GPU parity of the standalone FP8 E4M3B15 codec kernels against the CPU
oracle: every code, every f16 input and every f32 bit pattern -- bit-exact."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits

pytestmark = pytest.mark.gpu


def gpu(fn, src_np, out_dtype, n):
    src = torch.from_numpy(np.ascontiguousarray(src_np)).cuda()
    out = torch.empty(n, dtype=out_dtype, device="cuda")
    assert fn(src, out, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    return out


def test_decode_every_code():
    announce("codec decode all codes")
    codes = np.tile(np.arange(256, dtype=np.uint8), 33)  # vector body + tail
    h = gpu(mrr.mrr_fp8b15_to_f16, codes, torch.int16, codes.size)
    assert_bits_equal(bits(h).view(np.uint16), oracle.convert(codes, "fp8", "f16"), "f16", "->f16")
    f = gpu(mrr.mrr_fp8b15_to_f32, codes, torch.float32, codes.size)
    assert_bits_equal(bits(f), oracle.convert(codes, "fp8", "f32"), "f32", "->f32")


def test_encode_every_f16():
    announce("codec encode all f16")
    h = np.arange(65536, dtype=np.uint16)
    h = np.concatenate([h, h[:13]])
    out = gpu(mrr.mrr_f16_to_fp8b15, h.view(np.int16), torch.uint8, h.size)
    assert_bits_equal(bits(out), oracle.convert(h, "f16", "fp8"), "fp8", "f16->fp8")


def test_encode_f32_structured_and_random():
    announce("codec encode f32")
    mags = oracle.widen_f64(np.arange(0x78, dtype=np.uint8), "fp8")
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(1)), np.nextafter(mids, np.float32(0))])
    rng = np.random.default_rng(99)
    u = rng.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([near, -near, rng.uniform(-1.2, 1.2, 1 << 20).astype(np.float32),
                        (rng.uniform(-1, 1, 1 << 16) * 2.0 ** -13).astype(np.float32), u.view(np.float32),
                        np.array([0, -0.0, np.inf, -np.inf, np.nan, 1e-45, 2.0 ** -14], np.float32)])
    out = gpu(mrr.mrr_f32_to_fp8b15, x, torch.uint8, x.size)
    assert_bits_equal(bits(out), oracle.convert(x, "f32", "fp8"), "fp8", "f32->fp8")


def test_encode_every_f32_bit_pattern():
    """All 2^32 f32 inputs (finite, subnormal, infinite and NaN patterns of
    both signs) through the f32 -> E4M3B15 kernel, in 16 launches of 2^28
    elements, each against the oracle computed on host threads."""
    m, sub = 1 << 28, 1 << 24
    iota = torch.arange(m, dtype=torch.int32, device="cuda")
    out = torch.empty(m, dtype=torch.uint8, device="cuda")
    workers = min(16, os.cpu_count() or 1)

    def oracle_slice(lo):  # lo: unsigned bit pattern of the first input
        u = np.arange(lo, lo + sub, dtype=np.uint64).astype(np.uint32)
        return oracle.convert(u.view(np.float32), "f32", "fp8")

    with ThreadPoolExecutor(max_workers=workers) as pool:
        for s in range(16):
            base = s * m - (1 << 31)  # signed first pattern; base + m - 1 fits int32
            announce("codec f32 every pattern", s)
            x = iota + base
            assert mrr.mrr_f32_to_fp8b15(x.view(torch.float32), out, m) == mrr.MRR_OK
            lo = base & 0xFFFFFFFF
            want = list(pool.map(oracle_slice, range(lo, lo + m, sub)))
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for j, w in enumerate(want):  # exact codes, NaN codes included
                g = got[j * sub:(j + 1) * sub]
                bad = np.flatnonzero(g != w)
                assert bad.size == 0, "pattern %08x: got %02x want %02x (%d mismatches)" % (
                    lo + j * sub + bad[0], g[bad[0]], w[bad[0]], bad.size)


@pytest.mark.parametrize("off", [1, 3])
def test_unaligned(off):
    announce("codec unaligned", off)
    rng = np.random.default_rng(off)
    codes = rng.integers(0, 256, 5000 + off, dtype=np.uint8)
    src = torch.from_numpy(codes).cuda()[off:]
    out = torch.empty(5000 + off, dtype=torch.float32, device="cuda")[off:]
    assert mrr.mrr_fp8b15_to_f32(src, out, 5000) == mrr.MRR_OK
    torch.cuda.synchronize()
    assert_bits_equal(bits(out), oracle.convert(codes[off:], "fp8", "f32"), "f32", "unaligned")


def test_full_size_32mib_codes():
    """One 32 MiB buffer of finite codes: decode to f16, re-encode: identity."""
    import synth
    announce("codec 32MiB")
    n = 32 << 20
    codes = synth.fp8_finite_codes(n, 5, device="cuda")
    h = torch.empty(n, dtype=torch.int16, device="cuda")
    back = torch.empty(n, dtype=torch.uint8, device="cuda")
    assert mrr.mrr_fp8b15_to_f16(codes, h, n) == mrr.MRR_OK
    assert mrr.mrr_f16_to_fp8b15(h, back, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    neg_zero = codes == 0x80
    assert torch.equal(back[~neg_zero], codes[~neg_zero]) and torch.all(back[neg_zero] == 0x80)
    idx = torch.randint(0, n, (1 << 18,), device="cuda")
    assert_bits_equal(bits(h[idx]).view(np.uint16),
                      oracle.convert(bits(codes[idx]), "fp8", "f16"), "f16", "sampled")


@pytest.mark.parametrize("grid,cap", [(1, "1"), (5, "1"), (0, "0")])
def test_workgroups_walk_tiles(grid, cap, mrr_env):
    """Fewer workgroups than tiles: MRR_MAX_GRID (re-read through mrr_reload_env) caps the
    grid, so each workgroup walks several tiles, as calls above 2^22 tiles
    do; MRR_LDS_CAP=0 selects the persistent grid without LDS reservation."""
    announce("codec tile walk", grid, cap)
    rng = np.random.default_rng(40 + grid)
    n = 3 * 256 * 8 * 8 * 4 + 11  # several tiles of every direction, plus a tail
    codes = rng.integers(0, 256, n, dtype=np.uint8)
    f16 = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    f32 = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    if grid:
        mrr_env("MRR_MAX_GRID", str(grid))
    mrr_env("MRR_LDS_CAP", cap)
    c = torch.from_numpy(codes).cuda()
    h = torch.from_numpy(f16.view(np.int16)).cuda()
    f = torch.from_numpy(f32.view(np.int32)).cuda()
    o16 = torch.empty(n, dtype=torch.int16, device="cuda")
    o32 = torch.empty(n, dtype=torch.int32, device="cuda")
    e16 = torch.empty(n, dtype=torch.uint8, device="cuda")
    e32 = torch.empty(n, dtype=torch.uint8, device="cuda")
    assert mrr.mrr_fp8b15_to_f16(c, o16, n) == mrr.MRR_OK
    assert mrr.mrr_fp8b15_to_f32(c, o32, n) == mrr.MRR_OK
    assert mrr.mrr_f16_to_fp8b15(h, e16, n) == mrr.MRR_OK
    assert mrr.mrr_f32_to_fp8b15(f, e32, n) == mrr.MRR_OK
    torch.cuda.synchronize()
    mrr_env("MRR_MAX_GRID", None)
    mrr_env("MRR_LDS_CAP", None)
    assert_bits_equal(bits(o16).view(np.uint16), oracle.convert(codes, "fp8", "f16"), "f16", "dec16")
    assert_bits_equal(bits(o32).view(np.uint32), oracle.convert(codes, "fp8", "f32"), "f32", "dec32")
    assert np.array_equal(bits(e16), oracle.convert(f16, "f16", "fp8")), "enc16"
    assert np.array_equal(bits(e32), oracle.convert(f32.view(np.float32), "f32", "fp8")), "enc32"
