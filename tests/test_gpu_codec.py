"""GPU parity of the standalone FP8 E4M3B15 codec kernels against the CPU
oracle: every code, every f16 input, and f32 midpoints, neighbours and random
bit patterns -- bit-exact."""
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
