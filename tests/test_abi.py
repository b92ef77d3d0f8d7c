"""CPU checks of the C ABI: the library loads, exports every entry point that
include/mrr.h declares, and refuses bad arguments with the documented status
before touching the GPU.  Pointers here are fake device addresses that the
library never dereferences on these paths."""
import os
import re

import pytest

import allreduce_reduction_nranks_amd as mrr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mrr.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

BASE = 0x7F0000000000  # fake, 4 KiB aligned device address space
MiB = 1 << 20


def fake(i, size=64 * MiB, off=0):
    return BASE + i * size + off


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mrr_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return mrr.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(8):
        txt = mrr.mrr_status_string(s)
        assert txt.startswith(mrr.STATUS_NAMES[s])
    assert "unknown" in mrr.mrr_status_string(99)
    assert mrr.mrr_version() >= 10000


def read_golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            out[k] = [int(x) for x in v]
    return out


def rsag(n, count=1024, t="f16", acc="f32", out=None, rank=-1, ins=None, outs=None):
    ins = ins if ins is not None else [fake(r) for r in range(n)]
    outs = outs if outs is not None else [fake(64 + r) for r in range(n)]
    return mrr.mrr_allreduce_rsag_ex(ins, outs, count, t, acc, out or t, n, rank, stream=0)


def test_rank_counts_follow_the_pages(lib):
    g = read_golden("rsag_verification_sizes.txt")
    for n in g["rejected_nranks"] + [0, 1, 33, 64, -2]:
        assert rsag(max(n, 0) if n > 0 else n, ins=[fake(r) for r in range(max(n, 1))],
                    outs=[fake(64 + r) for r in range(max(n, 1))]) == mrr.MRR_EUNSUPPORTED
    for n in g["supported_nranks"]:
        assert rsag(n, count=0) == mrr.MRR_OK  # nothing to do: no launch


def test_rsag_argument_checks(lib):
    assert rsag(8, rank=-2) == mrr.MRR_EINVAL
    assert rsag(8, rank=8) == mrr.MRR_EINVAL
    assert mrr.load_library().mrr_allreduce_rsag_ex(None, None, 16, 2, 1, 2, 8, -1, None) \
        == mrr.MRR_EINVAL
    ins = [fake(r) for r in range(8)]
    ins[3] = 0
    assert rsag(8, ins=ins) == mrr.MRR_EINVAL


@pytest.mark.parametrize("t,acc,out", [("bf16", "f16", "bf16"), ("f16", "bf16", "f16"),
                                       ("f32", "f16", "f32"), ("f16", "f32", "f32"),
                                       ("bf16", "f32", "f16"), ("f32", "f32", "fp8"),
                                       ("fp8", "f32", "fp8fn"), ("fp8fn", "fp8", "fp8"),
                                       ("fp8fn", "f32", "fp8"), ("fp8fn", "bf16", "fp8fn")])
def test_rsag_unsupported_types(lib, t, acc, out):
    assert rsag(8, t=t, acc=acc, out=out) == mrr.MRR_EUNSUPPORTED


def test_rsag_alignment(lib):
    ins = [fake(r) for r in range(4)]
    ins[2] += 1  # odd address for f16
    assert rsag(4, ins=ins) == mrr.MRR_EALIGN
    outs = [fake(64 + r) for r in range(4)]
    outs[1] += 2  # f32 needs 4
    assert rsag(4, t="f32", outs=outs) == mrr.MRR_EALIGN


def test_rsag_overlap(lib):
    ins = [fake(r) for r in range(4)]
    # output 0 overlaps input 1 partially
    assert rsag(4, count=1024, ins=ins, outs=[fake(1, off=512)] + [fake(64 + r) for r in range(1, 4)]) \
        == mrr.MRR_EOVERLAP
    # output 2 equals input 1 exactly: only an output's own input may alias it
    outs = [fake(64 + r) for r in range(4)]
    outs[2] = ins[1]
    assert rsag(4, ins=ins, outs=outs) == mrr.MRR_EOVERLAP
    # two outputs overlap
    outs = [fake(64 + r) for r in range(4)]
    outs[3] = outs[2] + 16
    assert rsag(4, ins=ins, outs=outs) == mrr.MRR_EOVERLAP
    # fp8 -> f16 in place is impossible (sizes differ)
    assert rsag(4, t="fp8", acc="f32", out="f16", ins=ins, outs=list(ins)) == mrr.MRR_EOVERLAP


def test_packet_sizes(lib):
    assert mrr.mrr_packet_scratch_bytes(1000, "f16", 8) == 8 * 8 * 500 * 8
    assert mrr.mrr_packet_scratch_bytes(1023, "fp8", 4) == 4 * 4 * 256 * 8
    assert mrr.mrr_packet_scratch_bytes(7, "f32", 2) == 2 * 2 * 7 * 8
    assert mrr.mrr_packet_flag_bytes(8) == 8 * 1024 * 4
    assert mrr.mrr_packet_flag_bytes(0) == 0


def packet(n=8, count=4096, t="f16", acc="f32", scratch=None, sbytes=None, flags=None,
           blocks=0, threads=0, ins=None, outs=None):
    ins = ins if ins is not None else [fake(r) for r in range(n)]
    outs = outs if outs is not None else [fake(64 + r) for r in range(n)]
    scratch = scratch if scratch is not None else fake(200)
    sbytes = sbytes if sbytes is not None else mrr.mrr_packet_scratch_bytes(count, t, n)
    flags = flags if flags is not None else fake(300)
    return mrr.mrr_allreduce_packet_ex(ins, outs, scratch, sbytes, flags, count, t, acc, n,
                                       1000, 0, blocks, threads, stream=0)


def test_packet_argument_checks(lib):
    assert packet(n=3) == mrr.MRR_EUNSUPPORTED
    assert packet(t="bf16", acc="f16") == mrr.MRR_EUNSUPPORTED
    assert packet(sbytes=mrr.mrr_packet_scratch_bytes(4096, "f16", 8) - 8) == mrr.MRR_ESCRATCH
    assert packet(threads=100) == mrr.MRR_EINVAL
    assert packet(threads=2048) == mrr.MRR_EINVAL
    assert packet(threads=1024) == mrr.MRR_EINVAL  # the allpair kernel is built for <= 512
    assert packet(blocks=1025) == mrr.MRR_EINVAL
    assert packet(scratch=fake(200, off=4)) == mrr.MRR_EALIGN
    ins = [fake(r) for r in range(8)]
    ins[5] += 2
    assert packet(ins=ins) == mrr.MRR_EALIGN
    assert packet(flags=fake(200, off=64)) == mrr.MRR_EOVERLAP  # flags inside scratch
    assert packet(scratch=fake(3)) == mrr.MRR_EOVERLAP  # scratch over an input
    assert packet(count=0) == mrr.MRR_OK


def test_packet_reduce_and_pack_checks(lib):
    ins = [fake(r) for r in range(4)]
    L = mrr
    assert L.mrr_packet_reduce(ins + [fake(4)], fake(100), 64, "f16", "f32", 5, 1, 2, 10, None,
                               0) == mrr.MRR_EUNSUPPORTED
    assert L.mrr_packet_reduce(ins, fake(100, off=4), 64, "f16", "f32", 4, 1, 2, 10, None, 0) \
        == mrr.MRR_EALIGN
    assert L.mrr_packet_reduce(ins, fake(1, off=64), 64, "f16", "f32", 4, 1, 2, 10, None, 0) \
        == mrr.MRR_EOVERLAP
    assert L.mrr_packet_reduce(ins, fake(100), 0, "f16", "f32", 4, 1, 2, 10, None, 0) == mrr.MRR_OK
    assert L.mrr_pack(fake(0, off=2), fake(1), 100, 1, 0) == mrr.MRR_EALIGN
    assert L.mrr_pack(fake(0), fake(0, off=64), 100, 1, 0) == mrr.MRR_EOVERLAP
    assert L.mrr_unpack(fake(0, off=4), fake(1), 100, 0) == mrr.MRR_EALIGN
    assert L.mrr_pack(0, fake(1), 100, 1, 0) == mrr.MRR_EINVAL
    assert L.mrr_pack(fake(0), fake(1), 0, 1, 0) == mrr.MRR_OK


def test_codec_checks(lib):
    assert mrr.mrr_fp8b15_to_f16(fake(0), fake(1, off=1), 16, 0) == mrr.MRR_EALIGN
    assert mrr.mrr_f32_to_fp8b15(fake(0, off=2), fake(1), 16, 0) == mrr.MRR_EALIGN
    assert mrr.mrr_fp8b15_to_f32(fake(0), fake(0, off=8), 16, 0) == mrr.MRR_EOVERLAP
    assert mrr.mrr_f16_to_fp8b15(0, fake(1), 16, 0) == mrr.MRR_EINVAL
    assert mrr.mrr_f16_to_fp8b15(fake(0), fake(1), 0, 0) == mrr.MRR_OK


def test_stream_copy_checks(lib):
    assert mrr.mrr_stream_copy(fake(0), fake(1), 0, 0) == mrr.MRR_OK  # nothing to do
    assert mrr.mrr_stream_copy(0, fake(1), 64, 0) == mrr.MRR_EINVAL
    assert mrr.mrr_stream_copy(fake(0, off=8), fake(1), 64, 0) == mrr.MRR_EALIGN
    assert mrr.mrr_stream_copy(fake(0), fake(1, off=4), 64, 0) == mrr.MRR_EALIGN
    assert mrr.mrr_stream_copy(fake(0), fake(0, off=32), 64, 0) == mrr.MRR_EOVERLAP
    assert mrr.mrr_stream_copy(fake(0), fake(0), 64, 0) == mrr.MRR_EOVERLAP
    assert mrr.mrr_stream_copy(fake(0), fake(1), (1 << 40) + 16, 0) == mrr.MRR_EINVAL


def test_binding_names_match_header():
    names = declared_functions()
    for n in names:
        assert callable(getattr(mrr, n)), n


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "allreduce_reduction_nranks_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.lower(), f


def test_rank_buffer_pitch(lib):
    MiB = 1 << 20
    assert mrr.mrr_rank_buffer_pitch(0, 8) == 0 and mrr.mrr_rank_buffer_pitch(100, 0) == 0
    assert mrr.mrr_rank_buffer_pitch(1, 8) == 8192
    assert mrr.mrr_rank_buffer_pitch(64 * MiB, 8) == 64 * MiB + 4096
    assert mrr.mrr_rank_buffer_pitch(64 * MiB, 16) == 64 * MiB + 3072
    assert mrr.mrr_rank_buffer_pitch(64 * MiB + 1, 2) == 64 * MiB + 8192
    # odd multiples of 128 MiB take the other stagger; even ones and others do not
    assert mrr.mrr_rank_buffer_pitch(128 * MiB, 8) == 128 * MiB + 5120
    assert mrr.mrr_rank_buffer_pitch(384 * MiB - 100, 4) == 384 * MiB + 5120
    assert mrr.mrr_rank_buffer_pitch(128 * MiB, 16) == 128 * MiB + 8192
    assert mrr.mrr_rank_buffer_pitch(128 * MiB, 2) == 128 * MiB + 4096
    assert mrr.mrr_rank_buffer_pitch(128 * MiB + 1, 8) == 128 * MiB + 4096 + 4096
    assert mrr.mrr_rank_buffer_pitch(256 * MiB, 8) == 256 * MiB + 4096
    assert mrr.mrr_rank_buffer_pitch(256 * MiB, 32) == 256 * MiB + 3072
    for n in (2, 4, 8, 16, 32):
        for b in (4095, 4096, 4097, 12345, 128 * MiB, 256 * MiB, 384 * MiB):
            p = mrr.mrr_rank_buffer_pitch(b, n)
            assert p % 1024 == 0 and p >= b + 2048 and p <= b + 8192


def test_allreduce_dispatch_checks(lib):
    ins = [fake(r) for r in range(33)]
    outs = [fake(64 + r) for r in range(33)]
    for n in (0, 33, -1):
        assert mrr.mrr_allreduce(ins[:max(n, 1)], outs[:max(n, 1)], 1024, "f16", "f32", n,
                                 stream=0) == mrr.MRR_EUNSUPPORTED
    # rank counts outside {2,4,8,16,32} are accepted (runtime-N RS/AG); check the
    # validation reaches the buffers: an odd address is refused before any launch
    for n in (1, 3, 5, 7, 12, 31):
        bad = list(ins[:n])
        bad[0] += 1
        assert mrr.mrr_allreduce(bad, outs[:n], 1024, "f16", "f32", n, stream=0) == mrr.MRR_EALIGN
        assert mrr.mrr_allreduce(ins[:n], outs[:n], 0, "f16", "f32", n, stream=0) == mrr.MRR_OK
    # the RS/AG entry itself keeps the pages' rank-count contract
    assert rsag(3, ins=ins[:3], outs=outs[:3]) == mrr.MRR_EUNSUPPORTED
    assert mrr.mrr_allreduce(ins[:4], outs[:4], 64, "bf16", "f16", 4, stream=0) == mrr.MRR_EUNSUPPORTED


def test_packet_rsag_sizes_and_checks(lib):
    # chunk C = roundup(ceil(count / N), 16 / e) elements, cw = C * e / 4 words, 2 regions
    assert mrr.mrr_packet_rsag_scratch_bytes(1000, "f16", 8) == 2 * 8 * 8 * (128 * 2 // 4) * 8
    assert mrr.mrr_packet_rsag_scratch_bytes(5, "f16", 8) == 2 * 8 * 8 * 4 * 8
    assert mrr.mrr_packet_rsag_scratch_bytes(1023, "fp8", 4) == 2 * 4 * 4 * (256 // 4) * 8
    ins = [fake(r) for r in range(8)]
    outs = [fake(64 + r) for r in range(8)]
    need = mrr.mrr_packet_rsag_scratch_bytes(4096, "f16", 8)
    f = mrr.mrr_allreduce_packet_rsag
    assert f(ins, outs, fake(200), need - 8, fake(300), 4096, "f16", "f32", 8, 10, 0, 0, 0, 0) == mrr.MRR_ESCRATCH
    assert f(ins[:3], outs[:3], fake(200), need, fake(300), 4096, "f16", "f32", 3, 10, 0, 0, 0, 0) == mrr.MRR_EUNSUPPORTED
    assert f(ins, outs, fake(200), need, fake(300), 4096, "f16", "f32", 8, 10, 0, 0, 96, 0) == mrr.MRR_EINVAL
    assert f(ins, outs, fake(200), need, fake(300), 0, "f16", "f32", 8, 10, 0, 0, 0, 0) == mrr.MRR_OK


def test_rsag_dual_checks(lib):
    """mrr_allreduce_rsag_dual: refusals before any launch."""
    n = 8
    ins = [fake(r) for r in range(n)]
    o16 = [fake(64 + r) for r in range(n)]
    o8 = [fake(128 + r) for r in range(n)]
    f = mrr.mrr_allreduce_rsag_dual
    assert f(ins, o16, o8, 0, "fp8", "f32", n, stream=0) == mrr.MRR_OK  # nothing to do
    assert f(ins[:3], o16[:3], o8[:3], 1024, "fp8", "f32", 3, stream=0) == mrr.MRR_EUNSUPPORTED
    for t, acc in (("f16", "f32"), ("bf16", "f32"), ("fp8", "bf16"), ("fp8fn", "fp8"),
                   ("fp8", "fp8fn")):
        assert f(ins, o16, o8, 1024, t, acc, n, stream=0) == mrr.MRR_EUNSUPPORTED, (t, acc)
    assert f(ins, o16, o8, 1024, "fp8", "f32", n, rank=8, stream=0) == mrr.MRR_EINVAL
    assert f(ins, o16, o8, 1024, "fp8", "f32", n, rank=-2, stream=0) == mrr.MRR_EINVAL
    assert lib.mrr_allreduce_rsag_dual(None, None, None, 16, 4, 1, n, -1, None) == mrr.MRR_EINVAL
    bad = list(o8)
    bad[2] = 0
    assert f(ins, o16, bad, 1024, "fp8", "f32", n, stream=0) == mrr.MRR_EINVAL
    bad = list(o8)
    bad[5] = fake(128 + 5, off=8)  # 8-byte aligned only
    assert f(ins, o16, bad, 1024, "fp8", "f32", n, stream=0) == mrr.MRR_EALIGN
    bad = list(o16)
    bad[1] = ins[1]  # an f16 output on top of an input
    assert f(ins, bad, o8, 1024, "fp8", "f32", n, stream=0) == mrr.MRR_EOVERLAP
    bad = list(o8)
    bad[3] = o16[3] + 512  # an FP8 output inside an f16 output
    assert f(ins, o16, bad, 1024, "fp8", "f32", n, stream=0) == mrr.MRR_EOVERLAP
    bad = list(o8)
    bad[4] = o8[6]
    assert f(ins, o16, bad, 1024, "fp8", "f32", n, stream=0) == mrr.MRR_EOVERLAP


@pytest.mark.parametrize("compiler,std", [("gcc", "c99"), ("g++", "c++11")])
def test_header_is_plain_c_and_cxx(tmp_path, compiler, std):
    """include/mrr.h compiles on its own as C99 and as C++11 with every
    warning an error: no HIP or torch types leak into the C ABI."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip("%s not present" % compiler)
    src = tmp_path / ("use.c" if compiler == "gcc" else "use.cpp")
    src.write_text('#include "mrr.h"\nint f(void) { return (int)MRR_OK + mrr_version(); }\n')
    r = subprocess.run([compiler, "-std=" + std, "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.dirname(HEADER), "-c", str(src), "-o", str(tmp_path / "u.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_packet_size_helpers_refuse_what_the_calls_refuse(lib):
    huge = (1 << 64) - 1
    for f in (mrr.mrr_packet_scratch_bytes, mrr.mrr_packet_rsag_scratch_bytes):
        assert f(huge, "f16", 8) == 0
        assert f(1 << 60, "f32", 8) == 0
        assert f(1024, "f16", 33) == 0 and f(1024, "f16", 0) == 0
        assert f(1024, "f16", 8) > 0
    assert mrr.mrr_packet_flag_bytes(33) == 0 and mrr.mrr_packet_flag_bytes(32) == 32 * 1024 * 4


def test_binding_refuses_short_pointer_lists_and_small_tensors(lib):
    """The C ABI reads nranks entries of every pointer array: the binding
    refuses a shorter list before the call, and a tensor smaller than the
    call's byte count (CPU tensors here; nothing reaches the library)."""
    import torch
    ins = [fake(r) for r in range(4)]
    outs = [fake(64 + r) for r in range(4)]
    with pytest.raises(ValueError, match="entries"):
        mrr.mrr_allreduce_rsag(ins[:3], outs, 1024, "f16", 4, stream=0)
    with pytest.raises(ValueError, match="entries"):
        mrr.mrr_allreduce_rsag_ex(ins, outs[:2], 1024, "f16", "f32", "f16", 4, -1, stream=0)
    with pytest.raises(ValueError, match="entries"):
        mrr.mrr_allreduce(ins[:1], outs, 1024, "f16", "f32", 4, stream=0)
    with pytest.raises(ValueError, match="entries"):
        mrr.mrr_allreduce_packet(ins, outs[:3], fake(200), 1 << 20, fake(300), 16, "f16", "f32",
                                 4, 10, None, 0)
    with pytest.raises(ValueError, match="entries"):
        mrr.mrr_packet_reduce(ins[:2], fake(100), 64, "f16", "f32", 4, 1, 2, 10, None, 0)
    small = [torch.empty(1023, dtype=torch.float16) for _ in range(4)]
    with pytest.raises(ValueError, match="holds"):
        mrr.mrr_allreduce_rsag(small, outs, 1024, "f16", 4, stream=0)
    with pytest.raises(ValueError, match="holds"):  # f32 outputs of FP8 inputs: 4 bytes each
        mrr.mrr_allreduce_rsag_ex(ins, [torch.empty(1024, dtype=torch.float16)] * 4, 1024,
                                  "fp8", "f32", "f32", 4, -1, stream=0)
    with pytest.raises(ValueError, match="holds"):
        mrr.mrr_fp8b15_to_f32(fake(0), torch.empty(15, dtype=torch.float32), 16, 0)
    with pytest.raises(ValueError, match="holds"):
        mrr.mrr_allreduce_packet(ins, outs, torch.empty(8, dtype=torch.int64), 128, fake(300),
                                 16, "f16", "f32", 4, 10, None, 0)
    with pytest.raises(ValueError, match="holds"):
        mrr.mrr_allreduce_packet(ins, outs, fake(200), 1 << 20, torch.zeros(4095, dtype=torch.int32),
                                 16, "f16", "f32", 4, 10, None, 0)
    # longer lists are fine: the library reads the first nranks entries
    assert mrr.mrr_allreduce_rsag(ins + [fake(9)], outs + [fake(99)], 0, "f16", 4, stream=0) \
        == mrr.MRR_OK


def test_noalloc_refusals(lib):
    """Checks that run before the library touches its workspace or the GPU."""
    ins = [fake(r) for r in range(8)]
    outs = [fake(64 + r) for r in range(8)]
    f = mrr.mrr_allreduce_packet_noalloc
    assert f(ins, outs, 1024, "f16", "f32", 3, 100, None, 0) == mrr.MRR_EUNSUPPORTED
    assert f(ins, outs, 1024, "bf16", "f16", 8, 100, None, 0) == mrr.MRR_EUNSUPPORTED
    assert f(ins, outs, 0, "f16", "f32", 8, 100, None, 0) == mrr.MRR_OK
    # 8 ranks of f16: at most 32 MiB / (8 * 8 * 8 B) packets of 4 bytes
    most = mrr.MRR_NOALLOC_SCRATCH_BYTES // (8 * 8 * 8) * 2
    assert f(ins, outs, most + 1, "f16", "f32", 8, 100, None, 0) == mrr.MRR_ESCRATCH
    assert f(ins[:2] + [fake(9)], outs[:3], 1 << 30, "f32", "f32", 2, 100, None, 0) \
        == mrr.MRR_ESCRATCH
    bad = list(ins)
    bad[4] += 2
    assert f(bad, outs, 1024, "f16", "f32", 8, 100, None, 0) == mrr.MRR_EALIGN
    assert f(ins, [ins[1]] + outs[1:], 1024, "f16", "f32", 8, 100, None, 0) == mrr.MRR_EOVERLAP


def test_fullmesh_sizes_and_refusals(lib):
    # semaphores N*N*1024*8, then N*N inboxes of C = roundup(ceil(count/N), 16/e) elements
    assert mrr.mrr_fullmesh_scratch_bytes(1000, "f16", 8) == 8 * 8 * 1024 * 8 + 8 * 8 * 128 * 2
    assert mrr.mrr_fullmesh_scratch_bytes(5, "f32", 8) == 8 * 8 * 1024 * 8 + 8 * 8 * 4 * 4
    assert mrr.mrr_fullmesh_scratch_bytes(1, "fp8", 33) == 0
    assert mrr.mrr_fullmesh_scratch_bytes(1, "auto", 2) == 0

    def fm(n=8, count=4096, t="f16", acc="f32", ins=None, outs=None, scratch=None, sbytes=None,
           flags=None, blocks=0, threads=0):
        ins = ins if ins is not None else [fake(r) for r in range(n)]
        outs = outs if outs is not None else [fake(64 + r) for r in range(n)]
        scratch = scratch if scratch is not None else fake(200)
        sbytes = sbytes if sbytes is not None else mrr.mrr_fullmesh_scratch_bytes(count, t, n)
        flags = flags if flags is not None else fake(300)
        return mrr.mrr_allreduce_fullmesh(ins, outs, scratch, sbytes, flags, count, t, acc, n,
                                          1000, 0, blocks, threads, stream=0)

    assert fm(n=6) == mrr.MRR_EUNSUPPORTED
    assert fm(t="bf16", acc="f16") == mrr.MRR_EUNSUPPORTED
    assert fm(sbytes=mrr.mrr_fullmesh_scratch_bytes(4096, "f16", 8) - 16) == mrr.MRR_ESCRATCH
    assert fm(threads=96) == mrr.MRR_EINVAL
    assert fm(threads=1024) == mrr.MRR_EINVAL
    assert fm(blocks=1025) == mrr.MRR_EINVAL
    ins = [fake(r) for r in range(8)]
    ins[3] += 4  # element-aligned, not 16-byte aligned: the full-mesh path needs 16
    assert fm(ins=ins) == mrr.MRR_EALIGN
    assert fm(scratch=fake(200, off=8)) == mrr.MRR_EALIGN
    assert fm(flags=fake(200, off=64)) == mrr.MRR_EOVERLAP
    outs = [fake(64 + r) for r in range(8)]
    outs[2] = ins[5]
    assert fm(outs=outs) == mrr.MRR_EOVERLAP
    assert fm(count=0) == mrr.MRR_OK
