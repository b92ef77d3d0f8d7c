"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the block
split the oracle's threaded legs use, the CPU-baseline legs, the parity
comparison's NaN rule and the kernel-source gate on committed counter
summaries."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import oracle  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env=dict(os.environ, **env), capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("lo,hi,parts,align", [(0, 1, 4, 4096), (0, 10000, 3, 4096),
                                               (5, 1 << 20, 16, 4096), (0, 1 << 22, 7, 1024),
                                               (100, 100, 4, 4096)])
def test_split_range_is_a_disjoint_cover(lo, hi, parts, align):
    blocks = bench.split_range(lo, hi, parts, align)
    assert len(blocks) <= max(1, parts)
    pos = lo
    for a, b in blocks:
        assert a == pos and a < b <= hi
        if b < hi:
            assert (b - lo) % align == 0
        pos = b
    assert pos == hi or (lo == hi and not blocks)


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_run_blocks_visits_every_element_once(threads):
    seen = np.zeros(50_000, dtype=np.int32)

    def fn(a, b):
        seen[a:b] += 1

    bench.run_blocks(fn, 0, seen.size, threads)
    assert np.all(seen == 1)


def test_oracle_legs_report_both_legs():
    orc = oracle.default()
    rng = np.random.default_rng(3)
    ins = [rng.standard_normal(300_000).astype(np.float16).view(np.uint16) for _ in range(4)]

    def block(a, b):
        orc.allreduce_all([x[a:b] for x in ins], "f16", "f32", "f16")

    r = bench.oracle_legs(block, ins[0].size, 4 * 4, 1 << 20, 2, "test")
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert [leg["threads"] for leg in r["legs"]] == [1, 2]
    assert r["cores"] == 2 and r["value"] == r["legs"][-1]["value"] > 0
    for leg in r["legs"]:
        assert len(leg["runs_s"]) == 3 and leg["median_s"] == sorted(leg["runs_s"])[1]
        assert 0 < leg["fraction_of_workload"] <= 1


def test_count_mismatches_nan_rule_and_offset():
    want = np.array([0x3C00, 0x7E00, 0x8000, 0x0001, 0x7C00], dtype=np.uint16)  # 1, NaN, -0, tiny, inf
    good = torch.from_numpy(np.array([0, 0, 0x3C00, 0x7FFF, 0x8000, 0x0001, 0x7C00],
                                     dtype=np.uint16).view(np.int16))
    assert bench.count_mismatches(torch, [good.view(torch.float16)], want, "f16", lo=2) == 0
    bad = good.clone()
    bad[4] = 0  # +0 where the oracle has -0
    bad[6] = 0x7E00  # NaN where the oracle has inf
    assert bench.count_mismatches(torch, [good.view(torch.float16), bad.view(torch.float16)],
                                  want, "f16", lo=2) == 2


def test_count_mismatches_fp8_nan_codes():
    want = np.array([0x79, 0x7F, 0x78], dtype=np.uint8)  # E4M3B15: NaN, NaN, +inf
    got = torch.tensor([0xFA, 0x7C, 0xF8], dtype=torch.uint8)  # NaN, NaN, -inf
    assert bench.count_mismatches(torch, [got], want, "fp8") == 1
    got_fn = torch.tensor([0x7F, 0xFF, 0x7E], dtype=torch.uint8)  # E4M3FN: NaN, NaN, 448
    assert bench.count_mismatches(torch, [got_fn], np.array([0xFF, 0x7F, 0x7E], np.uint8),
                                  "fp8fn") == 0


def test_traffic_is_read_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    key = "rsag_test"
    assert bench.measured_traffic(key) is None
    body = "# comment\nkernel_source_hash %s\nhbm_bytes_per_launch 1234\n"
    (tmp_path / ("%s_pmc.txt" % key)).write_text(body % bench.kernel_source_hash())
    assert bench.measured_traffic(key) == 1234.0
    (tmp_path / ("%s_pmc.txt" % key)).write_text(body % "0123456789abcdef")
    assert bench.measured_traffic(key) is None


def test_committed_summaries_match_the_current_sources():
    """Every committed FETCH/WRITE_SIZE summary the bench reads was taken on
    the kernel sources as they stand, so the bench line's traffic is set."""
    keys = {"rsag_8x64MiB_f16": None, "rsag_16x256MiB_bf16": None, "rsag_32x256MiB_bf16": None,
            "rsag_8x32MiB_fp8fn_to_fp8fn": None, "rsag_dual_8x32MiB_fp8": None,
            "rsag_16x32768KiB_fp8_to_f32": None,
            "codec_dec16_256Mi": bench.CODEC_SOURCES, "codec_enc32_256Mi": bench.CODEC_SOURCES}
    for key, src in keys.items():
        t = bench.measured_traffic(key, src)
        assert t is not None, key
        alg = float(dict(line.split()[:2] for line in open(
            os.path.join(bench.PROFILE_DIR, key + "_pmc.txt")) if not line.startswith("#")
            and len(line.split()) >= 2)["algorithmic_bytes_per_launch"])
        assert 1.0 <= t / alg < 1.001, key


def test_graph_timing_threshold():
    class A:
        graph = "auto"
    assert bench.use_graph(A, 64 * bench.MiB - 1) and not bench.use_graph(A, 64 * bench.MiB)
    A.graph = "off"
    assert not bench.use_graph(A, 1)
    A.graph = "on"
    assert bench.use_graph(A, 1 << 40)
