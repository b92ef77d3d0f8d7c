"""Concurrency and capture: the library keeps no device state, so calls
from several host threads on their own streams must not interfere, and every
entry point must replay correctly from a HIP graph.  Results are compared
with the CPU oracle (and, for replays, with the eager call) bit for bit."""
import threading

import numpy as np
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
import oracle
from gpu_common import announce, assert_bits_equal, bits, empty, inputs_for

pytestmark = pytest.mark.gpu


def test_threads_on_separate_streams():
    """Four host threads, each on its own stream (default priority), issue
    RS/AG, dispatcher and packet calls on their own buffers; every result
    matches the oracle."""
    announce("threads x streams")
    jobs = []
    for j in range(4):
        t = ["f16", "bf16", "fp8", "f32"][j]
        n = [8, 5, 4, 2][j]
        count = 40_000 + 1_111 * j
        kind = "fp8codes" if t == "fp8" else "normal"
        ins = inputs_for(t, n, count, seed0=500 + 10 * j, kind=kind)
        outs = [empty(t, count, 0x33) for _ in range(n)]
        jobs.append(dict(t=t, n=n, count=count, ins=ins, outs=outs, stream=torch.cuda.Stream(),
                         status=[]))
    pk = dict(n=8, count=6_000)
    pk["ins"] = inputs_for("f16", 8, pk["count"], seed0=777, kind="uniform")
    pk["outs"] = [empty("f16", pk["count"], 0x33) for _ in range(8)]
    pk["sbytes"] = mrr.mrr_packet_scratch_bytes(pk["count"], "f16", 8)
    pk["scratch"] = torch.zeros(pk["sbytes"] // 8, dtype=torch.int64, device="cuda")
    pk["flags"] = torch.zeros(8 * mrr.PKT_FLAG_SLOTS, dtype=torch.int32, device="cuda")
    pk["err"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    pk["stream"] = torch.cuda.Stream()
    pk["status"] = []
    torch.cuda.synchronize()

    def run(job):
        for _ in range(5):
            if job["n"] in (2, 4, 8, 16, 32):
                st = mrr.mrr_allreduce_rsag_ex(job["ins"], job["outs"], job["count"], job["t"], "f32",
                                               job["t"], job["n"], -1, stream=job["stream"])
            else:
                st = mrr.mrr_allreduce(job["ins"], job["outs"], job["count"], job["t"], "f32",
                                       job["n"], stream=job["stream"])
            job["status"].append(st)
        job["stream"].synchronize()

    def run_packets():
        for _ in range(5):
            pk["status"].append(mrr.mrr_allreduce_packet(
                pk["ins"], pk["outs"], pk["scratch"], pk["sbytes"], pk["flags"], pk["count"], "f16",
                "f32", 8, 2_000_000, pk["err"], stream=pk["stream"]))
        pk["stream"].synchronize()

    threads = [threading.Thread(target=run, args=(j,)) for j in jobs]
    threads.append(threading.Thread(target=run_packets))
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    for j in jobs:
        assert all(st == mrr.MRR_OK for st in j["status"]), j["status"]
        want = oracle.allreduce([bits(x) for x in j["ins"]], j["t"], "f32", j["t"])
        for k in range(j["n"]):
            assert_bits_equal(bits(j["outs"][k]), want, j["t"], "%s n=%d out[%d]" % (j["t"], j["n"], k))
    assert all(st == mrr.MRR_OK for st in pk["status"]) and int(pk["err"].item()) == 0
    want = oracle.allreduce([bits(x) for x in pk["ins"]], "f16", "f32")
    for k in range(8):
        assert_bits_equal(bits(pk["outs"][k]), want, "f16", "packet out[%d]" % k)
    assert np.all(pk["flags"].cpu().numpy().view(np.uint32) == 5)


def test_graph_of_dispatcher_dual_and_codec():
    """One HIP graph holding a runtime-N dispatcher call, a one-pass FP8
    reduction and a codec call, replayed three times with eager work and
    synchronisations in between; every replay equals the eager results."""
    announce("graph: dispatcher + dual + codec")
    n5, c5 = 5, 30_001
    ins5 = inputs_for("f16", n5, c5, seed0=900)
    n8, c8 = 8, 20_000
    ins8 = inputs_for("fp8", n8, c8, seed0=910, kind="fp8codes")
    codes = torch.arange(256, dtype=torch.uint8, device="cuda").repeat(40)

    def outputs():
        return ([empty("f16", c5, 0) for _ in range(n5)], [empty("f16", c8, 0) for _ in range(n8)],
                [empty("fp8", c8, 0) for _ in range(n8)], empty("f16", codes.numel(), 0))

    def calls(o5, o16, o8, h, stream=None):
        assert mrr.mrr_allreduce(ins5, o5, c5, "f16", "f32", n5, stream=stream) == mrr.MRR_OK
        assert mrr.mrr_allreduce_rsag_dual(ins8, o16, o8, c8, "fp8", "f32", n8,
                                           stream=stream) == mrr.MRR_OK
        assert mrr.mrr_fp8b15_to_f16(codes, h, codes.numel(), stream=stream) == mrr.MRR_OK

    eager = outputs()
    calls(*eager)
    torch.cuda.synchronize()
    graph_out = outputs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls(*graph_out, stream=s)
    torch.cuda.synchronize()
    flat_eager = eager[0] + eager[1] + eager[2] + [eager[3]]
    for rep in range(3):
        for x in graph_out[0] + graph_out[1] + graph_out[2] + [graph_out[3]]:
            x.view(torch.uint8).zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        flat = graph_out[0] + graph_out[1] + graph_out[2] + [graph_out[3]]
        for i, (a, b) in enumerate(zip(flat, flat_eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d buffer %d" % (rep, i)
    want = oracle.allreduce([bits(x) for x in ins5], "f16", "f32")
    assert_bits_equal(bits(eager[0][0]), want, "f16", "dispatcher vs oracle")


def test_default_stream_is_torch_current_stream():
    """stream=None resolves to torch's current stream on the current device,
    inside and outside a torch.cuda.stream context."""
    import allreduce_reduction_nranks_amd as mrr_mod
    assert mrr_mod._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert mrr_mod._stream(None) == s.cuda_stream
    assert mrr_mod._stream(None) == torch.cuda.current_stream().cuda_stream
