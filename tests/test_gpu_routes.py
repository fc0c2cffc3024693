"""GPU: the staged fp16-then-cast route against the direct bf16 store, and
GEMVs captured in a HIP graph against the same launches made eagerly.

The staged route (an fp16 GEMV into a staging buffer, then a separate
fp16 -> bf16 cast) is what the direct store replaces (onnx-genai pull
request "perf(cuda): let the split-K decode GEMV store bf16 directly",
opening paragraphs); both must give the same bf16 bits.  The graph test
replays a captured decode-style sequence several times, with eager work in
between, and compares every replay with the eager outputs bit for bit.  The
last test calls the library from several host threads at once.
"""
import numpy as np
import pytest
import torch

import block_wise_int4_matmulnbits_amd as mnb
from block_wise_int4_matmulnbits_amd import workloads as W
from tests import gpu_util as G
from tests.test_gpu_parity import launch_count

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    mnb.lib()


@pytest.mark.parametrize("m,K,N,a_dtype", [(1, 4096, 4096, W.F16), (3, 14336, 777, W.BF16)])
def test_staged_route_equals_direct_store(oracle_mod, m, K, N, a_dtype):
    d = W.generate(m, K, N, a_dtype, True, 0.001, 0.01, 1.0, 500 + m)
    A, B, S, Z = G.to_dev(d, m)
    direct = G.new_out(m, N, W.BF16)
    stage = G.new_out(m, N, W.F16)
    c0 = mnb.mnb_counters_get()
    mnb.matmul_nbits(A, B, S, Z, direct)
    mnb.matmul_nbits(A, B, S, Z, stage)
    staged = stage.to(torch.bfloat16)          # the separate narrowing launch
    torch.cuda.synchronize()
    c1 = mnb.mnb_counters_get()
    assert c1["elements_bf16_direct"] - c0["elements_bf16_direct"] == m * N
    assert c1["elements_f16"] - c0["elements_f16"] == m * N
    assert np.array_equal(G.bits(direct), G.bits(staged))
    # and both equal the oracle's narrowing of the GPU's fp16 result
    assert G.check2(G.bits(direct), G.bits(stage), oracle_mod).all()


def test_graph_replay_matches_eager():
    shapes = [(1, 4096, 4096, W.F16, True), (1, 4096, 28672, W.BF16, True),
              (2, 14336, 4096, W.BF16, True), (1, 1024, 1000, W.F16, False)]
    calls = []
    for i, (m, K, N, a_dtype, asym) in enumerate(shapes):
        d = W.generate(m, K, N, a_dtype, asym, 0.001, 0.01, 0.5, 600 + i)
        A, B, S, Z = G.to_dev(d, m)
        calls.append((A, B, S, Z, G.new_out(m, N, W.BF16)))

    def launch_all():
        for (A, B, S, Z, out) in calls:
            mnb.matmul_nbits(A, B, S, Z, out)

    launch_all()
    torch.cuda.synchronize()
    eager = [G.bits(c[4]) for c in calls]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch_all()
    torch.cuda.synchronize()
    for rep in range(3):
        for c in calls:
            c[4].fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e, c in zip(eager, calls):
            assert np.array_equal(e, G.bits(c[4])), "replay %d differs" % rep
        launch_all()                            # eager work between replays
        torch.cuda.synchronize()
        for e, c in zip(eager, calls):
            assert np.array_equal(e, G.bits(c[4]))


def test_concurrent_host_threads():
    """Several host threads call the library at once, each on its own stream
    (the header allows it): every output equals the same call made alone,
    and the counters account for every launch."""
    import threading
    shapes = [(1, 4096, 4096, W.F16), (3, 14336, 777, W.BF16), (40, 4096, 1000, W.BF16),
              (8, 4096, 2048, W.F16)]
    jobs = []
    for i, (m, K, N, a_dtype) in enumerate(shapes):
        d = W.generate(m, K, N, a_dtype, True, 0.001, 0.01, 0.5, 650 + i)
        A, B, S, Z = G.to_dev(d, m)
        jobs.append((A, B, S, Z, G.new_out(m, N, W.BF16), G.new_out(m, N, W.BF16)))
    for (A, B, S, Z, alone, _) in jobs:
        mnb.matmul_nbits(A, B, S, Z, alone)
    torch.cuda.synchronize()
    c0 = mnb.mnb_counters_get()
    reps = 20
    errors = []

    def worker(job):
        try:
            A, B, S, Z, _, out = job
            stream = torch.cuda.Stream()
            for _ in range(reps):
                mnb.matmul_nbits(A, B, S, Z, out, stream=stream)
            stream.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (_, _, _, _, alone, out) in jobs:
        assert np.array_equal(G.bits(alone), G.bits(out))
    c1 = mnb.mnb_counters_get()
    per_call = sum(launch_count(m, K, N) for (m, K, N, _) in shapes)
    assert c1["launches"] - c0["launches"] == reps * per_call
    assert c1["calls"] - c0["calls"] == reps * len(jobs)
