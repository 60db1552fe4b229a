"""The generation step captured in a HIP graph (how a serving loop replays it
without host work per launch): one appended row and three cross layers' query
projection + decode, captured once and replayed, equal the same calls run
eagerly, bit for bit, on every replay.  The kernels allocate nothing and
clear nothing with memsets (their arrival counters are reset by the kernels
themselves), so they can be captured.  Eager work and synchronizations run
between the replays."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")

COUNTER_BYTES = 16384            # the projection workspace's arrival counters
DECODE_COUNTER_BYTES = 64 * 1024  # the decode workspace's arrival counters


def test_generation_step_replays_bitwise_in_a_graph():
    print("graph capture: append + 3 x (q_project + decode), 3 replays", flush=True)
    n, d, hkv, hq, dh, layers = 4096, 3072, 8, 24, 128, 3
    r = np.random.default_rng(61)
    pc = W.make_project(n=n, d_model=d, unit_gain=False, seed=62)
    cache = y.KVCache(1, n + 8, hkv, dh, torch.bfloat16, zero=True)
    w_k, w_v, gain = to_dev(pc.w_k), to_dev(pc.w_v), torch.from_numpy(pc.gain).cuda()
    y.kv_project(cache, to_dev(pc.m[:-1]), w_k, w_v, gain, pc.eps)
    m_last = to_dev(pc.m[-1:])
    xs = [to_dev(W.store(r.standard_normal((1, d)).astype(np.float32), W.BF16)) for _ in range(layers)]
    wqs = [to_dev(W.store((r.standard_normal((d, hq * dh)) / np.sqrt(d)).astype(np.float32), W.BF16))
           for _ in range(layers)]
    pws = torch.zeros(max(y.project_workspace_bytes(1, d, hkv * dh, 2), y.project_workspace_bytes(1, d, hq * dh, 1)),
                      dtype=torch.uint8, device="cuda")
    dws = y.decode_workspace(cache, hq)
    qs = [torch.empty(1, hq, dh, dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    outs = [torch.empty(1, hq, dh, device="cuda") for _ in range(layers)]
    stream = torch.cuda.Stream()

    def step(s):
        cache.len[0] = n - 1
        y.kv_append(cache, m_last, w_k, w_v, gain, pc.eps, stream=s, workspace=pws)
        for l in range(layers):
            y.q_project(xs[l], wqs[l], hq, dh, out=qs[l], stream=s, workspace=pws)
            y.cross_attn_decode(qs[l], cache, workspace=dws, out=outs[l], stream=s)

    with torch.cuda.stream(stream):
        step(stream)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    row = cache.k[0, n - 1].clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(None)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        cache.k[0, n - 1].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache.k[0, n - 1], row), f"replay {rep}: appended row differs"
        for l in range(layers):
            assert torch.equal(outs[l], eager[l]), f"replay {rep}: layer {l} differs from the eager step"
        assert not bool(pws[:COUNTER_BYTES].any()), "an arrival counter was left non-zero"
        assert not bool(dws[:DECODE_COUNTER_BYTES].any()), "a decode arrival counter was left non-zero"
        # eager work between replays
        with torch.cuda.stream(stream):
            step(stream)
        torch.cuda.synchronize()
        for l in range(layers):
            assert torch.equal(outs[l], eager[l])
