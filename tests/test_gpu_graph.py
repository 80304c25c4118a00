"""shard_linear and combine_partials captured in a HIP graph (the way the
benchmark replays the decode step): every replay, with eager work and
synchronisations in between, matches the eager result bit for bit."""
import numpy as np
import pytest

from gpu_util import Q4Weight, dev, empty_bytes, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 16, 200])
def test_graph_replays_match_eager(M):
    t = torch()
    K, N, tp = 1024, 256, 2
    w = Q4Weight(K, N, 1200 + M, 1201, 1202)
    X = dev(synth.normal_bf16(1203 + M, (M, K)))
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    packed = [w.pack(sh) for sh in shards]
    parts = [t.empty((M, N), dtype=t.float32, device="cuda") for _ in shards]
    wss = []
    for sh in shards:
        n = tsl.shard_linear_workspace_size(sh, tsl.Q4G64, M)
        wss.append((empty_bytes(n) if n else None, n))
    out = t.empty((M, N), dtype=t.bfloat16, device="cuda")

    def step():
        for sh, (buf, nb), P, (wb, n) in zip(shards, packed, parts, wss):
            tsl.shard_linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, X[:, sh.k_off:], K, M, tsl.F32, P,
                             N, 0, wb, n)
        tsl.combine_partials(tsl.COMBINE_SUM, parts, tsl.F32, M, N, N, tsl.BF16, out, N)

    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    eager = out.clone()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for i in range(3):
        out.fill_(0)
        for P in parts:
            P.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(out, eager), "replay %d" % i
        step()  # eager work between replays
        t.cuda.synchronize()
        assert t.equal(out, eager)
