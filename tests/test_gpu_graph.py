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


def test_graph_replays_of_a_large_grouped_prefill_call():
    """A 4-bit grouped call of 512 GEMM tiles (prep pass, then one GEMM
    launch over items of two k lengths): captured in a graph, every replay
    matches the eager call bit for bit, with eager calls in between."""
    t = torch()
    M, N = 2048, 4096
    ks = (3072, 2048, 2048, 2048)
    items, outs, keep = [], [], []
    for i, K in enumerate(ks):
        w = Q4Weight(K, N, 1300 + i, 1301, 1302)
        sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
        buf, nb = w.pack(sh)
        X = dev(synth.normal_bf16(1310 + i, (M, K)))
        Y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
        keep += [buf, X]
        outs.append(Y)
        items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X, ldx=K, Y=Y, ldy=N,
                          ydtype=tsl.BF16))
    ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, M)
    wb = empty_bytes(ws)

    def step():
        tsl.shard_linear_group(items, tsl.Q4G64, tsl.BF16, M, wb, ws,
                               stream=t.cuda.current_stream().cuda_stream)

    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    eager = [Y.clone() for Y in outs]
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for i in range(3):
        for Y in outs:
            Y.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for Y, E in zip(outs, eager):
            assert t.equal(Y, E), "replay %d" % i
        step()
        t.cuda.synchronize()
        for Y, E in zip(outs, eager):
            assert t.equal(Y, E)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_graph_replays_of_decode_sum_sets(M):
    """Decode-sized grouped call whose two sum sets (4 row shards each) are
    added up inside the streaming launch (per-tile arrival counters tagged
    with the call's ticket): every replay of the captured call, eager calls
    of the same items in between, matches the eager result bit for bit, and
    that result is the row shards' products followed by combine_partials."""
    t = torch()
    K, N, tp = 2048, 1024, 4
    outs, items, plain, parts, keep = [], [], [], [], []
    for s in range(2):
        w = Q4Weight(K, N, 1400 + s, 1401, 1402)
        X = dev(synth.normal_bf16(1410 + 10 * s + M, (M, K)))
        Y = t.empty((M, N), dtype=t.bfloat16 if s else t.float32, device="cuda")
        outs.append(Y)
        shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
        for r, sh in enumerate(shards):
            buf, nb = w.pack(sh)
            P = t.empty((M, N), dtype=t.float32, device="cuda")
            keep += [buf, X]
            parts.append(P)
            items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K,
                              Y=Y if r == 0 else None, ldy=N,
                              ydtype=tsl.BF16 if s else tsl.F32, sum_next=int(r < tp - 1)))
            plain.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K,
                              Y=P, ldy=N))
    ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, M)
    wb = empty_bytes(ws)

    def step():
        tsl.shard_linear_group(items, tsl.Q4G64, tsl.BF16, M, wb, ws,
                               stream=t.cuda.current_stream().cuda_stream)

    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    eager = [Y.clone() for Y in outs]
    # the same products, then the ordered sums
    pws = tsl.shard_linear_group_workspace_size(plain, tsl.Q4G64, M)
    pwb = empty_bytes(pws) if pws else None
    tsl.shard_linear_group(plain, tsl.Q4G64, tsl.BF16, M, pwb, pws)
    for s, Y in enumerate(outs):
        want = t.empty_like(Y)
        tsl.combine_partials(tsl.COMBINE_SUM, parts[4 * s:4 * s + 4], tsl.F32, M, N, N,
                             tsl.BF16 if s else tsl.F32, want, N)
        t.cuda.synchronize()
        assert t.equal(eager[s], want), s
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for i in range(3):
        for Y in outs:
            Y.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for Y, E in zip(outs, eager):
            assert t.equal(Y, E), "replay %d" % i
        step()
        t.cuda.synchronize()
        for Y, E in zip(outs, eager):
            assert t.equal(Y, E)
