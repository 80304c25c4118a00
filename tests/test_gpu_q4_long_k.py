"""Long-k and few-tile 4-bit products on the GPU against the oracle: the
fused GEMM's launches that split k across workgroups (fewer tiles than a
quarter of the CUs; binary32 k-partials added in k order by a sum launch),
long products of many tiles, launches of a single record block per tile,
products of unequal k-lengths in one grouped call, accumulate and bf16
outputs of long-k products, bit-identical repeated calls on one workspace,
and HIP graph replays."""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, empty_bytes, host, linear, normwise, spec_dict, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu


def _case(M, K, N, seed, integer):
    w = Q4Weight(K, N, seed, seed + 1, seed + 2, integer=integer)
    X = (synth.small_int_bf16 if integer else synth.normal_bf16)(seed + 3, (M, K))
    sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
    buf, nb = w.pack(sh)
    ref = oracle.gemm(oracle.bf16_to_f64(X), w.shard_f64(spec_dict(sh)))
    return sh, buf, nb, dev(X), ref


@pytest.mark.parametrize("M,K,N", [(300, 8192, 256),   # 64 record blocks a tile, few tiles
                                   (2048, 5120, 4352),  # the gate shape: 136 tiles of 40 blocks
                                   (130, 4096, 48)])    # ragged columns and rows, k split
def test_long_k_products(M, K, N):
    print("q4 long k: M %d K %d N %d" % (M, K, N), flush=True)
    for integer in (True, False):
        sh, buf, nb, dX, ref = _case(M, K, N, 5000 + M, integer)
        Y = linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dX, K, M)
        if integer:
            assert np.array_equal(host(Y), ref)
        else:
            assert normwise(host(Y), ref) <= 2e-3
            # partial sums are added in a fixed order: a second call on a
            # fresh workspace gives the same bits
            Y2 = linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dX, K, M)
            assert torch().equal(Y, Y2)


@pytest.mark.parametrize("M,K,N", [(65, 128, 16), (65, 256, 128), (100, 384, 48), (129, 640, 200),
                                   (70, 896, 16)])
def test_launches_of_few_blocks(M, K, N):
    # 1 to 7 record blocks of 128 k per tile, a few tiles
    print("q4 few blocks: M %d K %d N %d" % (M, K, N), flush=True)
    sh, buf, nb, dX, ref = _case(M, K, N, 5100 + K, True)
    Y = linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dX, K, M)
    assert np.array_equal(host(Y), ref)


def test_unequal_k_lengths_in_one_launch():
    """Products of 128 to 8192 k in one grouped call: tiles of different
    lengths in one launch."""
    t = torch()
    M = 257
    shapes = [(8192, 96), (128, 512), (1152, 200), (4096, 64), (192, 1000), (2048, 256)]
    items, refs = [], []
    keep = []
    for i, (K, N) in enumerate(shapes):
        sh, buf, nb, dX, ref = _case(M, K, N, 5200 + 10 * i, True)
        Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=dX, ldx=K, Y=Y, ldy=N,
                          ydtype=tsl.F32))
        refs.append(ref)
        keep.append((buf, dX))
    print("q4 unequal k: %d products, M %d" % (len(items), M), flush=True)
    ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, M)
    tsl.shard_linear_group(items, tsl.Q4G64, tsl.BF16, M, empty_bytes(ws), ws)
    for it, ref, (K, N) in zip(items, refs, shapes):
        assert np.array_equal(host(it["Y"]), ref), (K, N)


def test_accumulate_and_bf16_outputs_of_long_k():
    """A few tiles of long k: the plain product is split along k, the
    accumulating one is not (only the sum launch could finish its split);
    bf16 output is the round-to-nearest-even of the split's binary32 sum."""
    t = torch()
    M, K, N = 200, 8192, 128
    sh, buf, nb, dX, ref = _case(M, K, N, 5300, False)
    print("q4 accumulate / bf16: M %d K %d N %d" % (M, K, N), flush=True)
    Y = linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dX, K, M)
    assert normwise(host(Y), ref) <= 2e-3
    Ya = t.ones((M, N), dtype=t.float32, device="cuda")
    linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dX, K, M, Y=Ya, ldy=N, accumulate=1)
    assert normwise(host(Ya), ref + 1.0) <= 2e-3
    Yb = linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dX, K, M, ydtype=tsl.BF16)
    assert np.array_equal(Yb.view(t.int16).cpu().numpy().view(np.uint16),
                          oracle.f64_to_bf16(host(Y)))


def test_repeated_calls_on_one_workspace_and_graph_replays():
    """The same workspace for every call (k-partials of earlier calls left
    in it), then the call captured in a graph and replayed with eager calls
    between: every result bit-identical."""
    t = torch()
    M, K, N = 300, 8192, 256
    sh, buf, nb, dX, ref = _case(M, K, N, 5400, False)
    ws = tsl.shard_linear_workspace_size(sh, tsl.Q4G64, M)
    wsb = empty_bytes(ws)
    Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")

    def call():
        tsl.shard_linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dX, K, M, tsl.F32, Y, N, 0, wsb, ws)

    print("q4 repeated calls and graph replays: M %d K %d N %d" % (M, K, N), flush=True)
    call()
    t.cuda.synchronize()
    eager = Y.clone()
    assert normwise(host(eager), ref) <= 2e-3
    for _ in range(3):
        Y.fill_(float("nan"))
        call()
        t.cuda.synchronize()
        assert t.equal(Y, eager)
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        call()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        call()
    for i in range(3):
        Y.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(Y, eager), "replay %d" % i
        Y.fill_(float("nan"))
        call()  # eager work between replays
        t.cuda.synchronize()
        assert t.equal(Y, eager)
