"""combine_to_ranks on the GPU: every rank's buffer after an all-reduce, a
reduce-scatter and an all-gather of rank outputs on one GPU, against the
oracle's per-rank results -- the rank-order binary32 sum bit for bit, its
bf16 rounding bit for bit, copies byte for byte -- over vector and scalar
paths, ragged widths, strides, M smaller than the rank count, and 1..64
ranks."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host_bits, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu

SHAPES = [(4, 256, 2048, 2048), (8, 64, 4096, 4096), (4, 1, 3584, 3584), (3, 5, 20, 24),
          (8, 3, 37, 37), (64, 70, 128, 128), (1, 7, 9, 9)]


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("R,M,n,ld", SHAPES)
def test_all_reduce_and_reduce_scatter(R, M, n, ld, ydt):
    t = torch()
    parts = [synth.normal_f32(700 + r, (M, ld)) for r in range(R)]
    d = [dev(p) for p in parts]
    want32 = oracle.sum_f32_seq([p[:, :n] for p in parts])
    code, tdt = (tsl.F32, t.float32) if ydt == "f32" else (tsl.BF16, t.bfloat16)

    def got(Y):
        return Y.cpu().numpy() if ydt == "f32" else host_bits(Y)

    def want(x):
        return x if ydt == "f32" else oracle.f64_to_bf16(x.astype(np.float64))

    # all-reduce: every rank's own full buffer (row stride n + 8)
    outs = [t.full((M, n + 8), float("nan"), dtype=tdt, device="cuda") for _ in range(R)]
    tsl.combine_to_ranks(tsl.ALL_REDUCE, d, tsl.F32, M, n, ld, code, outs, n + 8)
    for r, ar in enumerate(oracle.all_reduce([p[:, :n] for p in parts], R,
                                             sum_fn=oracle.sum_f32_seq)):
        assert np.array_equal(got(outs[r])[:, :n], want(ar)), r
    # reduce-scatter: the rank blocks side by side in one [M][n] buffer
    Y = t.full((M, n), float("nan"), dtype=tdt, device="cuda")
    blocks = [Y[oracle.rank_rows(M, R, r)[0]:] for r in range(R)]
    tsl.combine_to_ranks(tsl.REDUCE_SCATTER, d, tsl.F32, M, n, ld, code, blocks, n)
    rs = oracle.reduce_scatter([p[:, :n] for p in parts], R, sum_fn=oracle.sum_f32_seq)
    for r in range(R):
        lo, hi = oracle.rank_rows(M, R, r)
        assert np.array_equal(got(Y)[lo:hi], want(rs[r])), r
    assert np.array_equal(got(Y), want(want32))  # the blocks tile the whole sum


@pytest.mark.parametrize("pad", [4, 8])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("R,M,n,ld", SHAPES[:-2] + [(16, 4, 24, 24)])
def test_all_gather(R, M, n, ld, dt, pad):
    # pad 8 keeps bf16 output rows 16-byte aligned (the 16-byte path), pad 4
    # does not for bf16
    t = torch()
    if dt == "f32":
        parts = [synth.normal_f32(800 + r, (M, ld)) for r in range(R)]
        code, tdt = tsl.F32, t.float32
    else:
        parts = [synth.normal_bf16(800 + r, (M, ld)) for r in range(R)]
        code, tdt = tsl.BF16, t.bfloat16
    d = [dev(p) for p in parts]
    width = R * n
    outs = [t.zeros((M, width + pad), dtype=tdt, device="cuda") for _ in range(R)]
    tsl.combine_to_ranks(tsl.ALL_GATHER, d, code, M, n, ld, code, outs, width + pad)
    for r, ag in enumerate(oracle.all_gather([p[:, :n] for p in parts], R)):
        g = outs[r].cpu().numpy() if dt == "f32" else host_bits(outs[r])
        assert np.array_equal(g[:, :width], ag), r
        assert not g[:, width:].any()  # nothing written past the gathered width


def test_reduce_scatter_integer_exact():
    """Integer partials: every rank's block is the exact sum."""
    R, M, n = 8, 17, 96
    parts = [synth.small_int(900 + r, (M, n)) for r in range(R)]
    d = [dev(p) for p in parts]
    outs = [torch().full((max(hi - lo, 1), n), float("nan"), dtype=torch().float32,
                         device="cuda") for lo, hi in (oracle.rank_rows(M, R, r) for r in range(R))]
    tsl.combine_to_ranks(tsl.REDUCE_SCATTER, d, tsl.F32, M, n, n, tsl.F32, outs, n)
    exact = np.sum(np.stack(parts).astype(np.int64), axis=0)
    for r in range(R):
        lo, hi = oracle.rank_rows(M, R, r)
        assert np.array_equal(outs[r].cpu().numpy()[:hi - lo], exact[lo:hi]), r
