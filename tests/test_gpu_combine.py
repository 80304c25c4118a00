"""combine_partials on the GPU against the oracle: the rank-order binary32
sum bit for bit, its bf16 rounding bit for bit, and the concat byte for
byte, over vector and scalar paths, ragged widths, strides and 1..64 parts."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, host_bits, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("R,M,n,ld", [(2, 32, 2048, 2048), (4, 256, 2048, 2048), (8, 64, 4096, 4096),
                                      (8, 3, 37, 37), (3, 5, 20, 24), (64, 2, 128, 128),
                                      (1, 7, 9, 9)])
def test_sum_bit_exact(R, M, n, ld):
    parts = [synth.normal_f32(500 + r, (M, ld)) for r in range(R)]
    d = [dev(p) for p in parts]
    Y = torch().full((M, n), float("nan"), dtype=torch().float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, d, tsl.F32, M, n, ld, tsl.F32, Y, n)
    want = oracle.sum_f32_seq([p[:, :n] for p in parts])
    assert np.array_equal(Y.cpu().numpy(), want)
    # within the tolerance of the fp64 sum too
    exact = oracle.combine_sum([p[:, :n].astype(np.float64) for p in parts])
    assert np.max(np.abs(host(Y) - exact)) <= 1e-5 * np.max(np.abs(exact))
    # bf16 output: one rounding of the same binary32 sum
    Yb = torch().zeros((M, n), dtype=torch().bfloat16, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, d, tsl.F32, M, n, ld, tsl.BF16, Yb, n)
    assert np.array_equal(host_bits(Yb), oracle.f64_to_bf16(want.astype(np.float64)))


def test_sum_integer_exact_and_in_place():
    parts = [synth.small_int(520 + r, (16, 64)) for r in range(8)]
    d = [dev(p) for p in parts]
    exact = np.sum(np.stack(parts).astype(np.int64), axis=0).astype(np.float64)
    # Y aliases part 0 (same leading dimension)
    tsl.combine_partials(tsl.COMBINE_SUM, d, tsl.F32, 16, 64, 64, tsl.F32, d[0], 64)
    assert np.array_equal(host(d[0]), exact)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R,M,n,ld", [(2, 32, 1024, 1024), (4, 16, 128, 128), (8, 5, 13, 13),
                                      (3, 4, 24, 40)])
def test_concat_byte_exact(dtype, R, M, n, ld):
    if dtype == "f32":
        parts = [synth.normal_f32(540 + r, (M, ld)) for r in range(R)]
        code = tsl.F32
        Y = torch().zeros((M, R * n + 8), dtype=torch().float32, device="cuda")
    else:
        parts = [synth.normal_bf16(540 + r, (M, ld)) for r in range(R)]
        code = tsl.BF16
        Y = torch().zeros((M, R * n + 8), dtype=torch().bfloat16, device="cuda")
    d = [dev(p) for p in parts]
    tsl.combine_partials(tsl.COMBINE_CONCAT, d, code, M, n, ld, code, Y, R * n + 8)
    got = Y.cpu() if dtype == "f32" else Y.view(torch().int16).cpu()
    got = got.numpy().view(np.float32 if dtype == "f32" else np.uint16)
    want = oracle.combine_concat([p[:, :n] for p in parts])
    assert np.array_equal(got[:, :R * n], want)
    assert not got[:, R * n:].any()  # nothing written past the concat


def test_empty_inputs_enqueue_nothing():
    d = [dev(np.zeros((2, 8), np.float32)) for _ in range(2)]
    Y = torch().full((2, 8), 7.0, dtype=torch().float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, d, tsl.F32, 0, 8, 8, tsl.F32, Y, 8)
    tsl.combine_partials(tsl.COMBINE_CONCAT, d, tsl.F32, 2, 0, 8, tsl.F32, Y, 8)
    assert (Y.cpu().numpy() == 7.0).all()
