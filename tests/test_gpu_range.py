"""4-bit shard products over the whole bf16 range, against the oracle.

[wiki] "Tensor parallel processing", "Details" §1 defines the rank's product
Y_i = X_i W_i for whatever the activations hold.  The GEMM regime (M > 64)
feeds the matrix cores binary16 operands; these tests put into it what a
plain binary16 narrowing would break: activation rows of 1e6, 1e-30, bf16
subnormals, single elements of +-3e38 or of 65536, per-element magnitudes
2^+-60 apart, weight columns whose scales sit 10^+-30 apart with groups a
further 2^+-20 apart, and integer rows up to 2^20 checked bit for bit --
alone, in a grouped call, and inside joined row-shard sum sets whose
members' blocks differ in magnitude.  Tolerance 2e-3 (4-bit, binary32
accumulate), measured per row (activations) or per column (weights)."""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, host, linear, normwise, spec_dict, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


def per_row(y, r):
    """Largest over rows of max_j |y - r| / max_j |r| (rows of zeros skipped)."""
    den = np.max(np.abs(r), axis=1)
    num = np.max(np.abs(y - r), axis=1)
    ok = den > 0
    assert np.all(num[~ok] == 0)
    return float(np.max(num[ok] / den[ok])) if ok.any() else 0.0


def q4_wide_weight(K, N, seed):
    w = Q4Weight(K, N, seed, seed + 1, seed + 2)
    w.scales = synth.wide_scales_bf16(seed + 3, (K // 64, N))
    w.biases = synth.wide_biases_bf16(seed + 4, w.scales)
    w.d_scales, w.d_biases = dev(w.scales), dev(w.biases)
    return w


@pytest.mark.parametrize("M", [65, 300, 2048])
@pytest.mark.parametrize("K,N", [(1024, 272), (640, 96)])
def test_wide_activation_rows(M, K, N):
    X = synth.wide_rows_bf16(5000 + M, M, K)
    Xf = oracle.bf16_to_f64(X)
    assert np.all(np.isfinite(Xf)) and np.max(np.abs(Xf)) > 1e38
    w = Q4Weight(K, N, 5001, 5002, 5003)
    sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
    buf, nb = w.pack(sh)
    Y = host(linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dev(X), K, M))
    ref = oracle.gemm(Xf, w.shard_f64(spec_dict(sh)))
    assert np.all(np.isfinite(ref))
    assert per_row(Y, ref) <= TOL, M
    assert normwise(Y, ref) <= TOL


@pytest.mark.parametrize("M", [65, 300, 2048])
def test_wide_weight_columns(M):
    K, N = 1024, 400
    w = q4_wide_weight(K, N, 5100)
    X = synth.normal_bf16(5105 + M, (M, K))
    for sh in tsl.plan_linear(K, N, 2, tsl.COLUMN, 64):
        s = spec_dict(sh)
        buf, nb = w.pack(sh)
        Y = host(linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dev(X), K, M))
        ref = oracle.gemm(oracle.bf16_to_f64(X), w.shard_f64(s))
        assert np.all(np.isfinite(ref))
        assert per_row(Y.T, ref.T) <= TOL, (M, s["rank"])


@pytest.mark.parametrize("M", [65, 300, 2048])
def test_integer_rows_to_2_pow_20_bit_exact(M):
    # |Y| <= 2^20 * 8 + 3 * 8 * K < 2^24: exact in binary32 in any order
    K, N = 1024, 144
    X = synth.big_int_rows_bf16(5200 + M, M, K)
    Xf = oracle.bf16_to_f64(X)
    w = Q4Weight(K, N, 5201, 5202, 5203, integer=True)
    sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
    buf, nb = w.pack(sh)
    Y = host(linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dev(X), K, M))
    ref = oracle.gemm(Xf, w.shard_f64(spec_dict(sh)))
    assert np.max(np.abs(ref)) < 2 ** 24
    assert np.array_equal(Y, ref)
    # bf16 output: the exact product rounded once, nearest even
    Yb = host(linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, dev(X), K, M, ydtype=tsl.BF16))
    assert np.array_equal(Yb, oracle.bf16_to_f64(oracle.f64_to_bf16(ref)))


def run_group(items, M):
    t = torch()
    ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, M)
    wsb = t.empty(max(ws, 256), dtype=t.uint8, device="cuda")
    tsl.shard_linear_group(items, tsl.Q4G64, tsl.BF16, M, wsb, ws)


@pytest.mark.parametrize("M,integer", [(300, False), (2048, False), (300, True)])
def test_joined_sum_set_members_of_different_magnitude(M, integer):
    """Row shards of one 4-bit weight as a sum set (joined along k in the
    GEMM regime): rank r's activation block is scaled by 2^(20 r) (random
    draws) or holds integers up to 2^20 (integer draws), and rank r's rows
    of W use scales 2^(10 r) apart; the set's one row and column exponent
    must cover every member (with per-member exponents rank 3's binary16
    operands would overflow)."""
    t = torch()
    K, N, tp = 2048, 264, 4
    w = Q4Weight(K, N, 5300, 5301, 5302, integer=integer)
    if integer:
        X = synth.big_int_rows_bf16(5303, M, K)
    else:
        xs = synth.bf16_bits_to_f32(synth.normal_bf16(5303, (M, K)))
        xs = xs * np.repeat(np.exp2(20.0 * np.arange(tp)), K // tp).astype(np.float32)
        X = synth.f32_to_bf16_bits(xs)
        sc = synth.bf16_bits_to_f32(w.scales)
        sc = sc * np.repeat(np.exp2(10.0 * np.arange(tp)), K // 64 // tp)[:, None]
        w.scales = synth.f32_to_bf16_bits(sc.astype(np.float32))
        w.biases = synth.wide_biases_bf16(5304, w.scales, 0.5)
        w.d_scales, w.d_biases = dev(w.scales), dev(w.biases)
    Xf = oracle.bf16_to_f64(X)
    dX = dev(X)
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    packs = [w.pack(sh) for sh in shards]
    ref = oracle.combine_sum([oracle.gemm(oracle.slice_input(Xf, spec_dict(sh)),
                                          w.shard_f64(spec_dict(sh))) for sh in shards])
    Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=K,
                    Y=Y if r == 0 else None, ldy=N, ydtype=tsl.F32, sum_next=int(r < tp - 1))
               for r, (sh, (b, nb)) in enumerate(zip(shards, packs))], M)
    if integer:
        assert np.max(np.abs(ref)) < 2 ** 24
        assert np.array_equal(host(Y), ref)
    else:
        assert per_row(host(Y), ref) <= TOL


def test_grouped_items_share_and_do_not_share_row_scales():
    """Three products in one call: two read the same wide-range X (one
    activation copy and one set of row exponents), one reads a different
    X of ordinary magnitude; each matches its own oracle product."""
    t = torch()
    M, K = 300, 1024
    Xa = synth.wide_rows_bf16(5400, M, K)
    Xb = synth.normal_bf16(5401, (M, K))
    dA, dB = dev(Xa), dev(Xb)
    ws_ = [Q4Weight(K, n, 5402 + 3 * i, 5403 + 3 * i, 5404 + 3 * i)
           for i, n in enumerate((256, 96, 160))]
    items, outs, refs = [], [], []
    for i, (w, dx, xb) in enumerate(zip(ws_, (dA, dA, dB), (Xa, Xa, Xb))):
        sh = tsl.plan_linear(K, w.N, 1, tsl.COLUMN, 64)[0]
        buf, nb = w.pack(sh)
        Y = t.full((M, w.N), float("nan"), dtype=t.float32, device="cuda")
        items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=dx, ldx=K, Y=Y, ldy=w.N,
                          ydtype=tsl.F32))
        outs.append(Y)
        refs.append(oracle.gemm(oracle.bf16_to_f64(xb), w.shard_f64(spec_dict(sh))))
    run_group(items, M)
    for Y, ref in zip(outs, refs):
        assert per_row(host(Y), ref) <= TOL
