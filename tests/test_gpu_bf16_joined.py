"""bf16 weights above 64 rows: a sum set of row shards (mlxcel manual
"Tensor parallelism", "Row Parallel": the ranks' partial products added
into one output) whose members' k-ranges are whole 64-k stages runs as one
GEMM over the members' k-ranges end to end -- the rank sum happens inside
the GEMM, with no binary32 rank partials, each member's activations read
at their own row stride.  Such a set gives bit for bit the unsharded
product of the same plan (the same k-splits, so the same accumulation
order) and the oracle's rank sum to the bf16 tolerance; a set that cannot
be joined keeps the partials and gives the members' products followed by
the ordered sum."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, empty_bytes, host, host_bits, normwise, pack, spec_dict, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


def run_group(items, M):
    ws = tsl.shard_linear_group_workspace_size(items, tsl.BF16, M)
    wb = empty_bytes(ws) if ws else None
    tsl.shard_linear_group(items, tsl.BF16, tsl.BF16, M, wb, ws)
    torch().cuda.synchronize()


def weights_and_input(M, K, N, seed, integer):
    if integer:
        W = synth.small_int_bf16(seed, (K, N), -3, 3)
        X = synth.small_int_bf16(seed + 1, (M, K), -3, 3)
    else:
        W = synth.normal_bf16(seed, (K, N), 0.02)
        X = synth.normal_bf16(seed + 1, (M, K))
    return W, X


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("M,K,N,tp", [(100, 2048, 4096, 4), (300, 4096, 640, 4),
                                      (65, 1024, 264, 8), (257, 14336, 512, 8),
                                      (257, 3584, 512, 8), (513, 2048, 2048, 2)])
def test_joined_bf16_sum_set_equals_unsharded_product(M, K, N, tp, integer):
    """Members of 512, 1024, 128, 1792, 448 and 1024 k.  The two N = 512
    launches have a few tiles, so the joined product is split along k:
    at K = 14336 into parts of whole members, at K = 3584 into 7 parts of 8
    stages over members of 7 stages (parts straddle members).  Ragged row
    and column tiles; binary32 and bf16 outputs.  Integer operands: every
    sum is exact, so the result equals the oracle's exactly."""
    t = torch()
    print("bf16 joined set M=%d K=%d N=%d tp=%d integer=%d" % (M, K, N, tp, integer), flush=True)
    Wb, Xb = weights_and_input(M, K, N, 8100 + K + N, integer)
    dW, dX = dev(Wb), dev(Xb)
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    assert all(sh.k_len % 64 == 0 for sh in shards)
    packs = [pack(sh, tsl.BF16, dW, N, 1) for sh in shards]
    full = tsl.plan_linear(K, N, 1, tsl.ROW, 64)[0]
    fbuf, fnb = pack(full, tsl.BF16, dW, N, 1)
    Xf, Wf = oracle.bf16_to_f64(Xb), oracle.bf16_to_f64(Wb)
    ref = oracle.combine_sum([oracle.gemm(oracle.slice_input(Xf, spec_dict(sh)),
                                          Wf[sh.k_off:sh.k_off + sh.k_len]) for sh in shards])
    for ydt, tdt in ((tsl.F32, t.float32), (tsl.BF16, t.bfloat16)):
        want = t.full((M, N), float("nan"), dtype=tdt, device="cuda")
        run_group([dict(shard=full, packed=fbuf, packed_bytes=fnb, X=dX, ldx=K, Y=want, ldy=N,
                        ydtype=ydt)], M)
        Y = t.full((M, N), float("nan"), dtype=tdt, device="cuda")
        run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=K,
                        Y=Y if r == 0 else None, ldy=N, ydtype=ydt, sum_next=int(r < tp - 1))
                   for r, (sh, (b, nb)) in enumerate(zip(shards, packs))], M)
        assert np.array_equal(host_bits(Y), host_bits(want)), (M, K, N, ydt)
        if integer:
            assert np.max(np.abs(ref)) < 2 ** 24
            if ydt == tsl.F32:
                assert np.array_equal(host(Y), ref)
            else:
                assert np.array_equal(host_bits(Y), oracle.f64_to_bf16(ref))
        else:
            assert normwise(host(Y), ref) <= TOL + (2.0 ** -9 if ydt == tsl.BF16 else 0.0)


def test_joined_bf16_members_in_their_own_buffers():
    """Each member's activations in a buffer of its own ([M, k_len], row
    stride k_len): the GEMM reads each stage from its member's buffer --
    bit for bit the unsharded product over the concatenated activations."""
    t = torch()
    M, K, N, tp = 300, 3072, 768, 4
    Wb, Xb = weights_and_input(M, K, N, 8200, False)
    dW, dX = dev(Wb), dev(Xb)
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    own = [dev(np.ascontiguousarray(Xb[:, sh.k_off:sh.k_off + sh.k_len])) for sh in shards]
    packs = [pack(sh, tsl.BF16, dW, N, 1) for sh in shards]
    full = tsl.plan_linear(K, N, 1, tsl.ROW, 64)[0]
    fbuf, fnb = pack(full, tsl.BF16, dW, N, 1)
    want = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    run_group([dict(shard=full, packed=fbuf, packed_bytes=fnb, X=dX, ldx=K, Y=want, ldy=N)], M)
    Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=x, ldx=sh.k_len,
                    Y=Y if r == 0 else None, ldy=N, sum_next=int(r < tp - 1))
               for r, (sh, (b, nb), x) in enumerate(zip(shards, packs, own))], M)
    assert t.equal(Y, want)
    ref = oracle.gemm(oracle.bf16_to_f64(Xb), oracle.bf16_to_f64(Wb))
    assert normwise(host(Y), ref) <= TOL


def test_joined_bf16_members_with_different_row_strides():
    """Member 0 reads its activations from a wider copy (row stride
    K + 64), the others from X (stride K): the set still joins (its
    members' strides travel with their bases) -- bit for bit the unsharded
    product over X."""
    t = torch()
    M, K, N, tp = 300, 4096, 640, 4
    Wb, Xb = weights_and_input(M, K, N, 8300 + K, False)
    dW, dX = dev(Wb), dev(Xb)
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    packs = [pack(sh, tsl.BF16, dW, N, 1) for sh in shards]
    wide = np.zeros((M, K + 64), dtype=np.uint16)
    wide[:, :K] = Xb
    dWide = dev(wide)
    full = tsl.plan_linear(K, N, 1, tsl.ROW, 64)[0]
    fbuf, fnb = pack(full, tsl.BF16, dW, N, 1)
    want = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    run_group([dict(shard=full, packed=fbuf, packed_bytes=fnb, X=dX, ldx=K, Y=want, ldy=N)], M)
    Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    run_group([dict(shard=sh, packed=b, packed_bytes=nb,
                    X=(dWide if r == 0 else dX)[:, sh.k_off:], ldx=K + 64 if r == 0 else K,
                    Y=Y if r == 0 else None, ldy=N, sum_next=int(r < tp - 1))
               for r, (sh, (b, nb)) in enumerate(zip(shards, packs))], M)
    assert t.equal(Y, want)


def test_bf16_sum_set_that_is_not_joined():
    """Members whose k-ranges are not whole 64-k stages (K = 1152 over 4
    ranks: 288 k): the set keeps its binary32 rank partials -- bit for bit
    the members' products followed by combine_partials(SUM), and the
    oracle's sum."""
    t = torch()
    M, K, N, tp = 200, 1152, 512, 4
    Wb, Xb = weights_and_input(M, K, N, 8300 + K, False)
    dW, dX = dev(Wb), dev(Xb)
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 0)
    assert all(sh.k_len == K // tp and sh.k_len % 64 for sh in shards)
    packs = [pack(sh, tsl.BF16, dW, N, 1) for sh in shards]
    ps = [t.full((M, N), float("nan"), dtype=t.float32, device="cuda") for _ in shards]
    run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=K, Y=P, ldy=N)
               for sh, (b, nb), P in zip(shards, packs, ps)], M)
    want = t.empty((M, N), dtype=t.float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, ps, tsl.F32, M, N, N, tsl.F32, want, N)
    Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=K,
                    Y=Y if r == 0 else None, ldy=N, sum_next=int(r < tp - 1))
               for r, (sh, (b, nb)) in enumerate(zip(shards, packs))], M)
    assert t.equal(Y, want)
    ref = oracle.gemm(oracle.bf16_to_f64(Xb), oracle.bf16_to_f64(Wb))
    assert normwise(host(Y), ref) <= TOL


def test_more_joined_bf16_sets_than_one_launch_takes():
    """20 joined sets of 2 members between lone column products: a launch
    holds the member tables of 16 joined sets, so the group runs as more
    launches than its item count alone asks for; every set equals its
    unsharded product bit for bit and every lone product its oracle."""
    t = torch()
    M, K, N = 130, 512, 96
    full = tsl.plan_linear(K, N, 1, tsl.ROW, 64)[0]
    halves = tsl.plan_linear(K, N, 2, tsl.ROW, 64)
    col = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
    items, checks, keep = [], [], []
    for s in range(20):
        Wb, Xb = weights_and_input(M, K, N, 8400 + 7 * s, False)
        dW, dX = dev(Wb), dev(Xb)
        keep += [dW, dX]
        fb = pack(full, tsl.BF16, dW, N, 1)
        want = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        run_group([dict(shard=full, packed=fb[0], packed_bytes=fb[1], X=dX, ldx=K, Y=want,
                        ldy=N)], M)
        Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        for r, sh in enumerate(halves):
            b, nb = pack(sh, tsl.BF16, dW, N, 1)
            keep.append(b)
            items.append(dict(shard=sh, packed=b, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=K,
                              Y=Y if r == 0 else None, ldy=N, sum_next=int(r == 0)))
        checks.append(("set", Y, want))
        if s % 3 == 0:  # a lone product between the sets
            cb, cnb = pack(col, tsl.BF16, dW, N, 1)
            Yc = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
            keep.append(cb)
            items.append(dict(shard=col, packed=cb, packed_bytes=cnb, X=dX, ldx=K, Y=Yc, ldy=N))
            checks.append(("lone", Yc, oracle.gemm(oracle.bf16_to_f64(Xb),
                                                    oracle.bf16_to_f64(Wb))))
    run_group(items, M)
    for kind, Y, want in checks:
        if kind == "set":
            assert t.equal(Y, want)
        else:
            assert normwise(host(Y), want) <= TOL
