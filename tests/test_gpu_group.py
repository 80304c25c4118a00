"""shard_linear_group on the GPU: several shard products in one pass.

Every projection of two ranks of a layer runs as one group (q, k, v read
one activation matrix, gate and up another, o and down their own rank
blocks), each output checked against the oracle like a single call; groups
longer than one launch's item table; column shards writing disjoint blocks
of one output (concat-free); and in the GEMM regime the group's results
match separate shard_linear calls to binary32 rounding (the same kernels;
a launch too small to fill the chip splits k, so a lone call may add its
k-partials in other groupings).
"""
import numpy as np
import pytest

import oracle
from gpu_util import (Q4Weight, dev, empty_bytes, host, host_bits, linear, normwise, spec_dict,
                      torch)
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import configs, synth
from test_gpu_layers import LayerWeights, activations, check, sample_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3


def run_group(items, wdtype, M):
    ws = tsl.shard_linear_group_workspace_size(items, wdtype, M)
    wb = empty_bytes(ws) if ws else None
    tsl.shard_linear_group(items, wdtype, tsl.BF16 if wdtype != tsl.F32 else tsl.F32, M, wb, ws)
    torch().cuda.synchronize()


CASES = [(layer, M) for layer in (configs.LLAMA2K, configs.DEC7B, configs.GQA8, configs.PRE27B)
         for M in layer.ms]


@pytest.mark.parametrize("variant", ["random", "integer"])
@pytest.mark.parametrize("layer,M", CASES, ids=["%s-M%d" % (l.name, m) for l, m in CASES])
def test_layer_group_two_ranks(layer, M, variant):
    t = torch()
    shards = tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                             layer.ffn, layer.tp, layer.group)
    # one input per consumer: attention input (q, k, v), FFN input (gate,
    # up), and the full inputs of o and down (ranks read their blocks)
    src = {"q": "q", "k": "q", "v": "q", "gate": "gate", "up": "gate", "o": "o", "down": "down"}
    X, dX, weights, items, keep = {}, {}, {}, [], []
    for proj in configs.PROJS:
        weights[proj] = LayerWeights(layer, proj, variant)
        if src[proj] == proj:
            X[proj] = activations(layer, proj, M, weights[proj].K, variant)
            dX[proj] = dev(X[proj])
    ranks = sorted({0, layer.tp - 1})
    for r in ranks:
        for pi, proj in enumerate(configs.PROJS):
            sh = shards[r * tsl.NPROJ + pi]
            w = weights[proj]
            buf, nb = w.pack(sh)
            # the last rank's column outputs in bf16: one group, mixed types
            bf = variant == "random" and r != 0 and proj not in ("o", "down")
            Y = t.full((M, sh.n_len), float("nan"), dtype=t.bfloat16 if bf else t.float32,
                       device="cuda")
            x = dX[src[proj]]
            items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=x[:, sh.k_off:],
                              ldx=sh.K, Y=Y, ldy=sh.n_len, ydtype=tsl.BF16 if bf else tsl.F32))
            keep.append((r, proj, sh, buf, nb, Y))
    wdtype = weights["q"].wdtype
    run_group(items, wdtype, M)
    for r, proj, sh, buf, nb, Y in keep:
        s = spec_dict(sh)
        rows = sample_rows(M, sh.k_len, sh.n_len)
        Xf = oracle.bf16_to_f64(X[src[proj]][rows])
        ref = oracle.gemm(oracle.slice_input(Xf, s), weights[proj].shard_f64(s))
        what = "%s M=%d rank %d %s" % (layer.name, M, r, proj)
        if Y.dtype == t.bfloat16:  # one more rounding, half a bf16 ulp
            assert normwise(host(Y)[rows], ref) <= TOL + 2.0 ** -9, what
            continue
        check(host(Y)[rows], ref, variant, what)
        if M > 64 and proj in ("k", "down"):
            # GEMM regime: a separate call computes the same products
            single = linear(sh, wdtype, buf, nb, tsl.BF16, dX[src[proj]][:, sh.k_off:], sh.K, M)
            if variant == "integer":
                assert t.equal(single, Y), (proj, r)
            else:
                assert normwise(host(single), host(Y)) <= 1e-5, (proj, r)


@pytest.mark.parametrize("M", [1, 5, 64, 65, 300])
@pytest.mark.parametrize("wdtype", [tsl.Q4G64, tsl.BF16])
def test_long_group_concat_free(M, wdtype):
    """160 column shards (more than one launch holds) of 5 weights, each
    writing its block of the weight's full bf16 output (ldy = N)."""
    t = torch()
    K, N, tp = 384, 320, 32
    X = synth.normal_bf16(3100 + M, (M, K))
    dX = dev(X)
    items, checks = [], []
    for wi in range(5):
        outs = t.full((M, N), float("nan"), dtype=t.bfloat16, device="cuda")
        if wdtype == tsl.Q4G64:
            q = Q4Weight(K, N, 3200 + wi, 3210 + wi, 3220 + wi)
            full = oracle.dequant_q4(q.codes, q.scales, q.biases)
        else:
            W = synth.normal_bf16(3230 + wi, (K, N), 0.05)
            dW = dev(W)
            full = oracle.bf16_to_f64(W)
        for sh in tsl.plan_linear(K, N, tp, tsl.COLUMN, 64):
            if wdtype == tsl.Q4G64:
                buf, nb = q.pack(sh)
            else:
                from gpu_util import pack
                buf, nb = pack(sh, tsl.BF16, dW, N, 1)
            items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=dX, ldx=K,
                              Y=outs[:, sh.n_off:], ldy=N, ydtype=tsl.BF16))
        checks.append((outs, full))
    assert len(items) == 160
    run_group(items, wdtype, M)
    ref_x = oracle.bf16_to_f64(X)
    for outs, full in checks:
        ref = oracle.gemm(ref_x, full)
        err = normwise(host(outs), ref)
        assert err <= TOL + 2.0 ** -9, err


@pytest.mark.parametrize("variant", ["random", "integer"])
@pytest.mark.parametrize("layer,M", CASES, ids=["%s-M%d" % (l.name, m) for l, m in CASES])
def test_row_layers_as_sum_sets(layer, M, variant):
    """o and down of every rank in one group, each projection's ranks a sum
    set: the on-device rank sum happens inside the grouped call."""
    t = torch()
    shards = tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                             layer.ffn, layer.tp, layer.group)
    items, checks, keep = [], [], []
    for proj in ("o", "down"):
        pi = configs.PROJS.index(proj)
        w = LayerWeights(layer, proj, variant)
        X = activations(layer, proj, M, w.K, variant)
        dX = dev(X)
        bf = variant == "random" and proj == "down"  # one bf16 output
        Y = t.full((M, w.N), float("nan"), dtype=t.bfloat16 if bf else t.float32, device="cuda")
        rows = sample_rows(M, w.K // layer.tp, w.N)
        Xf = oracle.bf16_to_f64(X[rows])
        refs = []
        for r in range(layer.tp):
            sh = shards[r * tsl.NPROJ + pi]
            buf, nb = w.pack(sh)
            keep.append(buf)
            items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=w.K,
                              Y=Y if r == 0 else None, ldy=w.N,
                              ydtype=tsl.BF16 if bf else tsl.F32,
                              sum_next=1 if r < layer.tp - 1 else 0))
            s = spec_dict(sh)
            refs.append(oracle.gemm(oracle.slice_input(Xf, s), w.shard_f64(s)))
        keep.append(dX)
        checks.append((proj, Y, rows, oracle.combine_sum(refs)))
    run_group(items, tsl.Q4G64 if layer.wdtype == configs.Q4 else tsl.BF16, M)
    for proj, Y, rows, ref in checks:
        what = "%s M=%d %s sum set" % (layer.name, M, proj)
        if Y.dtype == t.bfloat16:
            assert normwise(host(Y)[rows], ref) <= TOL + 2.0 ** -9, what
        else:
            check(host(Y)[rows], ref, variant, what)


@pytest.mark.parametrize("M,K,N", [(1, 2048, 4096), (3, 2048, 4096), (16, 2048, 4096),
                                   (100, 1280, 4096), (100, 768, 512)])
def test_sum_set_equals_products_then_combine(M, K, N):
    """A sum set gives the ordered binary32 sum of its members' products:
    bit for bit what separate products + combine_partials(SUM) give when the
    products are computed the same way (here: one group of the same items
    without sets -- at M = 100 the members' 320- and 192-k ranges are not
    joined into one product, and at K = 768, N = 512 the launch has 4 tiles,
    whose products the GEMM splits into k-partials in both calls), and the
    bf16 output is that sum rounded once; the set also matches the oracle."""
    t = torch()
    tp = 4
    w = Q4Weight(K, N, 3300, 3301, 3302)
    X = dev(synth.normal_bf16(3303 + M, (M, K)))
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    packs = [w.pack(sh) for sh in shards]
    parts = [t.full((M, N), float("nan"), dtype=t.float32, device="cuda") for _ in shards]
    plain = [dict(shard=sh, packed=b, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K, Y=P, ldy=N)
             for sh, (b, nb), P in zip(shards, packs, parts)]
    run_group(plain, tsl.Q4G64, M)
    want = t.empty((M, N), dtype=t.float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, parts, tsl.F32, M, N, N, tsl.F32, want, N)
    for ydt, tdt in ((tsl.F32, t.float32), (tsl.BF16, t.bfloat16)):
        Y = t.full((M, N), float("nan"), dtype=tdt, device="cuda")
        sets = [dict(p, Y=Y if r == 0 else None, ydtype=ydt, sum_next=int(r < tp - 1))
                for r, p in enumerate(plain)]
        run_group(sets, tsl.Q4G64, M)
        if ydt == tsl.F32:
            assert t.equal(Y, want)
            Xf = oracle.bf16_to_f64(X.view(t.int16).cpu().numpy().view(np.uint16))
            ref = oracle.gemm(Xf, oracle.dequant_q4(w.codes, w.scales, w.biases))
            assert normwise(host(Y), ref) <= TOL
        else:
            assert np.array_equal(host_bits(Y), oracle.f64_to_bf16(host(want)))


@pytest.mark.parametrize("M,K,N,tp", [(100, 2048, 4096, 4), (100, 8192, 512, 4),
                                      (300, 4608, 640, 4), (65, 1024, 264, 8)])
def test_joined_sum_set_equals_unsharded_product(M, K, N, tp):
    """4-bit weights above 64 rows: a sum set of row shards whose k-ranges
    are whole 128-k records runs as one product over the members' k-ranges
    end to end -- bit for bit the product of the unsharded weight over the
    whole X (same plan, same k-splits: at K = 8192, N = 512 a launch of 8
    tiles split into k-partials), f32 and bf16 outputs; and the oracle's
    rank sum to the 4-bit tolerance."""
    t = torch()
    w = Q4Weight(K, N, 3400, 3401, 3402)
    X = dev(synth.normal_bf16(3403 + M, (M, K)))
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    assert all(sh.k_len % 128 == 0 for sh in shards)
    packs = [w.pack(sh) for sh in shards]
    full = tsl.plan_linear(K, N, 1, tsl.ROW, 64)[0]
    fbuf, fnb = w.pack(full)
    Xf = oracle.bf16_to_f64(X.view(t.int16).cpu().numpy().view(np.uint16))
    refs = []
    for sh in shards:
        s = spec_dict(sh)
        refs.append(oracle.gemm(oracle.slice_input(Xf, s), w.shard_f64(s)))
    ref = oracle.combine_sum(refs)
    for ydt, tdt in ((tsl.F32, t.float32), (tsl.BF16, t.bfloat16)):
        want = t.full((M, N), float("nan"), dtype=tdt, device="cuda")
        run_group([dict(shard=full, packed=fbuf, packed_bytes=fnb, X=X, ldx=K, Y=want, ldy=N,
                        ydtype=ydt)], tsl.Q4G64, M)
        Y = t.full((M, N), float("nan"), dtype=tdt, device="cuda")
        sets = [dict(shard=sh, packed=b, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K,
                     Y=Y if r == 0 else None, ldy=N, ydtype=ydt, sum_next=int(r < tp - 1))
                for r, (sh, (b, nb)) in enumerate(zip(shards, packs))]
        run_group(sets, tsl.Q4G64, M)
        assert np.array_equal(host_bits(Y), host_bits(want)), (M, K, N, ydt)
        assert normwise(host(Y), ref) <= TOL + (2.0 ** -9 if ydt == tsl.BF16 else 0.0)


@pytest.mark.parametrize("wdtype", ["bf16", "q4"])
@pytest.mark.parametrize("M,rows", [(300, (300, 1, 77, 256, 129, 65)), (16, (16, 1, 7, 3)),
                                    (4, (1, 4, 2))])
def test_items_with_their_own_rows(wdtype, M, rows):
    """Items of one call over different row counts (the per-expert products
    of a MoE layer): each equals the oracle over its own rows, nothing is
    written past them, and in the GEMM regime each matches a separate call
    over the same rows (bit for bit on integers, to binary32 rounding
    otherwise) when that call also takes the GEMM."""
    t = torch()
    K, N = 384, 200
    items, keep = [], []
    for i, rw in enumerate(rows):
        sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
        for integer in (False, True):
            seed = 3000 + 10 * i + integer
            if wdtype == "q4":
                w = Q4Weight(K, N, seed, seed + 1, seed + 2, integer=integer)
                buf, nb = w.pack(sh)
                Wf = w.shard_f64(spec_dict(sh))
                code = tsl.Q4G64
            else:
                W = synth.small_int_bf16(seed, (K, N)) if integer else \
                    synth.normal_bf16(seed, (K, N), 0.02)
                from gpu_util import pack
                buf, nb = pack(sh, tsl.BF16, dev(W), N, 1)
                Wf = oracle.bf16_to_f64(W)
                code = tsl.BF16
            X = synth.small_int_bf16(seed + 5, (M, K)) if integer else \
                synth.normal_bf16(seed + 5, (M, K))
            dX = dev(X)
            Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
            items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=dX, ldx=K, Y=Y, ldy=N,
                              rows=rw if rw != M or i % 2 else 0))
            keep.append((rw, integer, X, Wf, Y, sh, buf, nb, dX))
    run_group(items, code, M)
    for rw, integer, X, Wf, Y, sh, buf, nb, dX in keep:
        got = host(Y)
        assert np.isnan(got[rw:]).all(), rw  # rows past the item's own untouched
        ref = oracle.gemm(oracle.bf16_to_f64(X[:rw]), Wf)
        if integer:
            assert np.array_equal(got[:rw], ref), rw
        else:
            assert normwise(got[:rw], ref) <= TOL, rw
        if M > 64 and rw > 64:
            single = linear(sh, code, buf, nb, tsl.BF16, dX, K, rw)
            if integer:
                assert t.equal(single[:rw], Y[:rw]), rw
            else:
                assert normwise(host(single)[:rw], got[:rw]) <= 1e-5, rw


@pytest.mark.parametrize("M,K,N,tp", [(1, 1024, 1000, 8), (2, 512, 264, 2), (3, 4096, 4112, 4),
                                      (4, 2048, 64, 8)])
def test_decode_sum_sets_in_launch(M, K, N, tp):
    """Decode rows whose activations stay resident in LDS: the streaming
    launch adds each sum set itself (2, 4 or 8 members, ragged last
    column tiles, a bf16 and an f32 set in one call) -- bit for bit the
    members' products followed by combine_partials(SUM), and the oracle's
    rank sum to the 4-bit tolerance."""
    t = torch()
    items, plain, parts, checks, keep = [], [], [], [], []
    for s_i, ydt in enumerate((tsl.F32, tsl.BF16)):
        w = Q4Weight(K, N, 3500 + 10 * s_i, 3501, 3502)
        X = dev(synth.normal_bf16(3503 + 10 * s_i + M, (M, K)))
        Y = t.full((M, N), float("nan"), dtype=t.bfloat16 if ydt == tsl.BF16 else t.float32,
                   device="cuda")
        shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
        Xf = oracle.bf16_to_f64(X.view(t.int16).cpu().numpy().view(np.uint16))
        refs, ps = [], []
        for r, sh in enumerate(shards):
            buf, nb = w.pack(sh)
            keep += [buf, X]
            P = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
            ps.append(P)
            items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K,
                              Y=Y if r == 0 else None, ldy=N, ydtype=ydt,
                              sum_next=int(r < tp - 1)))
            plain.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K,
                              Y=P, ldy=N))
            s = spec_dict(sh)
            refs.append(oracle.gemm(oracle.slice_input(Xf, s), w.shard_f64(s)))
        parts.append(ps)
        checks.append((Y, ydt, oracle.combine_sum(refs)))
    run_group(items, tsl.Q4G64, M)
    run_group(plain, tsl.Q4G64, M)
    for (Y, ydt, ref), ps in zip(checks, parts):
        want = t.empty_like(Y)
        tsl.combine_partials(tsl.COMBINE_SUM, ps, tsl.F32, M, N, N, ydt, want, N)
        t.cuda.synchronize()
        assert np.array_equal(host_bits(Y), host_bits(want)), (M, K, N, tp, ydt)
        assert normwise(host(Y), ref) <= TOL + (2.0 ** -9 if ydt == tsl.BF16 else 0.0)


def test_decode_sum_set_across_launches():
    """A decode group of 130 items whose last sum set straddles the
    128-item launch boundary (added by the sum launch) while the set
    before it lies inside the first launch (added in the launch): both
    give the ordered sum of the members' products bit for bit."""
    t = torch()
    M, K, N, tp = 1, 512, 256, 4
    w = Q4Weight(K, N, 3600, 3601, 3602)
    X = dev(synth.normal_bf16(3603, (M, K)))
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    packs = [w.pack(sh) for sh in shards]
    col = tsl.plan_linear(K, N, 2, tsl.COLUMN, 64)[0]
    cbuf, cnb = w.pack(col)
    items, keep = [], []
    # 122 lone column products, then a set at items 122..125 and one at
    # 126..129 (the second launch starts at item 128)
    for i in range(122):
        Yc = t.empty((M, col.n_len), dtype=t.float32, device="cuda")
        keep.append(Yc)
        items.append(dict(shard=col, packed=cbuf, packed_bytes=cnb, X=X, ldx=K, Y=Yc,
                          ldy=col.n_len))
    outs = []
    for s_i in range(2):
        Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        outs.append(Y)
        for r, (sh, (buf, nb)) in enumerate(zip(shards, packs)):
            items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K,
                              Y=Y if r == 0 else None, ldy=N, sum_next=int(r < tp - 1)))
    run_group(items, tsl.Q4G64, M)
    ps = [t.empty((M, N), dtype=t.float32, device="cuda") for _ in shards]
    run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=X[:, sh.k_off:], ldx=K, Y=P, ldy=N)
               for sh, (b, nb), P in zip(shards, packs, ps)], tsl.Q4G64, M)
    want = t.empty((M, N), dtype=t.float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, ps, tsl.F32, M, N, N, tsl.F32, want, N)
    t.cuda.synchronize()
    for Y in outs:
        assert t.equal(Y, want)


@pytest.mark.parametrize("wdtype", ["bf16", "q4"])
@pytest.mark.parametrize("M", [1, 100])
def test_sum_set_of_16_ranks(wdtype, M):
    """A sum set of 16 row shards -- longer than one sum launch takes, so
    its members are never split along k and a combine launch of its own
    adds them: bit for bit the members' products followed by
    combine_partials(SUM) (the same products: one group without the set),
    and the oracle's rank sum to the tolerance of the weight type."""
    t = torch()
    K, N, tp = 4096, 512, 16
    X = synth.normal_bf16(3700 + M, (M, K))
    dX = dev(X)
    Xf = oracle.bf16_to_f64(X)
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    if wdtype == "q4":
        w = Q4Weight(K, N, 3701, 3702, 3703)
        packs = [w.pack(sh) for sh in shards]
        Wf = oracle.dequant_q4(w.codes, w.scales, w.biases)
        code, tol = tsl.Q4G64, TOL
    else:
        from gpu_util import pack
        Wb = synth.normal_bf16(3704, (K, N), 0.02)
        dW = dev(Wb)
        packs = [pack(sh, tsl.BF16, dW, N, 1) for sh in shards]
        Wf = oracle.bf16_to_f64(Wb)
        code, tol = tsl.BF16, TOL
    ps = [t.full((M, N), float("nan"), dtype=t.float32, device="cuda") for _ in shards]
    run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=K, Y=P, ldy=N)
               for sh, (b, nb), P in zip(shards, packs, ps)], code, M)
    want = t.empty((M, N), dtype=t.float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, ps, tsl.F32, M, N, N, tsl.F32, want, N)
    Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
    run_group([dict(shard=sh, packed=b, packed_bytes=nb, X=dX[:, sh.k_off:], ldx=K,
                    Y=Y if r == 0 else None, ldy=N, sum_next=int(r < tp - 1))
               for r, (sh, (b, nb)) in enumerate(zip(shards, packs))], code, M)
    assert t.equal(Y, want)
    assert normwise(host(Y), oracle.gemm(Xf, Wf)) <= tol
