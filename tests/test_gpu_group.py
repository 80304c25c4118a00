"""shard_linear_group on the GPU: several shard products in one pass.

Every projection of two ranks of a layer runs as one group (q, k, v read
one activation matrix, gate and up another, o and down their own rank
blocks), each output checked against the oracle like a single call; groups
longer than one launch's item table; column shards writing disjoint blocks
of one output (concat-free); and in the GEMM regime the group's results
equal separate shard_linear calls bit for bit (same kernels, same k order).
"""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, empty_bytes, host, linear, normwise, spec_dict, torch
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
            # GEMM regime: the group equals a separate call bit for bit
            single = linear(sh, wdtype, buf, nb, tsl.BF16, dX[src[proj]][:, sh.k_off:], sh.K, M)
            assert t.equal(single, Y), (proj, r)


@pytest.mark.parametrize("M", [1, 5, 64, 65, 300])
@pytest.mark.parametrize("wdtype", [tsl.Q4G64, tsl.BF16])
def test_long_group_concat_free(M, wdtype):
    """40 column shards (more than one launch holds) of 5 weights, each
    writing its block of the weight's full bf16 output (ldy = N)."""
    t = torch()
    K, N, tp = 384, 320, 8
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
    assert len(items) == 40
    run_group(items, wdtype, M)
    ref_x = oracle.bf16_to_f64(X)
    for outs, full in checks:
        ref = oracle.gemm(ref_x, full)
        err = normwise(host(outs), ref)
        assert err <= TOL + 2.0 ** -9, err
