"""Products that read their X rows through a row index (tsl_linear_item
row_index): the tokens routed to an expert are read where they lie
([mlxcel] "MoE expert parallelization").  Each case runs the same products
twice, once through the index and once on rows gathered beforehand by
moe_gather (the same meaning of the index: a row of zeros for an index
outside [0, x_rows)), and the outputs agree value for value: 4-bit weights
above 64 rows (the activation pass reads through the index), 4-bit
decode-sized rows, bf16 and fp32 weights (the call gathers into its
workspace); items sharing an X and an index share one copy; a joined sum
set whose members read through indices; and the MoE layout of
moe_dispatch.  The 4-bit products also match the oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, empty_bytes, host, normwise, pack, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


def run_group(items, wdtype, M):
    t = torch()
    ws = tsl.shard_linear_group_workspace_size(items, wdtype, M)
    wb = empty_bytes(ws) if ws else None
    tsl.shard_linear_group(items, wdtype, tsl.F32 if wdtype == tsl.F32 else tsl.BF16, M, wb, ws)
    t.cuda.synchronize()


def gathered(X, ldx, x_rows, dtype, idx, M, K):
    t = torch()
    out = t.empty((M, K), dtype=X.dtype, device="cuda")
    tsl.moe_gather(X, ldx, x_rows, dtype, idx, M, K, out, K)
    return out


def weight(wdtype, K, N, seed):
    """(pack function, oracle f64 weight or None)."""
    if wdtype == tsl.Q4G64:
        w = Q4Weight(K, N, seed, seed + 1, seed + 2)
        return w.pack, oracle.dequant_q4(w.codes, w.scales, w.biases)
    if wdtype == tsl.BF16:
        W = dev(synth.normal_bf16(seed, (K, N), 0.02))
        return (lambda sh: pack(sh, tsl.BF16, W, N, 1)), None
    W = dev(synth.normal_f32(seed, (K, N), 0.02))
    return (lambda sh: pack(sh, tsl.F32, W, N, 1)), None


@pytest.mark.parametrize("wdtype", ["q4", "bf16", "f32"])
@pytest.mark.parametrize("M", [300, 16, 4])
def test_row_index_matches_gathered_rows(wdtype, M):
    """Three column products of one weight over X [150, K]: two read it
    through the same index (one shared copy), one through another; indices
    repeat rows, and -1 and x_rows + 5 read rows of zeros."""
    t = torch()
    code = {"q4": tsl.Q4G64, "bf16": tsl.BF16, "f32": tsl.F32}[wdtype]
    K, N, x_rows = 1024, 384, 150
    print("row index %s M=%d" % (wdtype, M), flush=True)
    if code == tsl.F32:
        Xh = synth.normal_f32(9100 + M, (x_rows, K))
        X = dev(Xh)
    else:
        Xh = synth.normal_bf16(9100 + M, (x_rows, K))
        X = dev(Xh)
    xd = tsl.F32 if code == tsl.F32 else tsl.BF16
    rng = np.random.default_rng(9101 + M)
    idx = [rng.integers(0, x_rows, M).astype(np.int32) for _ in range(2)]
    idx[0][0] = -1
    idx[1][M - 1] = x_rows + 5
    didx = [dev(i) for i in idx]
    packf, Wf = weight(code, K, N, 9102)
    sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64 if code == tsl.Q4G64 else 0)[0]
    buf, nb = packf(sh)
    ydt = t.float32
    which = (0, 0, 1)
    Ys = [t.full((M, N), float("nan"), dtype=ydt, device="cuda") for _ in which]
    run_group([dict(shard=sh, packed=buf, packed_bytes=nb, X=X, ldx=K, Y=Y, ldy=N,
                    row_index=didx[w], x_rows=x_rows) for w, Y in zip(which, Ys)], code, M)
    # the same call (same plan: the same k-splits) over rows gathered first
    Gs = [gathered(X, K, x_rows, xd, didx[w], M, K) for w in range(2)]
    wants = [t.full((M, N), float("nan"), dtype=ydt, device="cuda") for _ in which]
    run_group([dict(shard=sh, packed=buf, packed_bytes=nb, X=Gs[w], ldx=K, Y=Y, ldy=N)
               for w, Y in zip(which, wants)], code, M)
    for w, Y, want in zip(which, Ys, wants):
        assert np.array_equal(host(Y), host(want)), (wdtype, M, w)
        bad = (idx[w] < 0) | (idx[w] >= x_rows)
        assert np.all(host(Y)[bad] == 0)
        if Wf is not None:
            Xg = oracle.bf16_to_f64(Xh)[np.clip(idx[w], 0, x_rows - 1)]
            Xg[bad] = 0.0
            assert normwise(host(Y), oracle.gemm(Xg, Wf)) <= TOL


@pytest.mark.parametrize("wdtype", ["q4", "bf16"])
def test_row_index_in_a_joined_sum_set(wdtype):
    """Row shards of one weight as a sum set, every member reading its
    k-range of X [200, K] through one index: the same output as the set
    over rows gathered beforehand."""
    t = torch()
    code = tsl.Q4G64 if wdtype == "q4" else tsl.BF16
    M, K, N, tp, x_rows = 300, 2048, 512, 4, 200
    X = dev(synth.normal_bf16(9200, (x_rows, K)))
    rng = np.random.default_rng(9201)
    idx = dev(rng.integers(0, x_rows, M).astype(np.int32))
    packf, _ = weight(code, K, N, 9202)
    shards = tsl.plan_linear(K, N, tp, tsl.ROW, 64)
    packs = [packf(sh) for sh in shards]
    G = gathered(X, K, x_rows, tsl.BF16, idx, M, K)
    outs = []
    for src in ("index", "gathered"):
        Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        items = []
        for r, (sh, (b, nb)) in enumerate(zip(shards, packs)):
            it = dict(shard=sh, packed=b, packed_bytes=nb, ldx=K, Y=Y if r == 0 else None,
                      ldy=N, sum_next=int(r < tp - 1))
            if src == "index":
                it.update(X=X[:, sh.k_off:], row_index=idx, x_rows=x_rows)
            else:
                it.update(X=G[:, sh.k_off:])
            items.append(it)
        run_group(items, code, M)
        outs.append(Y)
    assert t.equal(outs[0], outs[1])


@pytest.mark.parametrize("wdtype,T", [("q4", 600), ("q4", 8), ("q4", 160), ("bf16", 160),
                                      ("bf16", 400)])
def test_row_index_in_the_moe_layout(wdtype, T):
    """16 experts, top-2 routing, one rank holding 8 experts: every held
    expert's gate product reads its tokens through its run of
    moe_dispatch's row layout (row_slot / k) -- the same outputs as
    moe_gather followed by the products over the gathered rows.  4-bit
    weights: about 75 rows an expert at T = 600 (the activation pass reads
    through the index), at most a few at T = 8 (the resident streaming
    kernel does), about 20 at T = 160 (windowed: the call gathers); bf16
    weights: about 20 and 50 rows (the call gathers; the experts' runs
    follow one another, so their gathers merge into one)."""
    t = torch()
    n_exp, k, H, F = 16, 2, 1024, 256
    rng = np.random.default_rng(9300 + T)
    topk = np.stack([rng.choice(n_exp, k, replace=False) for _ in range(T)]).astype(np.int32)
    held = list(range(0, n_exp, 2))
    off, row_slot, _ = tsl.moe_dispatch(topk, n_exp, held)
    R = int(off[-1])
    tok = dev((row_slot[:R] // k).astype(np.int32))
    X = dev(synth.normal_bf16(9301 + T, (T, H)))
    Xp = gathered(X, H, T, tsl.BF16, tok, R, H)
    sh = tsl.plan_linear(H, F, 1, tsl.COLUMN, 64)[0]
    if wdtype == "q4":
        code = tsl.Q4G64
        ws_ = [Q4Weight(H, F, 9310 + 3 * e, 9311 + 3 * e, 9312 + 3 * e) for e in held]
        packs = [w.pack(sh) for w in ws_]
    else:
        code = tsl.BF16
        Ws = [dev(synth.normal_bf16(9310 + e, (H, F), 0.02)) for e in held]
        packs = [pack(sh, tsl.BF16, W, F, 1) for W in Ws]
    Mmax = max(int(off[i + 1] - off[i]) for i in range(len(held)))
    Ya = t.full((R, F), float("nan"), dtype=t.float32, device="cuda")
    Yb = t.full((R, F), float("nan"), dtype=t.float32, device="cuda")
    ia, ib = [], []
    for i in range(len(held)):
        o, rows = int(off[i]), int(off[i + 1] - off[i])
        if rows == 0:
            continue
        b, nb = packs[i]
        ia.append(dict(shard=sh, packed=b, packed_bytes=nb, X=X, ldx=H, Y=Ya[o:], ldy=F,
                       rows=rows, row_index=tok[o:], x_rows=T))
        ib.append(dict(shard=sh, packed=b, packed_bytes=nb, X=Xp[o:], ldx=H, Y=Yb[o:], ldy=F,
                       rows=rows))
    run_group(ia, code, Mmax)
    run_group(ib, code, Mmax)
    assert t.equal(Ya, Yb), (wdtype, T, Mmax)
