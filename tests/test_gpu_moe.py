"""Mixture-of-experts FFN products on the GPU against the oracle.

Per rank: moe_dispatch lays out the rows of the rank's experts, moe_gather
collects their inputs, one shard_linear_group call runs every held
expert's gate and up products (each item over its own rows), another the
down products, and moe_combine forms the rank's router-weighted token
outputs; the ranks' outputs are then summed (combine_partials).  Checked:
the gathered rows bit for bit, gate/up rows and the joined output against
the oracle (random draws max|y - r| / max|r| <= 2e-3, integer draws
bit-exact), in both sharding modes, and at the moe30b size on sampled
tokens and columns; each also with the products reading their rows
through the routing's row index instead of gathered copies (as the bench
does).  The activation between gate/up and down is not part of the path:
down reads its own per-slot inputs.
"""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, empty_bytes, host, host_bits, normwise, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import configs, synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


class Experts:
    """Full 4-bit gate, up (W[hidden][ffn]) and down (W[ffn][hidden]) of
    every expert."""

    def __init__(self, c, integer):
        self.c = c
        iv = 1 if integer else 0
        self.w = {}
        for e in range(c.n_experts):
            for pi, (p, K, N) in enumerate((("gate", c.hidden, c.expert_ffn),
                                            ("up", c.hidden, c.expert_ffn),
                                            ("down", c.expert_ffn, c.hidden))):
                s = synth.seed_of(c.index, 10 * e + pi, 0, iv)
                self.w[e, p] = Q4Weight(K, N, s + synth.T_CODES, s + synth.T_SCALES,
                                        s + synth.T_BIASES, integer=integer,
                                        scale_lo=c.scale_lo, scale_hi=c.scale_hi,
                                        bias_std=c.bias_std)

    def f64(self, e, p, spec, cols=None):
        w = self.w[e, p]
        if cols is None:
            return w.shard_f64(spec)
        codes, sc, bi = oracle.slice_q4(w.codes, w.scales, w.biases, spec)
        return oracle.dequant_q4(codes[:, cols], sc[:, cols], bi[:, cols])


def inputs(c, T, integer):
    xs = synth.seed_of(c.index, 0, synth.T_X, 1 if integer else 0) + T
    if integer:
        X = synth.small_int_bf16(xs, (T, c.hidden))
        H = synth.small_int_bf16(xs + 1, (T * c.top_k, c.expert_ffn))
    else:
        X = synth.normal_bf16(xs, (T, c.hidden), c.x_std)
        H = synth.normal_bf16(xs + 1, (T * c.top_k, c.expert_ffn), c.x_std)
    topk, w = synth.router(xs + 2, T, c.top_k, c.n_experts)
    if integer:  # small integer weights keep every sum exact
        w = synth.small_int(xs + 3, (T, c.top_k), 1, 3)
    return X, H, topk, w


def run_rank(c, ex, plan, r, T, dX, dH, topk, dw, via_index=False):
    """One rank's MoE products; returns (rows layout, gathered inputs, gate
    and up rows, the rank's token outputs).  via_index: the products read
    their rows through the routing's row index (tsl_linear_item.row_index)
    instead of the gathered copies."""
    t = torch()
    mine = [(e, sh) for e, rr, sh in plan if rr == r]
    held = [e for e, _ in mine]
    off, row_slot, slot_row = tsl.moe_dispatch(topk, c.n_experts, held)
    R = int(off[-1])
    k = c.top_k
    Yr = t.full((T, c.hidden), float("nan"), dtype=t.float32, device="cuda")
    if R == 0:
        tsl.moe_combine(None, c.hidden, 0, dev(slot_row), dw, T, k, c.hidden, tsl.F32, Yr,
                        c.hidden)
        return off, row_slot, None, None, None, Yr
    d_tok = dev((row_slot // k).astype(np.int32))
    d_slot = dev(row_slot.astype(np.int32))
    Xp = t.empty((R, c.hidden), dtype=t.bfloat16, device="cuda")
    tsl.moe_gather(dX, c.hidden, T, tsl.BF16, d_tok, R, c.hidden, Xp, c.hidden)
    f = mine[0][1].gate.n_len  # the rank's ffn width
    G = t.full((R, f), float("nan"), dtype=t.float32, device="cuda")
    U = t.full((R, f), float("nan"), dtype=t.float32, device="cuda")
    kd = mine[0][1].down
    Hp = t.empty((R, kd.k_len), dtype=t.bfloat16, device="cuda")
    tsl.moe_gather(dH[:, kd.k_off:], c.expert_ffn, T * k, tsl.BF16, d_slot, R, kd.k_len, Hp,
                   kd.k_len)
    P = t.full((R, c.hidden), float("nan"), dtype=t.float32, device="cuda")
    gu, dn = [], []
    for i, (e, sh) in enumerate(mine):
        rows = int(off[i + 1] - off[i])
        if rows == 0:
            continue
        o = int(off[i])
        xin = dict(X=dX, ldx=c.hidden, row_index=d_tok[o:], x_rows=T) if via_index else \
            dict(X=Xp[o:], ldx=c.hidden)
        hin = dict(X=dH[:, kd.k_off:], ldx=c.expert_ffn, row_index=d_slot[o:], x_rows=T * k) \
            if via_index else dict(X=Hp[o:], ldx=kd.k_len)
        for p, Y in (("gate", G), ("up", U)):
            s = getattr(sh, p)
            buf, nb = ex.w[e, p].pack(s)
            gu.append(dict(shard=s, packed=buf, packed_bytes=nb, Y=Y[o:], ldy=f, rows=rows,
                           **xin))
        buf, nb = ex.w[e, "down"].pack(sh.down)
        dn.append(dict(shard=sh.down, packed=buf, packed_bytes=nb, Y=P[o:], ldy=c.hidden,
                       rows=rows, **hin))
    Mmax = int(np.max(np.diff(off)))
    for items in (gu, dn):
        ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, Mmax)
        wb = empty_bytes(ws) if ws else None
        tsl.shard_linear_group(items, tsl.Q4G64, tsl.BF16, Mmax, wb, ws)
    tsl.moe_combine(P, c.hidden, R, dev(slot_row), dw, T, k, c.hidden, tsl.F32, Yr, c.hidden)
    return off, row_slot, Xp, G, U, Yr


def check(got, ref, integer, what):
    if integer:
        assert np.array_equal(got, ref), what
    else:
        err = normwise(got, ref)
        assert err <= TOL, "%s: %.3g" % (what, err)


@pytest.mark.parametrize("via_index", [False, True], ids=["gathered", "row_index"])
@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("mode", [tsl.MOE_EXPERT_PARALLEL, tsl.MOE_WITHIN_EXPERT])
@pytest.mark.parametrize("T", configs.MOE_SMALL.tokens)
def test_moe_ranks_against_oracle(T, mode, integer, via_index):
    t = torch()
    c = configs.MOE_SMALL
    ex = Experts(c, integer)
    X, H, topk, w = inputs(c, T, integer)
    dX, dH, dw = dev(X), dev(H), dev(np.ascontiguousarray(w, dtype=np.float32).ravel())
    plan = [(x.expert, x.rank, x) for x in
            tsl.plan_experts(c.n_experts, c.hidden, c.expert_ffn, c.tp, mode, 64)]
    oplan = oracle.plan_experts(c.n_experts, c.hidden, c.expert_ffn, c.tp, mode, 64)
    Xf, Hf = oracle.bf16_to_f64(X), oracle.bf16_to_f64(H)
    k = c.top_k
    xs = np.repeat(Xf[:, None, :], k, axis=1)
    hs = Hf.reshape(T, k, -1)
    parts = []
    for r in range(c.tp):
        off, row_slot, Xp, G, U, Yr = run_rank(c, ex, plan, r, T, dX, dH, topk, dw, via_index)
        specs = {e: s for e, rr, s in oplan if rr == r}
        if Xp is not None:
            # gathered inputs: bit for bit the token rows of each slot
            assert np.array_equal(host_bits(Xp), X[row_slot // k])
            for p, Y in (("gate", G), ("up", U)):
                ys = oracle.moe_linear_slots(xs, topk, lambda e: ex.f64(e, p, specs[e][p])
                                             if e in specs else None,
                                             next(iter(specs.values()))[p]["n_len"])
                want = ys.reshape(T * k, -1)[row_slot]
                check(host(G if p == "gate" else U), want, integer, "%s rank %d" % (p, r))
        # the rank's token outputs over its own slots
        sd = {e: s["down"] for e, s in specs.items()}
        d0 = next(iter(sd.values()))  # every held expert's down covers the same k block
        hr = hs[:, :, d0["k_off"]:d0["k_off"] + d0["k_len"]]
        ys = oracle.moe_linear_slots(hr, topk, lambda e: ex.f64(e, "down", sd[e])
                                     if e in sd else None, c.hidden)
        want_r = oracle.moe_combine(ys, w, np.isin(topk, list(sd)))
        got_r = host(Yr)
        check(got_r, want_r, integer, "rank %d output" % r)
        none = ~np.isin(topk, list(sd)).any(axis=1)
        assert np.all(Yr.cpu().numpy()[none].view(np.uint32) == 0x80000000)  # -0.0
        parts.append(Yr)
    Y = t.full((T, c.hidden), float("nan"), dtype=t.float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, parts, tsl.F32, T, c.hidden, c.hidden, tsl.F32, Y,
                         c.hidden)
    full = oracle.moe_combine(oracle.moe_linear_slots(
        hs, topk, lambda e: ex.f64(e, "down", {"strategy": oracle.REPLICATED}), c.hidden), w)
    check(host(Y), full, integer, "joined output")


@pytest.mark.parametrize("via_index", [False, True], ids=["gathered", "row_index"])
def test_moe30b_expert_parallel_sampled(via_index):
    """moe30b prefill size, expert parallel: every rank's products (rows
    gathered first, or read through the routing's row index as the bench
    does); the joined output on sampled tokens and columns."""
    t = torch()
    c = configs.MOE30B
    T = c.tokens[0]
    ex = Experts(c, False)
    X, H, topk, w = inputs(c, T, False)
    dX, dH, dw = dev(X), dev(H), dev(np.ascontiguousarray(w).ravel())
    plan = [(x.expert, x.rank, x) for x in
            tsl.plan_experts(c.n_experts, c.hidden, c.expert_ffn, c.tp,
                             tsl.MOE_EXPERT_PARALLEL, 64)]
    parts = []
    rng = synth.rng(606)
    for r in range(c.tp):
        off, row_slot, Xp, G, U, Yr = run_rank(c, ex, plan, r, T, dX, dH, topk, dw, via_index)
        parts.append(Yr)
        # gate rows of a sample: first and last rows of a few experts
        k = c.top_k
        pick = np.unique(np.concatenate([off[:-1][:3], off[1:][:3] - 1,
                                         rng.choice(int(off[-1]), 8, replace=False)]))
        pick = pick[(pick >= 0) & (pick < off[-1])]
        held = [e for e, rr, _ in plan if rr == r]
        for row in pick:
            slot = int(row_slot[row])
            e = int(topk.ravel()[slot])
            assert e in held
            ref = oracle.gemm(oracle.bf16_to_f64(X[slot // k][None, :]),
                              ex.f64(e, "gate", {"strategy": oracle.REPLICATED}))
            assert normwise(host(G)[row][None, :], ref) <= TOL, (r, row)
    Y = t.full((T, c.hidden), float("nan"), dtype=t.float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, parts, tsl.F32, T, c.hidden, c.hidden, tsl.F32, Y,
                         c.hidden)
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 14, replace=False)]))
    cols = np.unique(np.concatenate([[0, c.hidden - 1], rng.choice(c.hidden, 62, replace=False)]))
    Hf = oracle.bf16_to_f64(H).reshape(T, c.top_k, -1)
    ref = np.zeros((len(toks), len(cols)))
    for i, tk in enumerate(toks):
        for j in range(c.top_k):
            e = int(topk[tk, j])
            ref[i] += float(w[tk, j]) * (Hf[tk, j][None, :] @ ex.f64(
                e, "down", {"strategy": oracle.REPLICATED}, cols))[0]
    assert normwise(host(Y)[np.ix_(toks, cols)], ref) <= TOL


def test_moe_combine_many_tokens_and_scalar_path():
    """More tokens than one launch's grid height, and a width that takes the
    one-column path: the router-weighted sum against the oracle."""
    t = torch()
    for T, k, n, R in ((70001, 2, 8, 1000), (300, 3, 10, 500)):
        rng = synth.rng(T + n)
        P = synth.normal_f32(T, (R, n))
        slot_row = rng.integers(-1, R, size=T * k).astype(np.int32)
        w = synth.normal_f32(T + 1, (T, k))
        Y = t.full((T, n), float("nan"), dtype=t.float32, device="cuda")
        tsl.moe_combine(dev(P), n, R, dev(slot_row), dev(w.ravel()), T, k, n, tsl.F32, Y, n)
        ys = np.zeros((T, k, n))
        held = slot_row.reshape(T, k) >= 0
        ys[held] = P[slot_row.reshape(T, k)[held]]
        want = oracle.moe_combine(ys, w, held)
        assert normwise(host(Y), want) <= 1e-6, (T, n)
