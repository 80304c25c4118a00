"""Vocabulary-parallel embedding and LM head on the GPU against the oracle.

embed_lookup: every rank's partial is its owned rows copied bit for bit
(widened exactly, or rounded to nearest-even for binary32 tables read into
bf16) and -0.0 elsewhere; the rank-ordered binary32 sum of the partials is
then the full lookup bit for bit, a -0.0 table entry included.  Covers the
16-byte and scalar paths, a column block of the table, ids on every slice
edge, ids outside the vocabulary, and the full 152064-token vocabulary.

LM head: the rank's column shard over the vocabulary through
shard_linear_group, every rank writing its slice of the full logits
(concat-free), against the oracle on sampled vocabulary columns (all token
rows); random draws max|y - r| / max|r| <= 2e-3, integer draws bit-exact.
"""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, empty_bytes, host, host_bits, normwise, spec_dict, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import configs, synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
NEG0_F32, NEG0_BF16 = 0x80000000, 0x8000


def edge_tokens(vocab, tp, seed, M):
    """Ids on both sides of every slice edge, out-of-range ids, repeats and
    uniform draws."""
    w = vocab // tp
    edges = []
    for r in range(tp + 1):
        edges += [r * w - 1, r * w, r * w + 1]
    special = [-1, vocab, 2 ** 31 - 1, -2 ** 31, 5, 5]
    rest = synth.token_ids(seed, max(M - len(edges) - len(special), 0), vocab)
    return np.concatenate([np.array(edges + special, dtype=np.int64), rest]).astype(np.int32)


def table_f64(E, tdt):
    return oracle.bf16_to_f64(E) if tdt == "bf16" else E.astype(np.float64)


def run_lookup(shards, dE, ld, tdt, d_tok, M, ydt):
    t = torch()
    code = tsl.F32 if tdt == "f32" else tsl.BF16
    ycode, ytype = (tsl.F32, t.float32) if ydt == "f32" else (tsl.BF16, t.bfloat16)
    outs = []
    for sh in shards:
        Y = t.full((M, sh.n_len), float("nan"), dtype=ytype, device="cuda")
        tsl.embed_lookup(sh, code, dE[sh.k_off:], ld, d_tok, M, ycode, Y, sh.n_len)
        outs.append(Y)
    return outs


def check_partials(outs, shards, E, tdt, tokens, ydt):
    Ef = table_f64(E, tdt)
    for Y, sh in zip(outs, shards):
        s = spec_dict(sh)
        want = oracle.embed_lookup(Ef, tokens, s)
        owned = (tokens.astype(np.int64) >= s["k_off"]) & (tokens < s["k_off"] + s["k_len"])
        if ydt == "f32":
            got = Y.cpu().numpy()
            bits = got.view(np.uint32)
            assert np.array_equal(got[owned].astype(np.float64), want[owned]), sh.rank
            assert np.all(bits[~owned] == NEG0_F32), sh.rank
        else:
            bits = host_bits(Y)
            assert np.array_equal(bits[owned], oracle.f64_to_bf16(want[owned])), sh.rank
            assert np.all(bits[~owned] == NEG0_BF16), sh.rank


def full_rows(Ef, tokens):
    out = np.zeros((len(tokens), Ef.shape[1]))
    for m, tk in enumerate(tokens):
        if 0 <= tk < Ef.shape[0]:
            out[m] = Ef[tk]
    return out


@pytest.mark.parametrize("tdt,ydt", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32"),
                                     ("f32", "bf16")])
@pytest.mark.parametrize("vocab,hidden,tp,M", [(1024, 96, 4, 61), (1000, 30, 8, 45),
                                              (64, 8, 1, 9), (4096, 260, 2, 300)])
def test_embed_lookup_partials_and_sum(vocab, hidden, tp, M, tdt, ydt):
    t = torch()
    seed = 900 + vocab + hidden
    E = synth.normal_bf16(seed, (vocab, hidden), 0.02) if tdt == "bf16" else \
        synth.normal_f32(seed, (vocab, hidden), 0.02)
    # a -0.0 entry: the sum of the partials must keep its sign
    E[5, 0] = NEG0_BF16 if tdt == "bf16" else np.float32(-0.0)
    tokens = edge_tokens(vocab, tp, seed + 1, M)
    M = len(tokens)
    shards = tsl.plan_vocab(vocab, hidden, tp)[0::2]
    dE, d_tok = dev(E), dev(tokens)
    outs = run_lookup(shards, dE, hidden, tdt, d_tok, M, ydt)
    check_partials(outs, shards, E, tdt, tokens, ydt)
    full = full_rows(table_f64(E, tdt), tokens)
    # sum of binary32 partials: the full lookup, bit for bit
    f32 = outs if ydt == "f32" else run_lookup(shards, dE, hidden, tdt, d_tok, M, "f32")
    Y = t.full((M, hidden), float("nan"), dtype=t.float32, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, f32, tsl.F32, M, hidden, hidden, tsl.F32, Y, hidden)
    got = Y.cpu().numpy()
    assert np.array_equal(got.astype(np.float64), full)
    outside = (tokens.astype(np.int64) < 0) | (tokens >= vocab)
    assert np.all(got[outside].view(np.uint32) == NEG0_F32)  # owned by no rank: -0.0
    row5 = np.nonzero(tokens == 5)[0]
    assert np.all(got[row5, 0].view(np.uint32) == NEG0_F32)  # -0.0 survives the sum
    # every rank's copy of the joined rows (all-reduce), in bf16
    outs_b = [t.full((M, hidden), float("nan"), dtype=t.bfloat16, device="cuda")
              for _ in range(tp)]
    tsl.combine_to_ranks(tsl.ALL_REDUCE, f32, tsl.F32, M, hidden, hidden, tsl.BF16, outs_b,
                         hidden)
    want = oracle.f64_to_bf16(full)
    want[outside] = NEG0_BF16
    for o in outs_b:
        assert np.array_equal(host_bits(o), want)


def test_embed_lookup_column_block_and_strides():
    # a column block of the table (any strategy is a block of W), table and
    # output row strides wider than the block, M = 0
    t = torch()
    vocab, hidden = 256, 64
    E = synth.normal_bf16(31, (vocab, hidden + 8))
    sh = tsl.plan_linear(vocab, hidden, 4, tsl.COLUMN)[2]  # columns 32..47, every token
    tokens = edge_tokens(vocab, 4, 32, 40)
    M = len(tokens)
    Y = t.full((M, 40), float("nan"), dtype=t.float32, device="cuda")
    dE = dev(E)
    tsl.embed_lookup(sh, tsl.BF16, dE[:, sh.n_off:], hidden + 8, dev(tokens), M, tsl.F32, Y, 40)
    Ef = oracle.bf16_to_f64(E[:, :hidden])
    want = oracle.embed_lookup(Ef, tokens, spec_dict(sh))
    got = Y.cpu().numpy()
    inside = (tokens.astype(np.int64) >= 0) & (tokens < vocab)
    assert np.array_equal(got[inside, :16].astype(np.float64), want[inside])
    assert np.all(got[~inside, :16].view(np.uint32) == NEG0_F32)
    assert np.all(np.isnan(got[:, 16:]))  # nothing written past the block
    tsl.embed_lookup(sh, tsl.BF16, dE, hidden + 8, dev(tokens), 0, tsl.F32, Y, 40)


def test_embed_lookup_full_vocabulary():
    """vocab7b: 152064 x 3584 bf16 table, 2048 uniform ids, tp=4."""
    t = torch()
    c = configs.VOCAB7B
    E = synth.normal_bf16(synth.seed_of(c.index, 0, synth.T_W), (c.vocab, c.hidden), c.e_std)
    tokens = edge_tokens(c.vocab, c.tp, synth.seed_of(c.index, 0, synth.T_X), c.lookup_m)
    M = len(tokens)
    shards = tsl.plan_vocab(c.vocab, c.hidden, c.tp)[0::2]
    dE, d_tok = dev(E), dev(tokens)
    outs = run_lookup(shards, dE, c.hidden, "bf16", d_tok, M, "f32")
    Y = t.full((M, c.hidden), float("nan"), dtype=t.bfloat16, device="cuda")
    tsl.combine_partials(tsl.COMBINE_SUM, outs, tsl.F32, M, c.hidden, c.hidden, tsl.BF16, Y,
                         c.hidden)
    bits = host_bits(Y)
    for m, tk in enumerate(tokens):
        want = E[tk] if 0 <= tk < c.vocab else np.full(c.hidden, NEG0_BF16, np.uint16)
        assert np.array_equal(bits[m], want), (m, int(tk))
    check_partials(outs[:1], shards[:1], E, "bf16", tokens, "f32")


@pytest.fixture(scope="module")
def lm_head():
    c = configs.VOCAB7B
    seed = lambda tt: synth.seed_of(c.index, 1, tt)
    return {v: Q4Weight(c.hidden, c.vocab, seed(synth.T_CODES) + iv, seed(synth.T_SCALES) + iv,
                        seed(synth.T_BIASES) + iv, integer=(v == "integer"),
                        scale_lo=c.scale_lo, scale_hi=c.scale_hi, bias_std=c.bias_std)
            for iv, v in enumerate(("random", "integer"))}


@pytest.mark.parametrize("variant", ["random", "integer"])
@pytest.mark.parametrize("M", configs.VOCAB7B.head_ms)
def test_lm_head_logits_vocab_parallel(lm_head, M, variant):
    t = torch()
    c = configs.VOCAB7B
    w = lm_head[variant]
    heads = tsl.plan_vocab(c.vocab, c.hidden, c.tp, 64)[1::2]
    xs = synth.seed_of(c.index, 1, synth.T_X, 1 if variant == "integer" else 0) + M
    X = synth.small_int_bf16(xs, (M, c.hidden)) if variant == "integer" else \
        synth.normal_bf16(xs, (M, c.hidden))
    dX = dev(X)
    logits = t.full((M, c.vocab), float("nan"), dtype=t.float32, device="cuda")
    packs = [w.pack(sh) for sh in heads]
    items = [dict(shard=sh, packed=buf, packed_bytes=nb, X=dX, ldx=c.hidden,
                  Y=logits[:, sh.n_off:], ldy=c.vocab)
             for sh, (buf, nb) in zip(heads, packs)]
    ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, M)
    wsb = empty_bytes(ws) if ws else None
    tsl.shard_linear_group(items, tsl.Q4G64, tsl.BF16, M, wsb, ws)
    got = host(logits)
    assert not np.isnan(got).any()
    rng = synth.rng(77 + M)
    cols = [v for sh in heads for v in (sh.n_off, sh.n_off + 1, sh.n_off + sh.n_len - 1)]
    cols = np.unique(np.concatenate([np.array(cols), rng.choice(c.vocab, 384, replace=False)]))
    Wc = oracle.dequant_q4(w.codes[:, cols], w.scales[:, cols], w.biases[:, cols])
    ref = oracle.gemm(oracle.bf16_to_f64(X), Wc)
    if variant == "integer":
        assert np.array_equal(got[:, cols], ref)
    else:
        assert normwise(got[:, cols], ref) <= TOL


def test_embed_lookup_many_rows():
    """More token rows than one launch's grid height (65535): the rows loop."""
    t = torch()
    vocab, hidden, tp, M = 512, 8, 2, 70001
    E = synth.normal_bf16(41, (vocab, hidden))
    tokens = synth.token_ids(42, M, vocab)
    sh = tsl.plan_vocab(vocab, hidden, tp)[2]  # rank 1
    Y = t.full((M, hidden), float("nan"), dtype=t.float32, device="cuda")
    tsl.embed_lookup(sh, tsl.BF16, dev(E)[sh.k_off:], hidden, dev(tokens), M, tsl.F32, Y, hidden)
    want = oracle.embed_lookup(oracle.bf16_to_f64(E), tokens, spec_dict(sh))
    got = Y.cpu().numpy()
    owned = tokens >= sh.k_off
    assert np.array_equal(got[owned].astype(np.float64), want[owned])
    assert np.all(got[~owned].view(np.uint32) == NEG0_F32)
