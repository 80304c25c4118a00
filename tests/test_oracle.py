"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to something the pages or mathematics
fix: a value or shape the pages print (fixtures under tests/golden/), a
closed form, an invariant, an exact integer result, or a library routine
(numpy) on small inputs.  A plausible slip in the oracle -- a dropped term,
a wrong sign, a transposed operand, a wrong slice edge or group axis, a
wrong rounding rule or summation order -- fails at least one of them.
"""
import itertools

import numpy as np
import pytest

import oracle
from conftest import golden_rows
from tensor_sharded_linear_plan_amd import synth

STRAT = {"column": oracle.COLUMN, "row": oracle.ROW}
COMM = {"all-gather": oracle.CONCAT, "all-reduce": oracle.SUM, "none": oracle.NONE}


# --------------------------------------------------------------------------
# plan: the page's table, the page's GQA examples, brute-force properties
# --------------------------------------------------------------------------

def test_plan_matches_page_table():
    # mlxcel "Architecture-aware shard plan": strategies and communication
    rows = golden_rows("plan_table.txt")
    for hkv, tp in ((8, 4), (4, 8)):  # K/V sharded, then replicated
        plan = oracle.plan(2048, 32, hkv, 64, 8192, tp)
        for r in range(tp):
            for (name, strat, comm), proj in zip(rows, oracle.PROJS):
                assert name == proj + "_proj"
                s = oracle.spec(plan, r, proj)
                if comm == "gqa":
                    if hkv >= tp:
                        assert (s["strategy"], s["combine"]) == (oracle.COLUMN, oracle.CONCAT)
                    else:
                        assert (s["strategy"], s["combine"]) == (oracle.REPLICATED, oracle.NONE)
                else:
                    assert s["strategy"] == STRAT[strat]
                    assert s["combine"] == COMM[comm]


def test_plan_gqa_examples_from_page():
    # mlxcel "GQA-aware attention sharding", figure examples
    for tp, hq, hkv, _printed, q_per, kv_per, mode in golden_rows("gqa_examples.txt"):
        tp, hq, hkv, q_per = int(tp), int(hq), int(hkv), int(q_per)
        plan = oracle.plan(4096, hq, hkv, 128, 14336, tp)
        for r in range(tp):
            q = oracle.spec(plan, r, "q")
            assert (q["head_off"], q["head_cnt"]) == (r * q_per, q_per)
            for p in ("k", "v"):
                s = oracle.spec(plan, r, p)
                if mode == "sharded":
                    assert s["strategy"] == oracle.COLUMN
                    assert (s["head_off"], s["head_cnt"]) == (r * int(kv_per), int(kv_per))
                    assert s["n_len"] == int(kv_per) * 128
                else:
                    assert s["strategy"] == oracle.REPLICATED
                    assert (s["n_off"], s["n_len"]) == (0, hkv * 128)


def _check_plan_properties(hidden, hq, hkv, hd, ffn, tp):
    plan = oracle.plan(hidden, hq, hkv, hd, ffn, tp)
    for proj in oracle.PROJS:
        specs = [oracle.spec(plan, r, proj) for r in range(tp)]
        for r, s in enumerate(specs):
            assert s["rank"] == r and oracle.PROJS[s["proj"]] == proj
            assert 0 <= s["k_off"] and s["k_off"] + s["k_len"] <= s["K"]
            assert 0 <= s["n_off"] and s["n_off"] + s["n_len"] <= s["N"]
        strat = specs[0]["strategy"]
        if strat == oracle.COLUMN:
            cover = np.zeros(specs[0]["N"], dtype=int)
            for s in specs:
                assert s["k_off"] == 0 and s["k_len"] == s["K"]
                cover[s["n_off"]:s["n_off"] + s["n_len"]] += 1
            assert (cover == 1).all()  # disjoint and covering
            assert [s["n_off"] for s in specs] == sorted(s["n_off"] for s in specs)
        elif strat == oracle.ROW:
            cover = np.zeros(specs[0]["K"], dtype=int)
            for s in specs:
                assert s["n_off"] == 0 and s["n_len"] == s["N"]
                cover[s["k_off"]:s["k_off"] + s["k_len"]] += 1
            assert (cover == 1).all()
        else:
            for s in specs:
                assert (s["k_off"], s["k_len"], s["n_off"], s["n_len"]) == (0, s["K"], 0, s["N"])
    for r in range(tp):
        q, o = oracle.spec(plan, r, "q"), oracle.spec(plan, r, "o")
        g, d = oracle.spec(plan, r, "gate"), oracle.spec(plan, r, "down")
        # the row block of o is exactly the q columns this rank produced
        assert (o["k_off"], o["k_len"]) == (q["n_off"], q["n_len"])
        assert (d["k_off"], d["k_len"]) == (g["n_off"], g["n_len"])
        assert oracle.spec(plan, r, "up")["n_off"] == g["n_off"]
        k = oracle.spec(plan, r, "k")
        if hkv >= tp:
            # GQA locality: every local query head's KV head is local
            for h in range(q["head_off"], q["head_off"] + q["head_cnt"]):
                kvh = h // (hq // hkv)
                assert k["head_off"] <= kvh < k["head_off"] + k["head_cnt"]
        # shapes: q has hq/tp heads of hd
        assert q["n_len"] == (hq // tp) * hd and q["K"] == hidden


def test_plan_properties_brute_force():
    count = 0
    for tp in (1, 2, 4, 8, 16):
        for hkv in (1, 2, 4, 8, 16):
            for ratio in (1, 2, 4, 7):
                hq = hkv * ratio
                if hq % tp or (hkv >= tp and hkv % tp):
                    continue
                for hd, ffn in ((8, 32 * tp), (16, 48 * tp)):
                    _check_plan_properties(64, hq, hkv, hd, ffn, tp)
                    count += 1
    assert count > 40


def test_plan_rejections():
    ok = dict(hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64, ffn=8192, tp=4)
    oracle.plan(**ok)
    cases = [
        (dict(tp=3), oracle.TP_NOT_POW2),
        (dict(tp=6), oracle.TP_NOT_POW2),
        (dict(tp=0), oracle.INVALID),
        (dict(hidden=0), oracle.INVALID),
        (dict(n_q_heads=30), oracle.NOT_DIVISIBLE),      # 30 % 8
        (dict(n_q_heads=24, n_kv_heads=12, tp=8), oracle.NOT_DIVISIBLE),  # 12 >= 8, 12 % 8
        (dict(ffn=8190), oracle.NOT_DIVISIBLE),
        (dict(n_q_heads=48, n_kv_heads=8, tp=32), oracle.NOT_DIVISIBLE),  # 48 % 32
    ]
    for change, code in cases:
        args = dict(ok, **change)
        with pytest.raises(oracle.OracleError) as e:
            oracle.plan(**args)
        assert e.value.code == code, change
    # 4-bit: a row shard edge off a 64 boundary (o: 8 heads * 4 = 32 columns)
    with pytest.raises(oracle.OracleError) as e:
        oracle.plan(2048, 32, 8, 4, 8192, 4, group=64)
    assert e.value.code == oracle.GROUP_ALIGN
    oracle.plan(2048, 32, 8, 64, 8192, 4, group=64)


def test_plan_linear_worked_example_and_properties():
    # wiki "Examples" §1: 1024 -> 2048 on 2 ranks -> two [1024][1024] shards
    g = {r[0]: [int(v) for v in r[1:]] for r in golden_rows("worked_example.txt")}
    K, N, tp = g["in_features"][0], g["out_features"][0], g["num_gpus"][0]
    p = oracle.plan_linear(K, N, tp, oracle.COLUMN)
    for r in range(tp):
        s = dict(zip(oracle.FIELDS, (int(v) for v in p[r])))
        assert [s["k_len"], s["n_len"]] == g["shard_shape"]
        assert s["n_off"] == r * g["shard_shape"][1] and s["combine"] == oracle.CONCAT
    p = oracle.plan_linear(K, N, tp, oracle.ROW)
    for r in range(tp):
        s = dict(zip(oracle.FIELDS, (int(v) for v in p[r])))
        assert (s["k_off"], s["k_len"], s["n_len"]) == (r * 512, 512, 2048)
        assert s["combine"] == oracle.SUM
    with pytest.raises(oracle.OracleError) as e:
        oracle.plan_linear(1024, 2047, 2, oracle.COLUMN)
    assert e.value.code == oracle.NOT_DIVISIBLE
    with pytest.raises(oracle.OracleError) as e:
        oracle.plan_linear(1024, 2048, 3, oracle.COLUMN)
    assert e.value.code == oracle.TP_NOT_POW2
    with pytest.raises(oracle.OracleError) as e:
        oracle.plan_linear(192, 64, 2, oracle.ROW, group=64)  # 96-row shards
    assert e.value.code == oracle.GROUP_ALIGN


# --------------------------------------------------------------------------
# GEMM: library routine, closed forms, exact integers
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 5, 7), (32, 64, 48), (17, 200, 33), (64, 256, 128)])
def test_gemm_vs_numpy_f64(M, K, N):
    X = synth.normal_f32(11, (M, K)).astype(np.float64)
    W = synth.normal_f32(12, (K, N)).astype(np.float64)
    Y = oracle.gemm(X, W)
    R = np.matmul(X, W)
    assert Y.shape == (M, N)
    assert np.max(np.abs(Y - R)) <= 1e-12 * max(1.0, np.max(np.abs(R)))


def test_gemm_closed_forms():
    K = 40
    X = synth.normal_f32(21, (9, K)).astype(np.float64)
    W = synth.normal_f32(22, (K, 13)).astype(np.float64)
    # W = I gives Y = X exactly
    assert np.array_equal(oracle.gemm(X, np.eye(K)), X)
    # a one-hot row of X picks the matching row of W exactly
    E = np.zeros((K, K))
    E[np.arange(K), np.arange(K)[::-1]] = 1.0
    assert np.array_equal(oracle.gemm(E, W), W[::-1])
    # an all-ones row sums the columns of W (integer W: exact)
    Wi = synth.small_int(23, (K, 13)).astype(np.float64)
    assert np.array_equal(oracle.gemm(np.ones((1, K)), Wi)[0], Wi.sum(axis=0))
    # the operand order is X @ W, not W @ X or X @ W^T: a non-square case
    A = np.array([[1.0, 2.0, 3.0]])
    B = np.array([[1.0, 0.0], [0.0, 10.0], [100.0, 0.0]])
    assert np.array_equal(oracle.gemm(A, B), np.array([[301.0, 20.0]]))


def test_gemm_integer_exact_and_sampled():
    X = synth.small_int(31, (24, 300))
    W = synth.small_int(32, (300, 70))
    exact = X.astype(np.int64) @ W.astype(np.int64)
    Y = oracle.gemm(X, W)
    assert np.array_equal(Y, exact.astype(np.float64))
    rows = np.array([0, 5, 23, 23, 11])
    cols = np.array([0, 69, 0, 69, 34])
    assert np.array_equal(oracle.gemm_at(X, W, rows, cols), exact[rows, cols].astype(np.float64))


# --------------------------------------------------------------------------
# The method's invariants: concat of column shards and sum of row partials
# equal the unsharded product (wiki "Details" §1; blog: one logical layer)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_column_shards_concat_to_full(tp):
    X = synth.normal_f32(41, (16, 96)).astype(np.float64)
    W = synth.normal_f32(42, (96, 64)).astype(np.float64)
    full = oracle.gemm(X, W)
    plan = oracle.plan_linear(96, 64, tp, oracle.COLUMN)
    parts = [oracle.shard_forward(dict(zip(oracle.FIELDS, map(int, plan[r]))), X, W)
             for r in range(tp)]
    # bitwise: slicing columns does not change any element's k-sum
    assert np.array_equal(oracle.combine_concat(parts), full)


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_row_shards_sum_to_full(tp):
    Xi = synth.small_int(51, (16, 128))
    Wi = synth.small_int(52, (128, 40))
    plan = oracle.plan_linear(128, 40, tp, oracle.ROW)
    specs = [dict(zip(oracle.FIELDS, map(int, plan[r]))) for r in range(tp)]
    parts = [oracle.shard_forward(s, Xi, Wi) for s in specs]
    exact = (Xi.astype(np.int64) @ Wi.astype(np.int64)).astype(np.float64)
    assert np.array_equal(oracle.combine_sum(parts), exact)
    X = synth.normal_f32(53, (16, 128)).astype(np.float64)
    W = synth.normal_f32(54, (128, 40)).astype(np.float64)
    full = np.matmul(X, W)
    got = oracle.combine_sum([oracle.shard_forward(s, X, W) for s in specs])
    assert np.max(np.abs(got - full)) <= 1e-12 * np.max(np.abs(full))


def test_transformer_layer_shards_reassemble():
    # every projection of a small GQA layer: sharded == unsharded
    for hkv, tp in ((4, 2), (2, 4)):
        plan = oracle.plan(32, 8, hkv, 4, 64, tp)
        for pi, proj in enumerate(oracle.PROJS):
            s0 = oracle.spec(plan, 0, proj)
            X = synth.small_int(60 + pi, (5, s0["K"]))
            W = synth.small_int(70 + pi, (s0["K"], s0["N"]))
            full = (X.astype(np.int64) @ W.astype(np.int64)).astype(np.float64)
            parts = [oracle.shard_forward(oracle.spec(plan, r, proj), X, W) for r in range(tp)]
            if s0["strategy"] == oracle.COLUMN:
                assert np.array_equal(oracle.combine_concat(parts), full)
            elif s0["strategy"] == oracle.ROW:
                assert np.array_equal(oracle.combine_sum(parts), full)
            else:
                for p in parts:
                    assert np.array_equal(p, full)


# --------------------------------------------------------------------------
# 4-bit dequantisation
# --------------------------------------------------------------------------

def test_dequant_closed_forms_and_group_axis():
    K, N = 192, 24
    codes = synth.q4_codes(81, (K, N))
    one = synth.const_bf16((K // 64, N), 1.0)
    m8 = synth.const_bf16((K // 64, N), -8.0)
    # scale 1, bias -8: w = q - 8 exactly
    assert np.array_equal(oracle.dequant_q4(codes, one, m8), codes.astype(np.float64) - 8.0)
    # scale 2, bias 0.5: w = 2q + 0.5 exactly
    two = synth.const_bf16((K // 64, N), 2.0)
    half = synth.const_bf16((K // 64, N), 0.5)
    assert np.array_equal(oracle.dequant_q4(codes, two, half), 2.0 * codes + 0.5)
    # groups run along K (64 input rows of one output column): zeroing the
    # pair (g=1, n=5) zeroes exactly W[64:128, 5]
    s = one.copy()
    b = m8.copy()
    s[1, 5] = 0
    b[1, 5] = 0
    W = oracle.dequant_q4(codes, s, b)
    ref = codes.astype(np.float64) - 8.0
    ref[64:128, 5] = 0.0
    assert np.array_equal(W, ref)


def test_dequant_group_sum_identity():
    # sum_k x_k (s q_k + b) = s sum_k x_k q_k + b sum_k x_k, per group
    K, N = 128, 6
    codes = synth.q4_codes(91, (K, N))
    sc = synth.uniform_bf16(92, (K // 64, N), 0.005, 0.02)
    bi = synth.normal_bf16(93, (K // 64, N), 0.05)
    x = synth.small_int(94, (1, K))
    W = oracle.dequant_q4(codes, sc, bi)
    y = oracle.gemm(x, W)[0]
    s = oracle.bf16_to_f64(sc)
    b = oracle.bf16_to_f64(bi)
    alt = np.zeros(N)
    for g in range(K // 64):
        xs = x[0, 64 * g:64 * (g + 1)].astype(np.float64)
        qs = codes[64 * g:64 * (g + 1)].astype(np.float64)
        alt += s[g] * (xs @ qs) + b[g] * xs.sum()
    assert np.max(np.abs(y - alt)) <= 1e-12 * np.max(np.abs(alt))


# --------------------------------------------------------------------------
# bf16 conversions
# --------------------------------------------------------------------------

def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4300], np.uint16)
    want = [1.0, -2.0, 0.25, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, 128.0]
    got = oracle.bf16_to_f64(bits)
    assert list(got) == want
    assert np.signbit(got[4])


def test_bf16_rounding_rule():
    f = oracle.f64_to_bf16
    assert f(np.array([1 + 2 ** -8]))[0] == 0x3F80          # tie -> even (down)
    assert f(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82      # tie -> even (up)
    assert f(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81  # above the tie
    assert f(np.array([-1.5]))[0] == 0xBFC0
    assert f(np.array([2.0 ** 200]))[0] == 0x7F80            # overflow -> inf
    # every finite bf16 value rounds to itself
    allbits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = allbits[(allbits & 0x7F80) != 0x7F80]
    assert np.array_equal(f(oracle.bf16_to_f64(finite)), finite)
    # midpoints of neighbouring positive values go to the even pattern, and
    # anything strictly between goes to the nearer one
    lo = np.arange(0x0001, 0x7F7F, 97, dtype=np.uint16)
    a = oracle.bf16_to_f64(lo)
    b = oracle.bf16_to_f64(lo + 1)
    mid = (a + b) / 2
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(f(mid), even)
    assert np.array_equal(f(a + (b - a) * 0.25), lo)
    assert np.array_equal(f(a + (b - a) * 0.75), (lo + 1).astype(np.uint16))
    assert np.array_equal(f(-mid), even | 0x8000)


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

def test_combine_sum_and_f32_order():
    parts = [synth.small_int(100 + r, (7, 9)) for r in range(5)]
    exact = np.sum(np.stack(parts).astype(np.int64), axis=0).astype(np.float64)
    assert np.array_equal(oracle.combine_sum(parts), exact)
    # ascending-rank binary32 order: (1e8 + 1) - 1e8 == 0 in binary32
    P = [np.array([1e8], np.float32), np.array([1.0], np.float32), np.array([-1e8], np.float32)]
    assert oracle.sum_f32_seq(P)[0] == np.float32(0.0)
    assert oracle.combine_sum(P)[0] == 1.0
    # against numpy binary32 additions done one rank at a time
    R = [synth.normal_f32(110 + r, (33, 17)) for r in range(8)]
    acc = R[0].copy()
    for r in R[1:]:
        acc = (acc + r).astype(np.float32)
    assert np.array_equal(oracle.sum_f32_seq(R), acc)


def test_combine_concat_layout():
    parts = [np.full((3, 2), r, dtype=np.float32) for r in range(4)]
    Y = oracle.combine_concat(parts)
    assert Y.shape == (3, 8)
    assert list(Y[1]) == [0, 0, 1, 1, 2, 2, 3, 3]


def test_slice_q4_commutes_with_dequant():
    # slicing codes and groups, then dequantising == dequantising, then slicing
    K, N = 256, 32
    codes = synth.q4_codes(121, (K, N))
    sc = synth.uniform_bf16(122, (K // 64, N), 0.005, 0.02)
    bi = synth.normal_bf16(123, (K // 64, N), 0.05)
    full = oracle.dequant_q4(codes, sc, bi)
    for strategy in (oracle.COLUMN, oracle.ROW, oracle.REPLICATED):
        p = oracle.plan_linear(K, N, 2, strategy, 64)
        for r in range(2):
            s = dict(zip(oracle.FIELDS, map(int, p[r])))
            got = oracle.dequant_q4(*oracle.slice_q4(codes, sc, bi, s))
            assert np.array_equal(got, oracle.slice_weight(full, s))


def test_collectives_results():
    """The three collectives' per-rank results against what fixes them: an
    all-reduce is a reduce-scatter followed by an all-gather (the pages'
    ring description), the reduce-scatter blocks tile the rows exactly
    once, the all-gather is the concat on every rank, and integer parts sum
    exactly."""
    rng = np.random.default_rng(91)
    for M, R in ((7, 4), (1, 4), (8, 8), (32, 2), (5, 3)):
        parts = [rng.integers(-3, 4, size=(M, 6)).astype(np.float64) for _ in range(R)]
        exact = np.sum(np.stack(parts), axis=0)
        rs = oracle.reduce_scatter(parts, R)
        # blocks are contiguous, disjoint, ordered and cover every row
        bounds = [oracle.rank_rows(M, R, r) for r in range(R)]
        assert bounds[0][0] == 0 and bounds[-1][1] == M
        assert all(bounds[r][1] == bounds[r + 1][0] for r in range(R - 1))
        assert all(0 <= hi - lo - M // R <= 1 for lo, hi in bounds)
        assert np.array_equal(np.concatenate(rs, axis=0), exact)
        # all-reduce == all-gather of the reduce-scatter blocks (as rows)
        ar = oracle.all_reduce(parts, R)
        gathered = np.concatenate(rs, axis=0)
        assert len(ar) == R and all(np.array_equal(a, gathered) for a in ar)
        ag = oracle.all_gather(parts, R)
        assert len(ag) == R and all(np.array_equal(a, np.hstack(parts)) for a in ag)
    # binary32 ordered sum flows through unchanged
    parts = [rng.standard_normal((6, 5)).astype(np.float32) for _ in range(3)]
    rs = oracle.reduce_scatter(parts, 3, sum_fn=oracle.sum_f32_seq)
    assert np.array_equal(np.concatenate(rs), oracle.sum_f32_seq(parts))


# --------------------------------------------------------------------------
# vocabulary-parallel embedding and LM head
# --------------------------------------------------------------------------

def test_plan_vocab_slices_and_rejections():
    # mlxcel "Vocab Parallel": every rank owns one contiguous slice of the
    # vocabulary; slices in rank order tile [0, vocab) without overlap
    for vocab, hidden, tp in itertools.product((8, 64, 1024, 152064), (64, 3584), (1, 2, 4, 8)):
        if vocab % tp:
            continue
        p = oracle.plan_vocab(vocab, hidden, tp)
        ends = 0
        for r in range(tp):
            e, h = oracle.spec(p, r, 0), oracle.spec(p, r, 1)
            assert (e["proj"], e["strategy"], e["combine"]) == (8, oracle.ROW, oracle.SUM)
            assert (h["proj"], h["strategy"], h["combine"]) == (9, oracle.COLUMN, oracle.CONCAT)
            assert (e["K"], e["N"], h["K"], h["N"]) == (vocab, hidden, hidden, vocab)
            assert e["k_off"] == ends and h["n_off"] == ends  # contiguous, rank order
            assert e["k_len"] == h["n_len"] == vocab // tp
            assert (e["n_off"], e["n_len"], h["k_off"], h["k_len"]) == (0, hidden, 0, hidden)
            ends += e["k_len"]
        assert ends == vocab
    for args, code in (((100, 64, 8), oracle.NOT_DIVISIBLE), ((96, 64, 3), oracle.TP_NOT_POW2),
                       ((96, 64, 0), oracle.INVALID), ((0, 64, 2), oracle.INVALID)):
        with pytest.raises(oracle.OracleError) as ei:
            oracle.plan_vocab(*args)
        assert ei.value.code == code, args
    with pytest.raises(oracle.OracleError) as ei:
        oracle.plan_vocab(96, 96, 2, group=64)
    assert ei.value.code == oracle.GROUP_ALIGN
    oracle.plan_vocab(96, 128, 2, group=64)


def test_embed_lookup_is_one_hot_product_and_partials_sum_to_rows():
    # a lookup is the one-hot row of the token times the table (numpy
    # matmul, exact for one-hot rows); the rank partials of a token are zero
    # except on its owner, so they add up to the full row
    rng = np.random.default_rng(11)
    vocab, hidden, tp = 64, 24, 4
    E = rng.standard_normal((vocab, hidden))
    tokens = np.array([0, 15, 16, 63, 31, 32, 5, 5, -1, 64, 200], dtype=np.int64)
    full = np.zeros((len(tokens), hidden))
    for m, t in enumerate(tokens):
        if 0 <= t < vocab:
            full[m] = E[t]
    p = oracle.plan_vocab(vocab, hidden, tp)
    total = np.zeros_like(full)
    for r in range(tp):
        s = oracle.spec(p, r, 0)
        part = oracle.embed_lookup(E, tokens, s)
        onehot = np.zeros((len(tokens), vocab))
        for m, t in enumerate(tokens):
            if s["k_off"] <= t < s["k_off"] + s["k_len"]:
                onehot[m, t] = 1.0
        assert np.array_equal(part, onehot @ E)
        owned = (tokens >= s["k_off"]) & (tokens < s["k_off"] + s["k_len"])
        assert not part[~owned].any()
        total += part
    assert np.array_equal(total, full)
    assert not total[-3:].any()  # ids outside the vocabulary belong to no rank
    # a column block of the table keeps only its columns
    s = dict(oracle.spec(p, 1, 0), n_off=8, n_len=10)
    assert np.array_equal(oracle.embed_lookup(E, tokens, s)[2], E[16, 8:18])


def test_lm_head_shards_concat_to_full_logits():
    # column shards over the vocabulary: concat of the rank logits == X W
    rng = np.random.default_rng(12)
    vocab, hidden, tp = 96, 32, 4
    X = rng.integers(-3, 4, (5, hidden)).astype(np.float64)
    W = rng.integers(-3, 4, (hidden, vocab)).astype(np.float64)
    p = oracle.plan_vocab(vocab, hidden, tp)
    parts = [oracle.shard_forward(oracle.spec(p, r, 1), X, W) for r in range(tp)]
    assert np.array_equal(oracle.combine_concat(parts), X @ W)


# --------------------------------------------------------------------------
# mixture-of-experts plans
# --------------------------------------------------------------------------

def test_plan_experts_page_example():
    # mlxcel "MoE expert parallelization", Expert Parallel figure
    for tp, ne, rank, held in golden_rows("moe_examples.txt"):
        plan = oracle.plan_experts(int(ne), 64, 128, int(tp), 0)
        got = [e for e, r, _ in plan if r == int(rank)]
        assert got == [int(x) for x in held.split(",")]


def test_plan_experts_expert_parallel_properties():
    # expert i whole on rank i % tp, each expert exactly once, ranks past the
    # expert count empty; gate/up not joined, down summed over ranks
    for ne, tp in itertools.product((1, 3, 8, 64, 128), (1, 2, 4, 8)):
        plan = oracle.plan_experts(ne, 256, 384, tp, 0, group=64)
        assert sorted(e for e, _, _ in plan) == list(range(ne))
        ranks = [r for _, r, _ in plan]
        assert ranks == sorted(ranks)  # rank-major
        for e, r, sh in plan:
            assert r == e % tp
            for p, (K, N, cb) in (("gate", (256, 384, oracle.NONE)), ("up", (256, 384, oracle.NONE)),
                                  ("down", (384, 256, oracle.SUM))):
                s = sh[p]
                assert (s["strategy"], s["combine"], s["K"], s["N"], s["rank"]) == \
                    (oracle.EXPERT, cb, K, N, r)
                assert (s["k_off"], s["k_len"], s["n_off"], s["n_len"]) == (0, K, 0, N)
            assert (sh["gate"]["proj"], sh["up"]["proj"], sh["down"]["proj"]) == (4, 5, 6)


def test_plan_experts_within_expert_matches_dense_ffn():
    # within-expert: each expert split like the dense FFN of the standard
    # plan (gate/up column, down row over the same ffn block, summed)
    ne, hidden, ffn = 5, 256, 512
    for tp in (1, 2, 4, 8):
        plan = oracle.plan_experts(ne, hidden, ffn, tp, 1, group=64)
        assert len(plan) == tp * ne
        dense = oracle.plan(hidden, 8, 8, 64, ffn, tp, 64)
        for i, (e, r, sh) in enumerate(plan):
            assert (e, r) == (i % ne, i // ne)
            for p in ("gate", "up", "down"):
                assert sh[p] == oracle.spec(dense, r, p), (tp, e, p)


def test_plan_experts_rejections():
    cases = [((4, 64, 128, 2, 2), oracle.INVALID), ((0, 64, 128, 2, 0), oracle.INVALID),
             ((4, 64, 128, 3, 0), oracle.TP_NOT_POW2), ((4, 64, 100, 8, 1), oracle.NOT_DIVISIBLE),
             ((4, 64, 96, 2, 0, 64), oracle.GROUP_ALIGN), ((4, 64, 128, 4, 1, 64),
                                                           oracle.GROUP_ALIGN)]
    for args, code in cases:
        with pytest.raises(oracle.OracleError) as ei:
            oracle.plan_experts(*args)
        assert ei.value.code == code, args
    oracle.plan_experts(4, 64, 128, 4, 0, 64)  # whole experts: 128 is a multiple of 64


def test_moe_dispatch_worked_and_brute_force():
    # hand-worked: tokens pick (0, 2), (2, 1), (0, 0); the rank holds 2 and 0
    off, row_slot, slot_row = oracle.moe_dispatch([[0, 2], [2, 1], [0, 0]], [2, 0])
    assert off.tolist() == [0, 2, 5]
    assert row_slot.tolist() == [1, 2, 0, 4, 5]
    assert slot_row.tolist() == [2, 0, 1, -1, 3, 4]
    rng = np.random.default_rng(5)
    for T, k, E in ((1, 1, 1), (7, 2, 8), (40, 8, 16), (33, 3, 5)):
        topk = rng.integers(0, E, (T, k))
        held = [e for e in rng.permutation(E)[: max(1, E // 2)]]
        off, row_slot, slot_row = oracle.moe_dispatch(topk, held)
        flat = topk.ravel()
        assert off[0] == 0 and np.all(np.diff(off) >= 0)
        for i, e in enumerate(held):
            seg = row_slot[off[i]:off[i + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
            assert len(seg) == np.count_nonzero(flat == e)
        owned = np.isin(flat, held)
        assert np.array_equal(np.sort(row_slot), np.nonzero(owned)[0])
        assert np.all(slot_row[~owned] == -1)
        assert np.array_equal(row_slot[slot_row[owned]], np.nonzero(owned)[0])


def _moe_case(T=9, k=2, E=6, K=64, N=40, seed=21):
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    wts = rng.random((T, k))
    wts /= wts.sum(axis=1, keepdims=True)
    X = rng.standard_normal((T, K))
    W = [rng.standard_normal((K, N)) for _ in range(E)]
    return topk, wts, X, W


def test_moe_combine_and_slots_closed_forms():
    topk, wts, X, W = _moe_case()
    T, k = topk.shape
    xs = np.repeat(X[:, None, :], k, axis=1)
    ys = oracle.moe_linear_slots(xs, topk, lambda e: W[e], W[0].shape[1])
    # per token with numpy matmul: sum_j w_tj x_t W_{e_tj}
    want = np.stack([sum(wts[t, j] * (X[t] @ W[topk[t, j]]) for j in range(k))
                     for t in range(T)])
    assert np.allclose(oracle.moe_combine(ys, wts), want, rtol=1e-12, atol=1e-12)
    # one-hot weights pick one choice; equal slot values with unit weight
    # sums give that value back
    one = np.zeros_like(wts)
    one[:, 1] = 1.0
    assert np.array_equal(oracle.moe_combine(ys, one), ys[:, 1])
    same = np.repeat(ys[:, :1], k, axis=1)
    assert np.allclose(oracle.moe_combine(same, wts), ys[:, 0], rtol=1e-12, atol=1e-12)
    # an expert nobody holds contributes zero
    z = oracle.moe_linear_slots(xs, topk, lambda e: None, 40)
    assert z.shape == (T, k, 40) and not z.any()


@pytest.mark.parametrize("tp", [1, 2, 4])
def test_moe_sharded_outputs_sum_to_unsharded(tp):
    # expert parallel: each slot is computed on exactly one rank, so the
    # rank outputs add up to the unsharded MoE; within-expert: the row
    # shards of down add up, the column shards of gate concatenate
    topk, wts, X, W = _moe_case(E=8)
    T, k = topk.shape
    K, N = W[0].shape
    xs = np.repeat(X[:, None, :], k, axis=1)
    full = oracle.moe_combine(oracle.moe_linear_slots(xs, topk, lambda e: W[e], N), wts)
    ep = oracle.plan_experts(8, N, K, tp, 0)  # down: W[K = ffn][N = hidden]
    total = np.zeros_like(full)
    for r in range(tp):
        held = {e for e, rr, _ in ep if rr == r}
        ys = oracle.moe_linear_slots(xs, topk, lambda e: W[e] if e in held else None, N)
        total += oracle.moe_combine(ys, wts, np.isin(topk, list(held)))
    assert np.allclose(total, full, rtol=1e-12, atol=1e-12)
    wep = oracle.plan_experts(8, N, K, tp, 1)
    total = np.zeros_like(full)
    for r in range(tp):
        sh = next(s for e, rr, s in wep if rr == r)["down"]
        xr = xs[:, :, sh["k_off"]:sh["k_off"] + sh["k_len"]]
        ys = oracle.moe_linear_slots(xr, topk, lambda e: oracle.slice_weight(W[e], sh), N)
        total += oracle.moe_combine(ys, wts)
    assert np.allclose(total, full, rtol=1e-12, atol=1e-12)
    # gate W[hidden = N][ffn = K] of expert e: the transpose of its down
    xg = np.repeat(X[:, None, :N], k, axis=1)  # token inputs of width hidden
    Wg = [w.T for w in W]
    gates = []
    for r in range(tp):
        sh = next(s for e, rr, s in wep if rr == r)["gate"]
        gates.append(oracle.moe_linear_slots(xg, topk, lambda e: oracle.slice_weight(Wg[e], sh),
                                             sh["n_len"]))
    fullg = oracle.moe_linear_slots(xg, topk, lambda e: Wg[e], K)
    assert np.array_equal(np.concatenate(gates, axis=2), fullg)
