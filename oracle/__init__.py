"""CPU oracle for one rank's share of tensor-parallel linear layers.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
imports, links or runs it, and it imports nothing from the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, double precision, naive
loops); this module marshals numpy arrays to it and does the slicing with
plain numpy indexing.  Pages cited (by title and section):

* mlxcel manual, "Tensor parallelism" (텐서 병렬화) -- sections "Column
  Parallel", "Row Parallel", "Replicated", "Architecture-aware shard plan",
  "GQA-aware attention sharding", "Configuration".
* wiki entry "Tensor parallel processing" (텐서 병렬 처리) -- "Details" §1
  (column: Y = [X W_1, ..., X W_n]; row: Y = sum_i X_i W_i) and "Examples"
  §1 (the column-parallel simulation: concat of the shard outputs).

Every function here has a pin in ``tests/test_oracle.py`` against something
other than itself (closed forms, invariants, library routines, the pages'
worked shapes and examples).
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# plan record layout (one int64 per field)
FIELDS = ("proj", "rank", "strategy", "combine", "K", "N", "k_off", "k_len",
          "n_off", "n_len", "head_off", "head_cnt")
PROJS = ("q", "k", "v", "o", "gate", "up", "down")
COLUMN, ROW, REPLICATED, EXPERT = 0, 1, 2, 3
NONE, CONCAT, SUM = 0, 1, 2

# error classes of oracle_plan
OK, INVALID, NOT_DIVISIBLE, TP_NOT_POW2, GROUP_ALIGN = 0, -1, -2, -3, -4


class OracleError(ValueError):
    def __init__(self, code):
        super().__init__("oracle_plan rejected the dimensions (class %d)" % code)
        self.code = code


def lib():
    """Load liboracle.so, compiling it with gcc first if it is missing."""
    global _LIB
    if _LIB is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(path)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.oracle_plan.argtypes = [i32] * 7 + [vp, i64]
        L.oracle_plan.restype = ctypes.c_int
        L.oracle_plan_linear.argtypes = [i64, i64, i32, i32, i32, vp, i64]
        L.oracle_plan_linear.restype = ctypes.c_int
        L.oracle_plan_vocab.argtypes = [i64, i64, i32, i32, vp, i64]
        L.oracle_plan_vocab.restype = ctypes.c_int
        L.oracle_plan_experts.argtypes = [i32, i64, i64, i32, i32, i32, vp, i64]
        L.oracle_plan_experts.restype = i64
        L.oracle_bf16_to_f64.argtypes = [vp, vp, i64]
        L.oracle_f64_to_bf16_rne.argtypes = [vp, vp, i64]
        L.oracle_dequant_q4.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.oracle_gemm.argtypes = [vp, vp, vp, i64, i64, i64]
        L.oracle_gemm_at.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp]
        L.oracle_sum.argtypes = [vp, i64, i64, vp]
        L.oracle_sum_f32_seq.argtypes = [vp, i64, i64, vp]
        for f in ("oracle_bf16_to_f64", "oracle_f64_to_bf16_rne", "oracle_dequant_q4",
                  "oracle_gemm", "oracle_gemm_at", "oracle_sum", "oracle_sum_f32_seq"):
            getattr(L, f).restype = None
        _LIB = L
    return _LIB


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def plan(hidden, n_q_heads, n_kv_heads, head_dim, ffn, tp, group=0):
    """The GQA-aware shard plan: int64 array [tp][7][12] (fields FIELDS).

    Raises OracleError(code) when the dimensions are rejected.
    """
    out = np.zeros((max(tp, 1), len(PROJS), len(FIELDS)), dtype=np.int64)
    rc = lib().oracle_plan(hidden, n_q_heads, n_kv_heads, head_dim, ffn, tp, group,
                           out.ctypes.data_as(ctypes.c_void_p), out.size)
    if rc != OK:
        raise OracleError(rc)
    return out


def plan_linear(K, N, tp, strategy, group=0):
    """Shards of one lone linear W[K][N]: int64 array [tp][12]."""
    out = np.zeros((max(tp, 1), len(FIELDS)), dtype=np.int64)
    rc = lib().oracle_plan_linear(K, N, tp, strategy, group,
                                  out.ctypes.data_as(ctypes.c_void_p), out.size)
    if rc != OK:
        raise OracleError(rc)
    return out


def plan_vocab(vocab, hidden, tp, group=0):
    """Vocabulary-parallel shards: int64 array [tp][2][12], entry [r][0] the
    embedding's row block, [r][1] the LM head's column block."""
    out = np.zeros((max(tp, 1), 2, len(FIELDS)), dtype=np.int64)
    rc = lib().oracle_plan_vocab(vocab, hidden, tp, group,
                                 out.ctypes.data_as(ctypes.c_void_p), out.size)
    if rc != OK:
        raise OracleError(rc)
    return out


def plan_experts(n_experts, hidden, ffn, tp, mode, group=0):
    """MoE FFN shards: a list of (expert, rank, {"gate": spec, "up": spec,
    "down": spec}) in rank-major, expert-ascending order."""
    rec_len = 2 + 3 * len(FIELDS)
    count = n_experts * (tp if mode == 1 else 1)
    out = np.zeros((max(count, 1), rec_len), dtype=np.int64)
    rc = lib().oracle_plan_experts(n_experts, hidden, ffn, tp, mode, group,
                                   out.ctypes.data_as(ctypes.c_void_p), out.size)
    if rc < 0:
        raise OracleError(int(rc))
    res = []
    for row in out[:rc]:
        sh = {p: dict(zip(FIELDS, (int(v) for v in row[2 + i * len(FIELDS):
                                                          2 + (i + 1) * len(FIELDS)])))
              for i, p in enumerate(("gate", "up", "down"))}
        res.append((int(row[0]), int(row[1]), sh))
    return res


def spec(plan_array, rank, proj):
    """One plan record as a dict."""
    p = PROJS.index(proj) if isinstance(proj, str) else proj
    return dict(zip(FIELDS, (int(v) for v in plan_array[rank, p])))


def bf16_to_f64(bits):
    bits, pb = _c(bits, np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().oracle_bf16_to_f64(pb, out.ctypes.data_as(ctypes.c_void_p), bits.size)
    return out


def f64_to_bf16(x):
    """Round doubles to bf16 (nearest, ties to even); returns uint16 bits."""
    x, px = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f64_to_bf16_rne(px, out.ctypes.data_as(ctypes.c_void_p), x.size)
    return out


def dequant_q4(codes, scales, biases, group=64):
    """W[k][n] = scale[k//group][n] * q[k][n] + bias[k//group][n], in double.

    codes: uint8 [K][N] in 0..15; scales, biases: bf16 bits [K/group][N].
    """
    codes, pc = _c(codes, np.uint8)
    K, N = codes.shape
    scales, ps = _c(scales, np.uint16)
    biases, pb = _c(biases, np.uint16)
    assert scales.shape == (K // group, N) and biases.shape == scales.shape
    W = np.empty((K, N), dtype=np.float64)
    lib().oracle_dequant_q4(pc, ps, pb, K, N, group, W.ctypes.data_as(ctypes.c_void_p))
    return W


def gemm(X, W):
    """Y = X W in double, naive loop with k ascending."""
    X, px = _c(X, np.float64)
    W, pw = _c(W, np.float64)
    M, K = X.shape
    K2, N = W.shape
    assert K == K2
    Y = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm(px, pw, Y.ctypes.data_as(ctypes.c_void_p), M, K, N)
    return Y


def gemm_at(X, W, rows, cols):
    """(X W)[rows[i], cols[i]] for each i, in double."""
    X, px = _c(X, np.float64)
    W, pw = _c(W, np.float64)
    rows, pr = _c(rows, np.int64)
    cols, pcol = _c(cols, np.int64)
    K, N = W.shape
    assert X.shape[1] == K and rows.shape == cols.shape
    out = np.empty(rows.shape, dtype=np.float64)
    lib().oracle_gemm_at(px, pw, K, N, pr, pcol, rows.size, out.ctypes.data_as(ctypes.c_void_p))
    return out


def slice_weight(W, s):
    """The rank's shard of the full logical W[K][N].

    Column shard: W[:, n_off:n_off+n_len]; row shard: W[k_off:k_off+k_len, :];
    replicated: the whole W (mlxcel manual "Column Parallel", "Row Parallel",
    "Replicated").
    """
    if s["strategy"] == COLUMN:
        return W[:, s["n_off"]:s["n_off"] + s["n_len"]]
    if s["strategy"] == ROW:
        return W[s["k_off"]:s["k_off"] + s["k_len"], :]
    return W


def slice_q4(codes, scales, biases, s, group=64):
    """The shard of a 4-bit weight before dequantisation: the code block as in
    slice_weight, and the (scale, bias) groups that cover it -- groups run
    along K, so a row block [k_off, k_off + k_len) owns groups
    [k_off / group, (k_off + k_len) / group) and a column block keeps every
    group of its columns."""
    c = slice_weight(codes, s)
    if s["strategy"] == ROW:
        g0, g1 = s["k_off"] // group, (s["k_off"] + s["k_len"]) // group
        return c, scales[g0:g1], biases[g0:g1]
    if s["strategy"] == COLUMN:
        sl = slice(s["n_off"], s["n_off"] + s["n_len"])
        return c, scales[:, sl], biases[:, sl]
    return c, scales, biases


def slice_input(X, s):
    """The rank's input: the full X for column/replicated shards, the matching
    column block X_i = X[:, k_off:k_off+k_len] for row shards (wiki "Details"
    §1, row-parallel: each rank multiplies its split X_i by its W_i)."""
    if s["strategy"] == ROW:
        return X[:, s["k_off"]:s["k_off"] + s["k_len"]]
    return X


def shard_forward(s, X, W):
    """One rank's output: slice_input(X) @ slice_weight(W), in double."""
    return gemm(slice_input(X, s), slice_weight(W, s))


def embed_lookup(E, tokens, s):
    """One rank's partial of a vocabulary-parallel lookup (mlxcel manual
    "Vocab Parallel": a rank looks up only the tokens of its own vocabulary
    slice).  E is the full table [vocab][hidden]; s the rank's block
    [k_off, k_off + k_len) x [n_off, n_off + n_len).  Row m is E[t][n-block]
    for an owned token t = tokens[m], else zero; in double."""
    E = np.asarray(E, dtype=np.float64)
    out = np.zeros((len(tokens), s["n_len"]), dtype=np.float64)
    for m, t in enumerate(tokens):
        t = int(t)
        if s["k_off"] <= t < s["k_off"] + s["k_len"]:
            out[m] = E[t, s["n_off"]:s["n_off"] + s["n_len"]]
    return out


def combine_concat(parts):
    """Y = [Y_0, ..., Y_{n-1}] along the feature (last) dimension (wiki
    "Details" §1, column-parallel; "Examples" §1 concatenates on the last
    dimension)."""
    return np.concatenate([np.asarray(p) for p in parts], axis=-1)


def combine_sum(parts):
    """Y = sum_i Y_i over ranks, ascending rank order, in double."""
    P, pp = _c(np.stack([np.asarray(p, dtype=np.float64) for p in parts]), np.float64)
    R = P.shape[0]
    Y = np.empty(P.shape[1:], dtype=np.float64)
    lib().oracle_sum(pp, R, Y.size, Y.ctypes.data_as(ctypes.c_void_p))
    return Y


def sum_f32_seq(parts):
    """((P0 + P1) + P2) + ... in binary32, ascending rank order."""
    P, pp = _c(np.stack([np.asarray(p, dtype=np.float32) for p in parts]), np.float32)
    R = P.shape[0]
    Y = np.empty(P.shape[1:], dtype=np.float32)
    lib().oracle_sum_f32_seq(pp, R, Y.size, Y.ctypes.data_as(ctypes.c_void_p))
    return Y


# ---- the collectives' results, every rank's buffer (mlxcel manual, "Tensor
# parallelism", "Communication patterns": all-reduce = reduce-scatter then
# all-gather; all-gather: every rank ends with the full tensor; reduce-
# scatter: every rank ends with 1/N of the reduced tensor) ----

def rank_rows(M, n_ranks, r):
    """Rows [lo, hi) of an [M][n] tensor held by rank r after a
    reduce-scatter: the ring splits the tensor into n_ranks chunks in memory
    order, read here as balanced blocks of whole rows."""
    return (r * M) // n_ranks, ((r + 1) * M) // n_ranks


def all_reduce(parts, n_ranks, sum_fn=None):
    """Every rank's buffer after an all-reduce: the full sum."""
    total = (sum_fn or combine_sum)(parts)
    return [total.copy() for _ in range(n_ranks)]


def reduce_scatter(parts, n_ranks, sum_fn=None):
    """Every rank's buffer after a reduce-scatter: its row block of the sum."""
    total = (sum_fn or combine_sum)(parts)
    M = total.shape[0]
    out = []
    for r in range(n_ranks):
        lo, hi = rank_rows(M, n_ranks, r)
        out.append(total[lo:hi].copy())
    return out


def all_gather(parts, n_ranks):
    """Every rank's buffer after an all-gather: the concatenated tensor."""
    full = combine_concat(parts)
    return [full.copy() for _ in range(n_ranks)]


def moe_dispatch(topk, experts):
    """Rows of a rank's expert products (mlxcel manual "MoE expert
    parallelization": the router runs everywhere, each rank runs only the
    experts it holds).  topk is [T][k] expert ids; experts lists the rank's
    experts in the order their products are laid out.  A row is one
    (token, choice) slot s = t*k + j whose expert the rank holds; the rows
    of expert experts[i] are its slots in ascending order and come after
    those of experts[:i].  Returns (offsets [n+1], row_slot [rows],
    slot_row [T*k], -1 for slots of other ranks' experts)."""
    topk = np.asarray(topk)
    T, k = topk.shape
    offsets, row_slot = [0], []
    slot_row = np.full(T * k, -1, dtype=np.int64)
    for e in experts:
        for t in range(T):
            for j in range(k):
                if topk[t, j] == e:
                    slot_row[t * k + j] = len(row_slot)
                    row_slot.append(t * k + j)
        offsets.append(len(row_slot))
    return np.array(offsets, dtype=np.int64), np.array(row_slot, dtype=np.int64), slot_row


def moe_combine(y_slots, weights, slot_mask=None):
    """A token's MoE output: sum_j weights[t][j] * y_slots[t][j] over its k
    choices (those in slot_mask when given), j ascending, in double."""
    y_slots = np.asarray(y_slots, dtype=np.float64)
    T, k = weights.shape
    out = np.zeros((T, y_slots.shape[-1]))
    for t in range(T):
        for j in range(k):
            if slot_mask is None or slot_mask[t, j]:
                out[t] += float(weights[t, j]) * y_slots[t, j]
    return out


def moe_linear_slots(x_slots, topk, shard_weight, n):
    """y[t][j] = x_slots[t][j] . W_e for e = topk[t][j], where
    shard_weight(e) is the rank's block (n output columns) of expert e's
    weight, or None when the rank does not hold e (y = 0), and x_slots[t][j]
    the matching input block; in double."""
    topk = np.asarray(topk)
    T, k = topk.shape
    out = np.zeros((T, k, n))
    for e in sorted(set(int(v) for v in topk.ravel())):
        W = shard_weight(e)
        if W is None:
            continue
        sel = [(t, j) for t in range(T) for j in range(k) if topk[t, j] == e]
        ys = gemm(np.stack([x_slots[t][j] for t, j in sel]), W)
        for (t, j), y in zip(sel, ys):
            out[t, j] = y
    return out
