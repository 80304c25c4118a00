/*
 * CPU oracle for one rank's share of tensor-parallel linear layers.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, plain, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it;
 * the product path never does.  It shares no source, header, helper, table
 * or constant with the GPU library, and it includes nothing from it.
 *
 * Everything is computed in double precision (IEEE binary64) with a fixed,
 * ascending summation order and no fused multiply-add (built with
 * -ffp-contract=off, never with -ffast-math).
 *
 * The method is defined by three web pages; citations name the page and the
 * section on it:
 *   [mlxcel]  mlxcel manual, "Tensor parallelism" (텐서 병렬화):
 *             sections "Column Parallel", "Row Parallel", "Replicated",
 *             "Communication patterns", "Architecture-aware shard plan"
 *             (table "Standard transformer"), "GQA-aware attention
 *             sharding" (figure), "Configuration" (--tp-size row).
 *   [wiki]    wiki entry "Tensor parallel processing" (텐서 병렬 처리):
 *             "Details" §1 "Operating mechanism (Column & Row
 *             Parallelism)", "Examples" §1 (column-parallel simulation).
 *   [blog]    "How does tensor parallelism split local AI inference across
 *             multiple GPUs?": section "Column and row shards split the
 *             matrix multiplication".
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *   - the logical weight is W[K][N] = [D_in][D_out] ([mlxcel] Column/Row
 *     Parallel block diagrams draw W as [D_in x D_out]);
 *   - dimensions must divide exactly by tp (the pages write D_out/N);
 *   - contiguous blocks are assigned in rank order;
 *   - when num_kv_heads < tp the full K/V projection is replicated;
 *   - 4-bit weights: w = scale * q + bias, q in 0..15, one (scale, bias)
 *     pair per 64 consecutive input-dimension elements of one output column;
 *   - a row-parallel shard of 4-bit weights must start and end on a group
 *     boundary;
 *   - rank partials are summed in ascending rank order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Error classes returned by oracle_plan (negative). */
#define OR_OK 0
#define OR_INVALID (-1)       /* non-positive size, bad tp, output too short */
#define OR_NOT_DIVISIBLE (-2) /* a dimension does not split evenly */
#define OR_TP_NOT_POW2 (-3)   /* tp is not a power of two */
#define OR_GROUP_ALIGN (-4)   /* 4-bit group boundary violated */

/* Projection order, strategies and combine modes of the plan records. */
enum { P_Q = 0, P_K, P_V, P_O, P_GATE, P_UP, P_DOWN, P_COUNT };
enum { S_COLUMN = 0, S_ROW = 1, S_REPLICATED = 2 };
enum { C_NONE = 0, C_CONCAT = 1, C_SUM = 2 };

#define FIELDS 12 /* proj rank strategy combine K N k_off k_len n_off n_len head_off head_cnt */

static void put(int64_t *rec, int64_t proj, int64_t rank, int64_t strategy, int64_t combine,
                int64_t K, int64_t N, int64_t k_off, int64_t k_len, int64_t n_off, int64_t n_len,
                int64_t head_off, int64_t head_cnt)
{
    rec[0] = proj;
    rec[1] = rank;
    rec[2] = strategy;
    rec[3] = combine;
    rec[4] = K;
    rec[5] = N;
    rec[6] = k_off;
    rec[7] = k_len;
    rec[8] = n_off;
    rec[9] = n_len;
    rec[10] = head_off;
    rec[11] = head_cnt;
}

/*
 * The architecture-aware shard plan of a standard transformer layer
 * ([mlxcel] "Architecture-aware shard plan", table "Standard transformer"):
 *   q, k, v  -> column parallel (q gathers its outputs; k/v are GQA-aware)
 *   o        -> row parallel, partials all-reduced (summed)
 *   gate, up -> column parallel, no communication
 *   down     -> row parallel, partials all-reduced (summed)
 * with the GQA rule of [mlxcel] "GQA-aware attention sharding": K/V are
 * sharded by heads when num_kv_heads >= tp and replicated on every rank
 * when num_kv_heads < tp.  tp must be a power of two ([mlxcel]
 * "Configuration", --tp-size).  Column shard r holds W[:, r*N/tp ...] and
 * row shard r holds W[r*K/tp ..., :] ([mlxcel] "Column Parallel",
 * "Row Parallel").
 *
 * group > 0 declares 4-bit group-quantised weights with that group size.
 * Output: tp * 7 records of FIELDS int64, rank-major, projections in the
 * order q k v o gate up down.
 */
int oracle_plan(int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                int32_t ffn, int32_t tp, int32_t group, int64_t *out, int64_t out_len)
{
    if (hidden < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 || ffn < 1 || tp < 1 ||
        group < 0)
        return OR_INVALID;
    if (out == 0 || out_len < (int64_t)tp * P_COUNT * FIELDS)
        return OR_INVALID;
    if ((tp & (tp - 1)) != 0)
        return OR_TP_NOT_POW2;
    if (n_q_heads % n_kv_heads != 0)
        return OR_NOT_DIVISIBLE;
    if (n_q_heads % tp != 0)
        return OR_NOT_DIVISIBLE;
    if (ffn % tp != 0)
        return OR_NOT_DIVISIBLE;
    int kv_sharded = n_kv_heads >= tp;
    if (kv_sharded && n_kv_heads % tp != 0)
        return OR_NOT_DIVISIBLE;

    int64_t q_width = (int64_t)n_q_heads * head_dim;   /* q output / o input */
    int64_t kv_width = (int64_t)n_kv_heads * head_dim; /* k, v output */
    int64_t q_heads_per_rank = n_q_heads / tp;
    int64_t ffn_per_rank = ffn / tp;

    if (group > 0) {
        /* every projection's input dimension holds whole groups ... */
        if (hidden % group != 0 || q_width % group != 0 || ffn % group != 0)
            return OR_GROUP_ALIGN;
        /* ... and every row shard starts and ends on a group boundary */
        if ((q_heads_per_rank * head_dim) % group != 0 || ffn_per_rank % group != 0)
            return OR_GROUP_ALIGN;
    }

    for (int64_t r = 0; r < tp; ++r) {
        int64_t *rec = out + r * P_COUNT * FIELDS;
        int64_t q_h0 = r * q_heads_per_rank;

        /* q: column shard over the rank's query heads */
        put(rec + P_Q * FIELDS, P_Q, r, S_COLUMN, C_CONCAT, hidden, q_width, 0, hidden,
            q_h0 * head_dim, q_heads_per_rank * head_dim, q_h0, q_heads_per_rank);

        /* k, v: GQA-aware */
        for (int p = P_K; p <= P_V; ++p) {
            if (kv_sharded) {
                int64_t kh = n_kv_heads / tp;
                put(rec + p * FIELDS, p, r, S_COLUMN, C_CONCAT, hidden, kv_width, 0, hidden,
                    r * kh * head_dim, kh * head_dim, r * kh, kh);
            } else {
                put(rec + p * FIELDS, p, r, S_REPLICATED, C_NONE, hidden, kv_width, 0, hidden,
                    0, kv_width, 0, n_kv_heads);
            }
        }

        /* o: row shard over the same head range as q */
        put(rec + P_O * FIELDS, P_O, r, S_ROW, C_SUM, q_width, hidden,
            q_h0 * head_dim, q_heads_per_rank * head_dim, 0, hidden, q_h0, q_heads_per_rank);

        /* gate, up: column shards, no communication */
        put(rec + P_GATE * FIELDS, P_GATE, r, S_COLUMN, C_NONE, hidden, ffn, 0, hidden,
            r * ffn_per_rank, ffn_per_rank, -1, -1);
        put(rec + P_UP * FIELDS, P_UP, r, S_COLUMN, C_NONE, hidden, ffn, 0, hidden,
            r * ffn_per_rank, ffn_per_rank, -1, -1);

        /* down: row shard over the same ffn range as gate/up */
        put(rec + P_DOWN * FIELDS, P_DOWN, r, S_ROW, C_SUM, ffn, hidden,
            r * ffn_per_rank, ffn_per_rank, 0, hidden, -1, -1);
    }
    return OR_OK;
}

/*
 * Shards of one lone linear layer W[K][N] split tp ways with one strategy
 * ([mlxcel] "Column Parallel", "Row Parallel", "Replicated"; [wiki]
 * "Examples" §1 splits a 1024 -> 2048 layer into two column shards).
 * Column shard r: columns [r*N/tp, (r+1)*N/tp), outputs concatenated;
 * row shard r: rows [r*K/tp, (r+1)*K/tp), partials summed; replicated:
 * all of W, nothing to join.  proj is 7 and the head fields are -1.
 * Output: tp records of FIELDS int64.
 */
int oracle_plan_linear(int64_t K, int64_t N, int32_t tp, int32_t strategy, int32_t group,
                       int64_t *out, int64_t out_len)
{
    if (K < 1 || N < 1 || tp < 1 || group < 0 || strategy < S_COLUMN || strategy > S_REPLICATED)
        return OR_INVALID;
    if (out == 0 || out_len < (int64_t)tp * FIELDS)
        return OR_INVALID;
    if ((tp & (tp - 1)) != 0)
        return OR_TP_NOT_POW2;
    if (strategy == S_COLUMN && N % tp != 0)
        return OR_NOT_DIVISIBLE;
    if (strategy == S_ROW && K % tp != 0)
        return OR_NOT_DIVISIBLE;
    if (group > 0 && (K % group != 0 || (strategy == S_ROW && (K / tp) % group != 0)))
        return OR_GROUP_ALIGN;
    for (int64_t r = 0; r < tp; ++r) {
        int64_t *rec = out + r * FIELDS;
        if (strategy == S_COLUMN)
            put(rec, P_COUNT, r, S_COLUMN, C_CONCAT, K, N, 0, K, r * (N / tp), N / tp, -1, -1);
        else if (strategy == S_ROW)
            put(rec, P_COUNT, r, S_ROW, C_SUM, K, N, r * (K / tp), K / tp, 0, N, -1, -1);
        else
            put(rec, P_COUNT, r, S_REPLICATED, C_NONE, K, N, 0, K, 0, N, -1, -1);
    }
    return OR_OK;
}

/*
 * Vocabulary-parallel shards of the token embedding and the LM head
 * ([mlxcel] "Weight sharding strategy", "Vocab Parallel"; "Embedding and
 * LM head sharding", mode vocab_parallel): the vocabulary is cut into tp
 * contiguous slices in rank order.  The embedding table E[vocab][hidden] is
 * read as W[K = vocab][N = hidden], so its slice is a row block whose
 * partial lookups are summed; the LM head W[K = hidden][N = vocab] is
 * column-split and its logits concatenated.  tp a power of two, vocab % tp
 * == 0; group > 0 (a 4-bit LM head) needs hidden % group == 0.
 * Output: tp * 2 records (embedding, LM head) of FIELDS int64, rank-major;
 * proj 8 is the embedding, 9 the LM head, head fields -1.
 */
int oracle_plan_vocab(int64_t vocab, int64_t hidden, int32_t tp, int32_t group, int64_t *out,
                      int64_t out_len)
{
    if (vocab < 1 || hidden < 1 || tp < 1 || (group != 0 && group != 64))
        return OR_INVALID;
    if (out == 0 || out_len < (int64_t)tp * 2 * FIELDS)
        return OR_INVALID;
    if ((tp & (tp - 1)) != 0)
        return OR_TP_NOT_POW2;
    if (vocab % tp != 0)
        return OR_NOT_DIVISIBLE;
    if (group > 0 && hidden % group != 0)
        return OR_GROUP_ALIGN;
    int64_t slice = vocab / tp;
    for (int64_t r = 0; r < tp; ++r) {
        put(out + (2 * r) * FIELDS, 8, r, S_ROW, C_SUM, vocab, hidden, r * slice, slice, 0, hidden,
            -1, -1);
        put(out + (2 * r + 1) * FIELDS, 9, r, S_COLUMN, C_CONCAT, hidden, vocab, 0, hidden,
            r * slice, slice, -1, -1);
    }
    return OR_OK;
}

/*
 * Mixture-of-experts FFN shards ([mlxcel] "MoE expert parallelization").
 * mode 0, expert parallel: expert e is held whole by rank e % tp (strategy
 * 3, "expert"), gate/up not joined, down summed over ranks.  mode 1,
 * within-expert: every rank holds every expert split like the dense FFN
 * ([mlxcel] table "Standard transformer": gate/up column, down row, summed).
 * Records: rank-major, experts ascending; each record is the expert index,
 * the rank, then three FIELDS-long shard records (gate, up, down).
 * Returns the number of records, or a negative error class.
 */
int64_t oracle_plan_experts(int32_t n_experts, int64_t hidden, int64_t ffn, int32_t tp,
                            int32_t mode, int32_t group, int64_t *out, int64_t out_len)
{
    if (n_experts < 1 || hidden < 1 || ffn < 1 || tp < 1 || (mode != 0 && mode != 1) ||
        (group != 0 && group != 64))
        return OR_INVALID;
    int64_t count = mode == 0 ? n_experts : (int64_t)tp * n_experts;
    int64_t rec_len = 2 + 3 * FIELDS;
    if (out == 0 || out_len < count * rec_len)
        return OR_INVALID;
    if ((tp & (tp - 1)) != 0)
        return OR_TP_NOT_POW2;
    if (mode == 1 && ffn % tp != 0)
        return OR_NOT_DIVISIBLE;
    if (group > 0 && (hidden % group != 0 || ffn % group != 0 ||
                      (mode == 1 && (ffn / tp) % group != 0)))
        return OR_GROUP_ALIGN;
    int64_t k = 0;
    for (int64_t r = 0; r < tp; ++r) {
        for (int64_t e = 0; e < n_experts; ++e) {
            if (mode == 0 && e % tp != r)
                continue;
            int64_t *rec = out + k * rec_len;
            rec[0] = e;
            rec[1] = r;
            if (mode == 0) {
                put(rec + 2, P_GATE, r, 3, C_NONE, hidden, ffn, 0, hidden, 0, ffn, -1, -1);
                put(rec + 2 + FIELDS, P_UP, r, 3, C_NONE, hidden, ffn, 0, hidden, 0, ffn, -1, -1);
                put(rec + 2 + 2 * FIELDS, P_DOWN, r, 3, C_SUM, ffn, hidden, 0, ffn, 0, hidden, -1,
                    -1);
            } else {
                int64_t w = ffn / tp;
                put(rec + 2, P_GATE, r, S_COLUMN, C_NONE, hidden, ffn, 0, hidden, r * w, w, -1, -1);
                put(rec + 2 + FIELDS, P_UP, r, S_COLUMN, C_NONE, hidden, ffn, 0, hidden, r * w, w,
                    -1, -1);
                put(rec + 2 + 2 * FIELDS, P_DOWN, r, S_ROW, C_SUM, ffn, hidden, r * w, w, 0, hidden,
                    -1, -1);
            }
            ++k;
        }
    }
    return k;
}

/* bf16 -> double: a bf16 value is the upper half of an IEEE binary32. */
void oracle_bf16_to_f64(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t bits = (uint32_t)in[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        out[i] = (double)f;
    }
}

/*
 * double -> bf16, round to nearest, ties to even, straight from the double
 * (no intermediate rounding to binary32).  bf16 has 8 significant bits and
 * the exponent range of binary32.
 */
static uint16_t to_bf16(double d)
{
    if (isnan(d))
        return 0x7FC0;
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    double a = fabs(d);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    int shift = 8 - e;
    if (e < -125) /* below the normal range: fixed spacing 2^-133 */
        shift = 133;
    double scaled = ldexp(a, shift); /* exact: power-of-two scaling */
    double r = nearbyint(scaled);    /* default mode: nearest, ties to even */
    double v = ldexp(r, -shift);
    if (v >= 0x1p128) /* beyond the largest finite bf16 after rounding */
        return sign | 0x7F80;
    float f = (float)v; /* exact: v has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

void oracle_f64_to_bf16_rne(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = to_bf16(in[i]);
}

/*
 * 4-bit affine group dequantisation (reading of the "-4bit" models listed
 * under [mlxcel] "Current runtime support"): for logical W[K][N],
 *   W[k][n] = scale[k / group][n] * q[k][n] + bias[k / group][n]
 * with q in 0..15 and bf16 scale and bias.  codes is one byte per weight,
 * logical [K][N]; scales and biases are bf16 bits, logical [K/group][N].
 */
void oracle_dequant_q4(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                       int64_t K, int64_t N, int64_t group, double *W)
{
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = k / group;
        for (int64_t n = 0; n < N; ++n) {
            double s, b;
            oracle_bf16_to_f64(&scales[g * N + n], &s, 1);
            oracle_bf16_to_f64(&biases[g * N + n], &b, 1);
            W[k * N + n] = s * (double)codes[k * N + n] + b;
        }
    }
}

/*
 * Y[m][n] = sum_{k=0}^{K-1} X[m][k] * W[k][n], accumulated in double with k
 * ascending for every (m, n).  This is the plain product that both
 * column shards (Y_i = X W_i) and row shards (Y_i = X_i W_i) evaluate
 * ([wiki] "Details" §1).  Rows are split across OpenMP threads; the
 * per-element order is the same whatever the thread count.
 */
void oracle_gemm(const double *X, const double *W, double *Y, int64_t M, int64_t K, int64_t N)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *y = Y + m * N;
        for (int64_t n = 0; n < N; ++n)
            y[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double x = X[m * K + k];
            const double *w = W + k * N;
            for (int64_t n = 0; n < N; ++n)
                y[n] += x * w[n];
        }
    }
}

/* The same sum, for selected output elements (rows[i], cols[i]) only. */
void oracle_gemm_at(const double *X, const double *W, int64_t K, int64_t N, const int64_t *rows,
                    const int64_t *cols, int64_t count, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += X[rows[i] * K + k] * W[k * N + cols[i]];
        out[i] = acc;
    }
}

/*
 * Sum of R rank partials, in ascending rank order, in double: the result
 * that the all-reduce after a row-parallel layer produces
 * ([mlxcel] "Row Parallel"; [wiki] "Details" §1: Y = sum_i Y_i).
 * P is [R][count].
 */
void oracle_sum(const double *P, int64_t R, int64_t count, double *Y)
{
    for (int64_t i = 0; i < count; ++i) {
        double acc = 0.0;
        for (int64_t r = 0; r < R; ++r)
            acc += P[r * count + i];
        Y[i] = acc;
    }
}

/*
 * The same sum evaluated in binary32 in ascending rank order,
 * ((P0 + P1) + P2) + ..., each addition rounded to nearest even: the
 * fixed-order reading of the all-reduce for partials that already are
 * binary32 values.
 */
void oracle_sum_f32_seq(const float *P, int64_t R, int64_t count, float *Y)
{
    for (int64_t i = 0; i < count; ++i) {
        float acc = P[i];
        for (int64_t r = 1; r < R; ++r)
            acc = acc + P[r * count + i];
        Y[i] = acc;
    }
}
