/*
 * tsl.h -- one rank's share of tensor-parallel linear layers on one AMD
 * Instinct MI355X (gfx950).  C ABI; every function returns a tsl_status and
 * nothing throws across it.
 *
 * The method is defined by three web pages, cited by title and section:
 *   [mlxcel] mlxcel manual, "Tensor parallelism" (텐서 병렬화)
 *   [wiki]   wiki entry "Tensor parallel processing" (텐서 병렬 처리)
 *   [blog]   "How does tensor parallelism split local AI inference across
 *            multiple GPUs?" (텐서 병렬 처리는 여러 GPU에서 로컬 AI 추론을
 *            어떻게 분할하나요?)
 *
 * Notation.  A linear layer computes Y[M][N] = X[M][K] * W[K][N]; K is the
 * input dimension (D_in), N the output dimension (D_out), M the number of
 * token rows (batch x sequence).  [mlxcel] "Column Parallel" and "Row
 * Parallel" draw W as [D_in x D_out]; that logical W[K][N] is the one used
 * throughout, whatever order its bytes are stored in.
 *
 * Conventions shared by every entry point:
 *   - Memory.  Every device buffer is allocated and owned by the caller
 *     (packed weights, activations, outputs, partials, workspace).  The
 *     library allocates nothing and frees nothing.
 *   - Streams.  `stream` is a hipStream_t passed as void*; NULL is the null
 *     stream.  Device work is enqueued on it asynchronously; no entry point
 *     synchronises the device.
 *   - Validation.  Shapes, strides, dtypes, buffer sizes and alignments are
 *     checked on the host before anything is enqueued; a failed check
 *     returns a negative status and has no side effects.  A HIP error from
 *     a launch is returned as TSL_ERR_HIP.
 *   - Alignment.  Device pointers must be 16-byte aligned; the packed-weight
 *     and workspace buffers 256-byte aligned.
 *   - Leading dimensions (ldx, ldy, ld_part) are in elements, not bytes.
 */
#ifndef TSL_H
#define TSL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; the declarations of
 * this header are its only exported names. */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

typedef enum tsl_status {
    TSL_OK = 0,
    TSL_ERR_INVALID_ARG = -1,      /* null pointer, non-positive size, bad enum */
    TSL_ERR_NOT_DIVISIBLE = -2,    /* a dimension does not split evenly across ranks */
    TSL_ERR_TP_NOT_POW2 = -3,      /* tp_size is not a power of two */
    TSL_ERR_GROUP_ALIGN = -4,      /* a 4-bit group would straddle a shard edge */
    TSL_ERR_BUFFER_TOO_SMALL = -5, /* an output, packed or workspace buffer is short */
    TSL_ERR_UNSUPPORTED = -6,      /* dtype combination or size the kernels do not take */
    TSL_ERR_MISALIGNED = -7,       /* pointer or leading dimension breaks alignment */
    TSL_ERR_HIP = -8               /* the HIP runtime reported an error */
} tsl_status;

/* How a weight is split across ranks ([mlxcel] "Weight sharding strategy"). */
typedef enum tsl_strategy {
    TSL_COLUMN = 0,    /* rank r holds W[:, n_off : n_off + n_len] ("Column Parallel") */
    TSL_ROW = 1,       /* rank r holds W[k_off : k_off + k_len, :] ("Row Parallel")    */
    TSL_REPLICATED = 2, /* every rank holds the whole W ("Replicated")                 */
    TSL_EXPERT = 3      /* the whole W of one MoE expert, on its owner rank only       */
} tsl_strategy;

/* How rank outputs are joined ([mlxcel] "Communication patterns"): the
 * concat is what an all-gather of column shards yields, the sum what an
 * all-reduce of row partials yields ([wiki] "Details" §1). */
typedef enum tsl_combine {
    TSL_COMBINE_NONE = 0,   /* the output stays sharded (no communication) */
    TSL_COMBINE_CONCAT = 1, /* Y = [Y_0, ..., Y_{tp-1}] along N            */
    TSL_COMBINE_SUM = 2     /* Y = Y_0 + ... + Y_{tp-1}, ascending rank    */
} tsl_combine;

/* Projections of a standard transformer layer, in plan order; TSL_LINEAR
 * tags a lone linear layer planned with plan_linear(), TSL_EMBED and
 * TSL_LM_HEAD the vocabulary-indexed weights planned with plan_vocab(). */
typedef enum tsl_proj {
    TSL_Q = 0, TSL_K = 1, TSL_V = 2, TSL_O = 3,
    TSL_GATE = 4, TSL_UP = 5, TSL_DOWN = 6,
    TSL_NPROJ = 7,
    TSL_LINEAR = 7,
    TSL_EMBED = 8,
    TSL_LM_HEAD = 9
} tsl_proj;

typedef enum tsl_dtype {
    TSL_F32 = 0,   /* IEEE binary32                                         */
    TSL_BF16 = 1,  /* bfloat16 (upper half of a binary32)                   */
    TSL_Q4G64 = 2  /* weights only: 4-bit codes q in 0..15, affine groups of
                      64 input elements with a bf16 scale s and bias b:
                      w = s * q + b                                         */
} tsl_dtype;

/* Dimensions of one transformer layer and the TP degree. */
typedef struct tsl_dims {
    int32_t hidden;     /* model width: q/k/v/gate/up input, o/down output */
    int32_t n_q_heads;
    int32_t n_kv_heads; /* grouped-query attention: n_q_heads % n_kv_heads == 0 */
    int32_t head_dim;
    int32_t ffn;        /* FFN width: gate/up output, down input */
    int32_t tp_size;    /* number of ranks; a power of two */
    int32_t group_size; /* 0 for dense weights, 64 for TSL_Q4G64 weights */
} tsl_dims;

/* One rank's share of one weight.  K, N describe the full logical W[K][N];
 * the shard is W[k_off : k_off + k_len, n_off : n_off + n_len].  For a
 * column shard k_len == K; for a row shard n_len == N; a replicated shard
 * covers all of W.  head_off/head_cnt give the attention heads a q/k/v/o
 * shard covers (-1 for FFN weights and lone linears). */
typedef struct tsl_shard {
    int32_t proj;     /* tsl_proj */
    int32_t rank;
    int32_t strategy; /* tsl_strategy */
    int32_t combine;  /* tsl_combine */
    int64_t K, N;
    int64_t k_off, k_len;
    int64_t n_off, n_len;
    int32_t head_off, head_cnt;
} tsl_shard;

/*
 * plan_shards -- the architecture-aware, GQA-aware shard plan of one
 * standard transformer layer ([mlxcel] "Architecture-aware shard plan",
 * table "Standard transformer"; "GQA-aware attention sharding").
 *
 *   q           column shard over query heads [r*hq/tp, (r+1)*hq/tp),
 *               combine CONCAT (the table's all-gather)
 *   k, v        n_kv_heads >= tp: column shard over KV heads, combine CONCAT;
 *               n_kv_heads <  tp: TSL_REPLICATED (the full K/V projection on
 *               every rank), combine NONE
 *   o           row shard over the same head range as q, combine SUM
 *   gate, up    column shard over [r*ffn/tp, (r+1)*ffn/tp), combine NONE
 *   down        row shard over the same ffn range, combine SUM
 *
 * Output: out[r * TSL_NPROJ + p] for rank r and projection p; out_len is
 * the number of records `out` can hold and must be >= tp_size * TSL_NPROJ.
 * Errors, checked in this order: TSL_ERR_INVALID_ARG (null, a size < 1,
 * group_size not 0 or 64, out_len short), TSL_ERR_TP_NOT_POW2 ([mlxcel]
 * "Configuration": --tp-size must be a power of two), TSL_ERR_NOT_DIVISIBLE
 * (n_q_heads % n_kv_heads, n_q_heads % tp, ffn % tp, or n_kv_heads >= tp
 * with n_kv_heads % tp), TSL_ERR_GROUP_ALIGN (a 4-bit projection input or
 * row-shard edge not on a multiple of group_size).  Host only.
 */
tsl_status plan_shards(const tsl_dims *dims, tsl_shard *out, int64_t out_len);

/*
 * plan_linear -- the shards of one lone linear layer W[K][N] split `tp`
 * ways with `strategy` ([mlxcel] "Column Parallel", "Row Parallel",
 * "Replicated"; [wiki] "Examples" §1 splits one 1024 -> 2048 layer into two
 * column shards).  Combine is CONCAT for column, SUM for row, NONE for
 * replicated; proj is TSL_LINEAR; heads are -1.  group_size 64 requires
 * every row-shard edge on a group boundary.  out_len >= tp.  Host only.
 */
tsl_status plan_linear(int64_t K, int64_t N, int32_t tp_size, int32_t strategy,
                       int32_t group_size, tsl_shard *out, int64_t out_len);

/*
 * plan_vocab -- the vocabulary-parallel shards of the token embedding and
 * the LM head ([mlxcel] "Weight sharding strategy", "Vocab Parallel": the
 * vocabulary dimension of both is split across ranks, each rank owning one
 * contiguous slice; "Embedding and LM head sharding", mode vocab_parallel).
 * Rank r owns tokens [r*vocab/tp, (r+1)*vocab/tp).
 *   out[2r]     TSL_EMBED: the table E[vocab][hidden] read as a linear
 *               layer W[K = vocab][N = hidden] (a lookup is a one-hot row
 *               times W), row shard over rank r's tokens, combine SUM: the
 *               rank partials of a lookup add up to the full row
 *               (embed_lookup).
 *   out[2r + 1] TSL_LM_HEAD: W[K = hidden][N = vocab], column shard over
 *               rank r's tokens, combine CONCAT (the logits' all-gather);
 *               a shard_linear weight like any other column shard.
 * head_off/head_cnt are -1.  group_size 64 (4-bit LM head) requires
 * hidden % 64 == 0; the embedding table itself is dense (embed_lookup).
 * Errors, in this order: TSL_ERR_INVALID_ARG (null, vocab/hidden/tp < 1,
 * group_size not 0 or 64, out_len < 2*tp), TSL_ERR_TP_NOT_POW2,
 * TSL_ERR_NOT_DIVISIBLE (vocab % tp; pad the vocabulary to a multiple of
 * tp), TSL_ERR_GROUP_ALIGN.  Host only.
 */
tsl_status plan_vocab(int64_t vocab, int64_t hidden, int32_t tp_size, int32_t group_size,
                      tsl_shard *out, int64_t out_len);

/* MoE sharding modes ([mlxcel] "MoE expert parallelization"). */
typedef enum tsl_moe_mode {
    TSL_MOE_EXPERT_PARALLEL = 0, /* expert e lives whole on rank e % tp     */
    TSL_MOE_WITHIN_EXPERT = 1    /* every expert's FFN split like a dense one */
} tsl_moe_mode;

/* The three FFN weights of one expert as held by one rank. */
typedef struct tsl_expert_shard {
    int32_t expert; /* expert index e, 0 <= e < n_experts */
    int32_t rank;   /* rank holding these shards */
    tsl_shard gate, up, down;
} tsl_expert_shard;

/*
 * plan_experts -- the shard plan of a mixture-of-experts FFN with
 * n_experts experts of width expert_ffn ([mlxcel] "MoE expert
 * parallelization", modes "Expert Parallel" and "Within-Expert Parallel").
 *   TSL_MOE_EXPERT_PARALLEL: experts are dealt round-robin, expert e whole
 *     on rank e % tp; its gate/up (W[hidden][expert_ffn]) and down
 *     (W[expert_ffn][hidden]) carry strategy TSL_EXPERT; gate/up combine
 *     NONE, down combine SUM (a token's experts sit on different ranks,
 *     so the rank outputs are summed).  Ranks past n_experts hold none.
 *   TSL_MOE_WITHIN_EXPERT: every rank holds every expert, whose gate/up
 *     are column shards over [r*f/tp, (r+1)*f/tp) of expert_ffn (combine
 *     NONE) and whose down is the matching row shard (combine SUM), the
 *     dense FFN pattern of plan_shards.
 * Records go rank-major, experts ascending within a rank; *n_out receives
 * the count (n_experts, or tp * n_experts).  proj is TSL_GATE / TSL_UP /
 * TSL_DOWN, heads -1.  Errors, in this order: TSL_ERR_INVALID_ARG (null,
 * a size < 1, bad mode, group_size not 0 or 64, out_len short),
 * TSL_ERR_TP_NOT_POW2, TSL_ERR_NOT_DIVISIBLE (within-expert with
 * expert_ffn % tp), TSL_ERR_GROUP_ALIGN (group_size 64 with hidden or
 * expert_ffn, or a within-expert slice, not a multiple of 64).  Host only.
 */
tsl_status plan_experts(int32_t n_experts, int64_t hidden, int64_t expert_ffn, int32_t tp_size,
                        int32_t mode, int32_t group_size, tsl_expert_shard *out, int64_t out_len,
                        int64_t *n_out);

/*
 * pack_shard_size -- bytes of the packed, kernel-ready copy of a shard.
 * Let Ks = shard rows (k_len), Ns = shard columns (n_len),
 * Nt = ceil(Ns / 16).  Packed layouts (all little-endian, zero padded):
 *   TSL_F32   [Nt][ceil(Ks/64)*4][64][4] f32: element (k, n) of the shard
 *             sits in tile (n/16, k/16), lane ((k%16)/4)*16 + n%16, slot k%4.
 *   TSL_BF16  [Nt][ceil(Ks/64)*2][64][8] bf16: tile (n/16, k/32),
 *             lane ((k%32)/8)*16 + n%16, slot k%8.
 *   TSL_Q4G64 records [Nt][ceil(Ks/128)] of 1152 bytes (rounded up to
 *             256 bytes): codes [64][4] u32, then scale/bias pairs [16][2]
 *             u32 (bf16 scale in the low half, bf16 bias in the high half).
 *             Code (k, n): record (n/16, k/128); with kk = k%128, word
 *             kk/32 of lane ((kk%32)/8)*16 + n%16; with j = kk%8 the nibble
 *             at bit 4*(j/2) for even j and 16 + 4*(j/2) for odd j.
 *             Pair (g, n) for group g = k/64: record (n/16, g/2), entry
 *             [n%16][g%2] (the two groups of a 128-k block side by side).
 *             Then the column exponents [Nt*16] int32 (rounded up to 256
 *             bytes): f_n = ilogb(max over the column's groups of
 *             15|s| + |b|, in binary32) - 14, and 0 for a column whose
 *             groups are all zero or not finite (and for padding columns).
 * Errors: TSL_ERR_INVALID_ARG, TSL_ERR_GROUP_ALIGN (Q4 with k_len % 64).
 */
tsl_status pack_shard_size(const tsl_shard *shard, tsl_dtype wdtype, size_t *bytes);

/*
 * pack_shard -- slice a rank's shard out of the full logical W and write it
 * in the packed layout above ([mlxcel] "Column Parallel" / "Row Parallel":
 * rank r holds a contiguous block of columns or rows, in rank order).
 *   W (F32/BF16): device pointer; element W[k][n] of the FULL weight is at
 *       W[k * stride_k + n * stride_n] (stride_k = N, stride_n = 1 for a
 *       [K][N] array; stride_k = 1, stride_n = K for an [N][K] array).
 *   Q4G64: W points at one byte per code (values 0..15) addressed the same
 *       way; scales and biases are device bf16 arrays addressed
 *       [g * sb_stride_g + n * sb_stride_n] for group g = k / 64 of the
 *       full weight.  For F32/BF16 scales/biases must be NULL.
 *   packed: device buffer of at least pack_shard_size() bytes,
 *       256-byte aligned.
 * Runs one kernel on `stream`.  Source strides may be any non-negative
 * values; the caller guarantees every addressed element lies in its
 * allocation.  Errors: TSL_ERR_INVALID_ARG, TSL_ERR_GROUP_ALIGN,
 * TSL_ERR_BUFFER_TOO_SMALL, TSL_ERR_MISALIGNED, TSL_ERR_HIP.
 */
tsl_status pack_shard(const tsl_shard *shard, tsl_dtype wdtype, const void *W, int64_t stride_k,
                      int64_t stride_n, const void *scales, const void *biases,
                      int64_t sb_stride_g, int64_t sb_stride_n, void *packed,
                      size_t packed_bytes, void *stream);

/*
 * shard_linear_workspace_size -- workspace bytes shard_linear needs for
 * this shard, weight type and row count (0 when none is needed): split-K
 * partial sums for decode-sized M (every M for F32 weights, M <= 64 for
 * Q4G64, M <= 32 for BF16: the weights are streamed); above that (the
 * GEMM regime), for 4-bit weights a
 * binary16 copy of the activations (M x k_len x 2 bytes, k_len rounded up
 * to 64) and their row exponents (4 bytes per row, rows rounded up to 256)
 * -- the weights stay packed -- for BF16 weights a zero-padded copy of
 * the activations when k_len is not a multiple of 64, and when the product
 * is too small to fill the chip the binary32 partials of its k-splits
 * (splits x M x n_len x 4 bytes).
 */
tsl_status shard_linear_workspace_size(const tsl_shard *shard, tsl_dtype wdtype, int64_t M,
                                       size_t *bytes);

/*
 * shard_linear -- one rank's share of a linear layer ([wiki] "Details" §1:
 * column shard Y_i = X W_i with the input replicated, row shard
 * Y_i = X_i W_i with X_i the rank's block of input columns; [mlxcel]
 * "Column Parallel", "Row Parallel"):
 *     Y[m][j] (+)= sum_{i < k_len} X[m][i] * Wshard[i][j],  m < M, j < n_len
 *   packed:  the shard packed by pack_shard with the same `wdtype`.
 *   X:       device, xdtype, row m at X + m * ldx; k_len columns are read.
 *            For a row shard pass the rank's block X_i -- e.g. a pointer to
 *            column k_off of the full X with ldx = full width.
 *   Y:       device, ydtype, row m at Y + m * ldy; n_len columns written.
 *            For a concat-free column layer pass column n_off of the full
 *            output with ldy = N.
 *   accumulate: 0 stores the product; 1 adds it to Y (ydtype must be F32),
 *            which sums rank partials in call order.
 *   workspace: device, >= shard_linear_workspace_size() bytes (may be NULL
 *            when that is 0); its contents on entry do not matter.
 * Supported types: (wdtype, xdtype) = (F32, F32), (BF16, BF16),
 * (Q4G64, BF16); ydtype F32 or BF16 (round to nearest even).  Products
 * accumulate in binary32.  Q4G64 with M <= 64 applies the affine groups
 * exactly: the matrix cores multiply bf16 activations by 128 + q and each
 * group adds s * sum(x (128 + q)) + (b - 128 s) * sum(x) in binary32, so
 * activations must stay below 2^114 in magnitude (larger ones overflow
 * those group sums).  Q4G64 with M > 64 runs on binary16 operands, scaled
 * by powers of two for any finite bf16 input: activation row m becomes
 * x * 2^-e_m with e_m = ilogb(max_k |x[m][k]|) - 15 and weight column n
 * becomes (s * q + b) * 2^-f_n with f_n the packed column exponent, each
 * rounded to nearest binary16 (weights via binary32), and the binary32
 * result is multiplied by 2^(e_m + f_n).  Values within 2^29 of their
 * row's (column's) largest keep binary16 precision (relative error
 * <= 2^-11); smaller ones carry an absolute error of at most 2^(e_m - 25)
 * (2^(f_n - 25)).  Non-finite inputs give non-finite outputs.  M may be 0
 * (nothing is enqueued).
 * BF16 weights with M > 32 and Q4G64 weights with M > 64 (the GEMM regime)
 * require ldx and the shard's K below 2^22 elements (else
 * TSL_ERR_UNSUPPORTED).
 * Errors: TSL_ERR_INVALID_ARG, TSL_ERR_UNSUPPORTED,
 * TSL_ERR_BUFFER_TOO_SMALL, TSL_ERR_MISALIGNED (X, Y 16-byte aligned;
 * ldx, ldy multiples of 8 for 16-bit and of 4 for 32-bit types), TSL_ERR_HIP.
 */
tsl_status shard_linear(const tsl_shard *shard, tsl_dtype wdtype, const void *packed,
                        size_t packed_bytes, tsl_dtype xdtype, const void *X, int64_t ldx,
                        int64_t M, tsl_dtype ydtype, void *Y, int64_t ldy, int accumulate,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * One product of a grouped call: the per-product arguments of
 * shard_linear.  shard points at HOST memory read during the call only;
 * packed, X and Y are device pointers with the same meaning, layout and
 * alignment rules as in shard_linear; ydtype is this product's output type
 * (F32 or BF16).
 *
 * sum_next = 1 links the item to the next one.  A maximal run of linked
 * items is a SUM SET: the row-parallel shards of one layer, whose products
 * are added into the run's first item's Y -- the on-device rank sum
 * ([mlxcel] "Communication patterns", all-reduce after row shards; [wiki]
 * "Details" §1):
 *     Y = (((X_0 W_0 + X_1 W_1) + X_2 W_2) + ...)
 * each product in binary32 (its k-partials, if the launch splits k, added
 * in k order first), the sum in item order, rounded once to the first
 * item's ydtype -- the result of the same products followed by
 * combine_partials(SUM).  All items of a set have the same n_len; the first
 * item's Y, ldy and ydtype apply and its accumulate must be 0; the Y, ldy,
 * ydtype and accumulate of the other items are ignored.  The last item of
 * a call has sum_next = 0.  The products of a set go to binary32 partials
 * in the workspace (rows x n_len x 4 bytes each, counted by
 * shard_linear_group_workspace_size); one more launch adds them.
 * Exception, the GEMM regime (M > 64 for Q4G64, M > 32 for BF16): a set of
 * at most 8 members whose k_len are equal multiples of 128 (Q4G64 weights)
 * or of 64 (BF16 weights) is ONE product over the members' k-ranges laid
 * end to end in item order, Y = [X_0 X_1 ...] [W_0; W_1; ...]
 * -- the same sum, accumulated in binary32 in that k order inside the GEMM
 * and rounded once (bit for bit the product of the unsharded weight over
 * the whole X when the members are the row shards of one weight), with no
 * partials and no sum launch.
 * Decode-sized M whose activation rows the streaming launch holds in LDS
 * (one to four token rows, as far as they fit): the launch adds each set of
 * at most 8 unsplit members itself -- the members' binary32 products are
 * written through to device-coherent memory, a counter per 16-column tile
 * (8 bytes each in the workspace) counts their arrival, and the last to
 * arrive adds them in item order, the same sum bit for bit.  A counter
 * word holds a 48-bit ticket drawn afresh for every call (a graph replay
 * repeats its call's ticket and finds the counters reset to zero); a word
 * that any other use of the workspace left behind counts as zero unless
 * it happens to hold this call's ticket (odds 2^-48 per tile).  Calls that
 * overlap in time must not share a workspace.
 *
 * rows: the item's token rows, 1 <= rows <= M (0 means M): it reads rows
 * [0, rows) of X and writes rows [0, rows) of Y.  Items of different row
 * counts share one launch -- the per-expert products of a mixture-of-
 * experts layer, each over the tokens routed to its expert ([mlxcel] "MoE
 * expert parallelization").  The members of a sum set have equal rows.
 *
 * row_index: null, or DEVICE int32 [rows]: row i of the product reads row
 * row_index[i] of X, which then has x_rows rows (1 <= x_rows < 2^31); an
 * index outside [0, x_rows) reads a row of zeros.  The tokens routed to an
 * expert are read where they lie, with no gather pass of their own
 * ([mlxcel] "MoE expert parallelization"; moe_gather's idx has the same
 * meaning): with Q4G64 weights above 64 rows, and in calls of a few
 * decode-sized rows whose activations the streaming kernel keeps in LDS,
 * the kernels read them where they lie; otherwise the call first gathers
 * each distinct (X, ldx, k_len, row_index, rows) into its workspace (a
 * bf16 / fp32 copy, zeros for out-of-range rows).  row_index must be 4-byte aligned and must not
 * overlap any output; x_rows is ignored when row_index is null.
 */
typedef struct {
    const tsl_shard *shard;
    const void *packed;
    size_t packed_bytes;
    const void *X;
    int64_t ldx;
    void *Y;
    int64_t ldy;
    int32_t ydtype;
    int32_t accumulate;
    int32_t sum_next;
    int32_t rows;
    const int32_t *row_index;
    int64_t x_rows;
} tsl_linear_item;

/*
 * shard_linear_group_workspace_size -- workspace bytes shard_linear_group
 * needs for these items (only their shards, sum_next, rows and whether
 * row_index is null are read), weight type and M.  An upper bound: a call
 * whose items read the same X (same pointer, ldx, k_len and row_index)
 * shares one activation copy and uses less.
 */
tsl_status shard_linear_group_workspace_size(int32_t n_items, const tsl_linear_item *items,
                                             tsl_dtype wdtype, int64_t M, size_t *bytes);

/*
 * shard_linear_group -- several shard products with the same weight and
 * activation types, each over M rows or its own row count, in one pass: the projections that read the same input
 * (q, k and v, or gate and up, of a column-parallel block; [wiki]
 * "Details" §1, [mlxcel] "Column Parallel"), or the shards of every rank
 * when all ranks' shares run on one GPU.  Each item computes what
 * shard_linear computes for its arguments, to the same accuracy (a call
 * too small to fill the chip splits k -- decode-sized M, or a GEMM launch
 * of few tiles -- so a group and separate calls may add k-partials in
 * different groupings and need not agree bitwise).  The items run in no particular order: no
 * item's Y may share an element with another item's Y or any item's X
 * (TSL_ERR_INVALID_ARG); column blocks of one output matrix with a common
 * ldy are fine.  The kernels are chosen by M (the largest row count).
 * Up to 128 items share one kernel launch (256 in the prefill regime);
 * 1 <= n_items <= 4096.  items is a HOST array.
 * Errors: as shard_linear, for any item.
 */
tsl_status shard_linear_group(int32_t n_items, const tsl_linear_item *items, tsl_dtype wdtype,
                              tsl_dtype xdtype, int64_t M, void *workspace, size_t ws_bytes,
                              void *stream);

/*
 * shard_linear_group_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): shard_linear_group with no workspace argument.  Its
 * workspace is a fixed device array of TSL_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on (one copy per device, from the
 * library's first use there until the process ends); the call allocates no
 * device memory.  Items, types, results and errors are those of
 * shard_linear_group; a call whose workspace would exceed the array (the
 * exact amount for these items: products that read the same X count their
 * activation copy once) returns TSL_ERR_BUFFER_TOO_SMALL before anything is
 * enqueued.  Every call on one GPU uses that GPU's one array, which keeps
 * the previous call's contents (none of them is read as input): calls on
 * one stream are ordered, but calls that overlap in time on one GPU (other
 * streams, other threads) race on the array and must not be issued.
 */
#define TSL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
tsl_status shard_linear_group_noalloc(int32_t n_items, const tsl_linear_item *items,
                                      tsl_dtype wdtype, tsl_dtype xdtype, int64_t M,
                                      void *stream);

/*
 * combine_partials -- join rank outputs that all live on this one GPU
 * ([mlxcel] "Communication patterns": all-gather after column shards,
 * all-reduce after row shards; [wiki] "Details" §1 and "Examples" §1).
 *   parts:   HOST array of n_parts DEVICE pointers; part r is [M][n_each]
 *            with row stride ld_part, type pdtype.
 *   CONCAT:  Y[m][r * n_each + j] = part_r[m][j]; pdtype must equal ydtype
 *            (a copy).
 *   SUM:     Y[m][j] = (((part_0 + part_1) + part_2) + ...)[m][j], each
 *            addition in binary32 in ascending rank order; pdtype F32;
 *            ydtype F32 or BF16 (rounded once, nearest even).
 *   Y:       device, row stride ldy.  For SUM with ydtype F32 and
 *            ldy == ld_part, Y may be part 0 itself (each element is read
 *            before it is written); any other overlap of Y with a part is
 *            rejected (TSL_ERR_INVALID_ARG).
 * 1 <= n_parts <= 64.  M == 0 or n_each == 0 enqueues nothing.
 * Errors: TSL_ERR_INVALID_ARG, TSL_ERR_UNSUPPORTED, TSL_ERR_MISALIGNED,
 * TSL_ERR_HIP.
 */
tsl_status combine_partials(tsl_combine mode, int32_t n_parts, const void *const *parts,
                            tsl_dtype pdtype, int64_t M, int64_t n_each, int64_t ld_part,
                            tsl_dtype ydtype, void *Y, int64_t ldy, void *stream);

/* The collectives that join rank outputs (see combine_to_ranks). */
typedef enum tsl_collective {
    TSL_ALL_REDUCE = 0,     /* every rank: the full ordered sum            */
    TSL_REDUCE_SCATTER = 1, /* rank r: its block of rows of that sum       */
    TSL_ALL_GATHER = 2      /* every rank: the parts concatenated along N  */
} tsl_collective;

/*
 * combine_to_ranks -- every rank's result of a collective over rank outputs
 * that all live on this one GPU ([mlxcel] "Communication patterns": the
 * ring all-reduce = reduce-scatter then all-gather, after row-parallel
 * layers; all-gather of column shards; reduce-scatter when the next op
 * needs only a shard of the reduced output).
 *   parts: HOST array of n DEVICE pointers; part r is [M][n_each], row
 *          stride ld_part, type pdtype.
 *   outs:  HOST array of n DEVICE pointers; outs[r] is rank r's result,
 *          row stride ldo, type odtype.
 *   ALL_REDUCE:     outs[r][m][j] = (((P_0 + P_1) + P_2) + ...)[m][j] for
 *                   every r (binary32 adds in rank order, rounded once to
 *                   odtype); pdtype F32, odtype F32 or BF16.
 *   REDUCE_SCATTER: the same sum, rank r keeping rows lo_r <= m < hi_r with
 *                   lo_r = floor(r M / n), at outs[r][m - lo_r] (the ring's
 *                   n chunks in memory order, as whole rows).
 *   ALL_GATHER:     outs[r][m][q n_each + j] = P_q[m][j] for every r;
 *                   pdtype == odtype (a copy), F32 or BF16.
 * No output may share an element with a part or another output
 * (TSL_ERR_INVALID_ARG).  1 <= n <= 64.  M == 0 or n_each == 0 enqueues
 * nothing.  Errors: TSL_ERR_INVALID_ARG, TSL_ERR_UNSUPPORTED,
 * TSL_ERR_MISALIGNED (pointers aligned to their element size), TSL_ERR_HIP.
 */
tsl_status combine_to_ranks(tsl_collective op, int32_t n, const void *const *parts,
                            tsl_dtype pdtype, int64_t M, int64_t n_each, int64_t ld_part,
                            tsl_dtype odtype, void *const *outs, int64_t ldo, void *stream);

/*
 * embed_lookup -- one rank's share of a vocabulary-parallel embedding
 * lookup ([mlxcel] "Vocab Parallel": each rank looks up the tokens of its
 * vocabulary slice; the joined result is every token's full row).
 *   shard:  the rank's block W[k_off : k_off + k_len, n_off : n_off + n_len]
 *           of the table W[K = vocab][N = hidden] (TSL_EMBED records of
 *           plan_vocab; any strategy is accepted).
 *   table:  DEVICE, that block as k_len rows of n_len elements, row stride
 *           ld_table >= n_len, type tdtype (F32 or BF16).
 *   tokens: DEVICE int32 [M], token ids.
 *   Y:      DEVICE [M][ldy], ldy >= n_len, type ydtype (F32 or BF16).
 * Y[m][j] = W[t][n_off + j] for t = tokens[m] when k_off <= t < k_off +
 * k_len (widened exactly, or rounded to nearest-even for F32 -> BF16);
 * otherwise -0.0, the additive identity of IEEE round-to-nearest, so the
 * rank-ordered binary32 SUM of the partials (combine_partials,
 * combine_to_ranks) reproduces the owning rank's row bit for bit.  Ids
 * outside [0, vocab) are owned by no rank and give -0.0 rows everywhere.
 * M == 0 enqueues nothing.  Y must not overlap table or tokens.  Errors:
 * TSL_ERR_INVALID_ARG, TSL_ERR_MISALIGNED (pointers aligned to their
 * element size), TSL_ERR_HIP.
 */
tsl_status embed_lookup(const tsl_shard *shard, tsl_dtype tdtype, const void *table,
                        int64_t ld_table, const int32_t *tokens, int64_t M, tsl_dtype ydtype,
                        void *Y, int64_t ldy, void *stream);

/*
 * moe_dispatch -- the rows of one rank's expert products for a batch of
 * routed tokens ([mlxcel] "MoE expert parallelization": the router runs on
 * every rank, each rank runs only the experts it holds).  Host only.
 *   topk:    HOST int32 [T][k], token t's k chosen experts (router output).
 *   experts: HOST int32 [n_local], the experts this rank holds, in the
 *            order their products are laid out (distinct, < n_experts).
 * A row is one slot s = t*k + j whose expert the rank holds.  Rows are
 * grouped by expert in `experts` order, slots ascending within an expert:
 *   offsets:  HOST int64 [n_local + 1], expert i owns rows
 *             [offsets[i], offsets[i+1]).
 *   row_slot: HOST int32 [T*k] (first offsets[n_local] entries written),
 *             the slot of each row (its token is row_slot / k).
 *   slot_row: HOST int32 [T*k], the row of each slot, -1 for slots whose
 *             expert another rank holds.
 * T == 0 is allowed (offsets all 0).  Errors: TSL_ERR_INVALID_ARG (null,
 * T < 0, k < 1, T*k >= 2^31, n_experts < 1, n_local < 0, an id in topk or
 * experts outside [0, n_experts), an expert listed twice).
 */
tsl_status moe_dispatch(const int32_t *topk, int64_t T, int32_t k, int32_t n_experts,
                        const int32_t *experts, int32_t n_local, int64_t *offsets,
                        int32_t *row_slot, int32_t *slot_row);

/*
 * moe_gather -- out[i][:] = src[idx[i]][:] for i < n, width elements per
 * row: the activations of a rank's expert rows in the layout moe_dispatch
 * gives (idx = row_slot / k for token inputs, or row_slot for per-slot
 * inputs).  src DEVICE [n_src][ld_src], out DEVICE [n][ldo], both of
 * type dtype (F32 or BF16, copied bit for bit); idx DEVICE int32 [n].  An
 * index outside [0, n_src) gives a row of -0.0.  out must not overlap src
 * or idx.  n == 0 enqueues nothing.  Errors: TSL_ERR_INVALID_ARG,
 * TSL_ERR_MISALIGNED (pointers aligned to their element size), TSL_ERR_HIP.
 */
tsl_status moe_gather(const void *src, int64_t ld_src, int64_t n_src, tsl_dtype dtype,
                      const int32_t *idx, int64_t n, int64_t width, void *out, int64_t ldo,
                      void *stream);

/*
 * moe_combine -- one rank's share of the MoE output: each token's weighted
 * sum over its choices whose expert the rank holds ([mlxcel] "MoE expert
 * parallelization"; the rank shares add up over ranks like row-parallel
 * partials, combine_partials SUM):
 *   Y[t][j] = sum over s < k with 0 <= r = slot_row[t*k+s] < n_rows of
 *             weights[t*k+s] * P[r][j]
 * in binary32, s ascending, each term a fused multiply-add onto the
 * running sum, which starts at -0.0 (a token with no held choice gets
 * -0.0, the additive identity); rounded once to ydtype.
 *   P:        DEVICE binary32 [n_rows][ldp], the expert rows (e.g. the
 *             down products of shard_linear_group).
 *   slot_row: DEVICE int32 [T*k] (moe_dispatch); weights DEVICE binary32
 *             [T*k], the router weights.
 *   Y:        DEVICE [T][ldy], ydtype F32 or BF16; must not overlap the
 *             inputs.
 * T == 0 or n == 0 enqueues nothing.  Errors: TSL_ERR_INVALID_ARG,
 * TSL_ERR_MISALIGNED, TSL_ERR_HIP.
 */
tsl_status moe_combine(const float *P, int64_t ldp, int64_t n_rows, const int32_t *slot_row,
                       const float *weights, int64_t T, int32_t k, int64_t n, tsl_dtype ydtype,
                       void *Y, int64_t ldy, void *stream);

/* A static, human-readable description of a status code. */
const char *tsl_status_string(tsl_status status);

/* The HIP runtime's description of the error behind the most recent
 * TSL_ERR_HIP returned on the calling thread ("no error" if none). */
const char *tsl_last_hip_error_string(void);

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* TSL_H */
