// Shard planning: which block of each weight a rank holds and how the rank
// outputs are joined.  Host code, integer arithmetic only.
//
// Sources: mlxcel manual "Tensor parallelism" -- "Weight sharding strategy"
// (Column Parallel, Row Parallel, Replicated), "Architecture-aware shard
// plan" (standard transformer table), "GQA-aware attention sharding",
// "Configuration" (--tp-size is a power of two).
#include <stdint.h>

#include <vector>

#include "tsl.h"

namespace {

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// One row of the standard-transformer plan table: the strategy and the
// combine that follows it.  K/V are listed as column shards; the GQA rule
// below may turn them into replicated ones.
struct TableRow {
    tsl_proj proj;
    tsl_strategy strategy;
    tsl_combine combine;
};
constexpr TableRow kStandardTransformer[TSL_NPROJ] = {
    {TSL_Q, TSL_COLUMN, TSL_COMBINE_CONCAT},   // q_proj: column, all-gather
    {TSL_K, TSL_COLUMN, TSL_COMBINE_CONCAT},   // k_proj: column, GQA-aware
    {TSL_V, TSL_COLUMN, TSL_COMBINE_CONCAT},   // v_proj: column, GQA-aware
    {TSL_O, TSL_ROW, TSL_COMBINE_SUM},         // o_proj: row, all-reduce
    {TSL_GATE, TSL_COLUMN, TSL_COMBINE_NONE},  // gate_proj: column, none
    {TSL_UP, TSL_COLUMN, TSL_COMBINE_NONE},    // up_proj: column, none
    {TSL_DOWN, TSL_ROW, TSL_COMBINE_SUM},      // down_proj: row, all-reduce
};

// A contiguous block [part * width, (part + 1) * width) of a dimension.
struct Block {
    int64_t off, len;
};
Block block_of(int64_t total, int64_t parts, int64_t part) {
    int64_t w = total / parts;
    return {part * w, w};
}

tsl_shard make(tsl_proj proj, int32_t rank, tsl_strategy st, tsl_combine cb, int64_t K, int64_t N) {
    tsl_shard s{};
    s.proj = proj;
    s.rank = rank;
    s.strategy = st;
    s.combine = cb;
    s.K = K;
    s.N = N;
    s.k_off = 0;
    s.k_len = K;
    s.n_off = 0;
    s.n_len = N;
    s.head_off = -1;
    s.head_cnt = -1;
    return s;
}

} // namespace

extern "C" tsl_status plan_shards(const tsl_dims *d, tsl_shard *out, int64_t out_len) {
    if (!d || !out)
        return TSL_ERR_INVALID_ARG;
    const int64_t tp = d->tp_size;
    if (d->hidden < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
        d->ffn < 1 || tp < 1)
        return TSL_ERR_INVALID_ARG;
    if (d->group_size != 0 && d->group_size != 64)
        return TSL_ERR_INVALID_ARG;
    if (out_len < tp * TSL_NPROJ)
        return TSL_ERR_INVALID_ARG;
    if (!pow2(tp))
        return TSL_ERR_TP_NOT_POW2;

    const int64_t hq = d->n_q_heads, hkv = d->n_kv_heads, hd = d->head_dim;
    const int64_t hidden = d->hidden, ffn = d->ffn, grp = d->group_size;
    if (hq % hkv || hq % tp || ffn % tp)
        return TSL_ERR_NOT_DIVISIBLE;
    // GQA rule: shard K/V by heads only when every rank gets whole heads.
    const bool kv_replicated = hkv < tp;
    if (!kv_replicated && hkv % tp)
        return TSL_ERR_NOT_DIVISIBLE;

    if (grp) {
        // Inputs of every projection and the edges of the two row shards.
        const int64_t edges[] = {hidden, hq * hd, ffn, (hq / tp) * hd, ffn / tp};
        for (int64_t e : edges)
            if (e % grp)
                return TSL_ERR_GROUP_ALIGN;
    }

    for (int64_t r = 0; r < tp; ++r) {
        for (const TableRow &row : kStandardTransformer) {
            const tsl_proj p = row.proj;
            tsl_shard s;
            Block heads{0, 0};
            switch (p) {
            case TSL_Q:
                s = make(p, (int32_t)r, row.strategy, row.combine, hidden, hq * hd);
                heads = block_of(hq, tp, r);
                s.n_off = heads.off * hd;
                s.n_len = heads.len * hd;
                break;
            case TSL_K:
            case TSL_V:
                if (kv_replicated) {
                    s = make(p, (int32_t)r, TSL_REPLICATED, TSL_COMBINE_NONE, hidden, hkv * hd);
                    heads = {0, hkv};
                } else {
                    s = make(p, (int32_t)r, row.strategy, row.combine, hidden, hkv * hd);
                    heads = block_of(hkv, tp, r);
                    s.n_off = heads.off * hd;
                    s.n_len = heads.len * hd;
                }
                break;
            case TSL_O:
                // Row block = the columns the same rank's q shard produced.
                s = make(p, (int32_t)r, row.strategy, row.combine, hq * hd, hidden);
                heads = block_of(hq, tp, r);
                s.k_off = heads.off * hd;
                s.k_len = heads.len * hd;
                break;
            case TSL_GATE:
            case TSL_UP: {
                s = make(p, (int32_t)r, row.strategy, row.combine, hidden, ffn);
                Block b = block_of(ffn, tp, r);
                s.n_off = b.off;
                s.n_len = b.len;
                break;
            }
            default: { // TSL_DOWN: row block = the gate/up columns of this rank
                s = make(p, (int32_t)r, row.strategy, row.combine, ffn, hidden);
                Block b = block_of(ffn, tp, r);
                s.k_off = b.off;
                s.k_len = b.len;
                break;
            }
            }
            if (p <= TSL_O) {
                s.head_off = (int32_t)heads.off;
                s.head_cnt = (int32_t)heads.len;
            }
            out[r * TSL_NPROJ + p] = s;
        }
    }
    return TSL_OK;
}

extern "C" tsl_status plan_linear(int64_t K, int64_t N, int32_t tp, int32_t strategy,
                                  int32_t group_size, tsl_shard *out, int64_t out_len) {
    if (!out || K < 1 || N < 1 || tp < 1)
        return TSL_ERR_INVALID_ARG;
    if (strategy != TSL_COLUMN && strategy != TSL_ROW && strategy != TSL_REPLICATED)
        return TSL_ERR_INVALID_ARG;
    if (group_size != 0 && group_size != 64)
        return TSL_ERR_INVALID_ARG;
    if (out_len < tp)
        return TSL_ERR_INVALID_ARG;
    if (!pow2(tp))
        return TSL_ERR_TP_NOT_POW2;
    if (strategy == TSL_COLUMN && N % tp)
        return TSL_ERR_NOT_DIVISIBLE;
    if (strategy == TSL_ROW && K % tp)
        return TSL_ERR_NOT_DIVISIBLE;
    if (group_size && (K % group_size || (strategy == TSL_ROW && (K / tp) % group_size)))
        return TSL_ERR_GROUP_ALIGN;

    for (int32_t r = 0; r < tp; ++r) {
        tsl_shard s;
        if (strategy == TSL_COLUMN) {
            s = make(TSL_LINEAR, r, TSL_COLUMN, TSL_COMBINE_CONCAT, K, N);
            Block b = block_of(N, tp, r);
            s.n_off = b.off;
            s.n_len = b.len;
        } else if (strategy == TSL_ROW) {
            s = make(TSL_LINEAR, r, TSL_ROW, TSL_COMBINE_SUM, K, N);
            Block b = block_of(K, tp, r);
            s.k_off = b.off;
            s.k_len = b.len;
        } else {
            s = make(TSL_LINEAR, r, TSL_REPLICATED, TSL_COMBINE_NONE, K, N);
        }
        out[r] = s;
    }
    return TSL_OK;
}

// Vocabulary-parallel embedding and LM head: the vocabulary dimension of
// both is cut into tp contiguous slices in rank order (mlxcel "Vocab
// Parallel").  The table E[vocab][hidden] is a linear W[vocab][hidden] fed a
// one-hot row, so its vocabulary slice is a row shard joined by a sum; the
// LM head W[hidden][vocab] is a column shard joined by a concat.
extern "C" tsl_status plan_vocab(int64_t vocab, int64_t hidden, int32_t tp, int32_t group_size,
                                 tsl_shard *out, int64_t out_len) {
    if (!out || vocab < 1 || hidden < 1 || tp < 1)
        return TSL_ERR_INVALID_ARG;
    if (group_size != 0 && group_size != 64)
        return TSL_ERR_INVALID_ARG;
    if (out_len < 2 * (int64_t)tp)
        return TSL_ERR_INVALID_ARG;
    if (!pow2(tp))
        return TSL_ERR_TP_NOT_POW2;
    if (vocab % tp)
        return TSL_ERR_NOT_DIVISIBLE;
    if (group_size && hidden % group_size)
        return TSL_ERR_GROUP_ALIGN;
    for (int32_t r = 0; r < tp; ++r) {
        const Block b = block_of(vocab, tp, r);
        tsl_shard e = make(TSL_EMBED, r, TSL_ROW, TSL_COMBINE_SUM, vocab, hidden);
        e.k_off = b.off;
        e.k_len = b.len;
        tsl_shard h = make(TSL_LM_HEAD, r, TSL_COLUMN, TSL_COMBINE_CONCAT, hidden, vocab);
        h.n_off = b.off;
        h.n_len = b.len;
        out[2 * r] = e;
        out[2 * r + 1] = h;
    }
    return TSL_OK;
}

// Mixture-of-experts FFN (mlxcel "MoE expert parallelization").  Expert
// parallel: experts dealt round-robin, expert e whole on rank e % tp, so
// each rank runs only its own experts and the token outputs of the ranks
// are summed.  Within-expert: each expert's gate/up/down split across all
// ranks exactly like the dense FFN (column gate/up, row down, sum).
extern "C" tsl_status plan_experts(int32_t n_experts, int64_t hidden, int64_t expert_ffn,
                                   int32_t tp, int32_t mode, int32_t group_size,
                                   tsl_expert_shard *out, int64_t out_len, int64_t *n_out) {
    if (!out || !n_out || n_experts < 1 || hidden < 1 || expert_ffn < 1 || tp < 1)
        return TSL_ERR_INVALID_ARG;
    if (mode != TSL_MOE_EXPERT_PARALLEL && mode != TSL_MOE_WITHIN_EXPERT)
        return TSL_ERR_INVALID_ARG;
    if (group_size != 0 && group_size != 64)
        return TSL_ERR_INVALID_ARG;
    const bool ep = mode == TSL_MOE_EXPERT_PARALLEL;
    const int64_t count = ep ? (int64_t)n_experts : (int64_t)tp * n_experts;
    if (out_len < count)
        return TSL_ERR_INVALID_ARG;
    if (!pow2(tp))
        return TSL_ERR_TP_NOT_POW2;
    if (!ep && expert_ffn % tp)
        return TSL_ERR_NOT_DIVISIBLE;
    if (group_size &&
        (hidden % group_size || expert_ffn % group_size || (!ep && (expert_ffn / tp) % group_size)))
        return TSL_ERR_GROUP_ALIGN;
    int64_t k = 0;
    for (int32_t r = 0; r < tp; ++r) {
        for (int32_t e = ep ? r : 0; e < n_experts; e += ep ? tp : 1) {
            tsl_expert_shard x;
            x.expert = e;
            x.rank = r;
            if (ep) {
                x.gate = make(TSL_GATE, r, TSL_EXPERT, TSL_COMBINE_NONE, hidden, expert_ffn);
                x.up = make(TSL_UP, r, TSL_EXPERT, TSL_COMBINE_NONE, hidden, expert_ffn);
                x.down = make(TSL_DOWN, r, TSL_EXPERT, TSL_COMBINE_SUM, expert_ffn, hidden);
            } else {
                const Block b = block_of(expert_ffn, tp, r);
                x.gate = make(TSL_GATE, r, TSL_COLUMN, TSL_COMBINE_NONE, hidden, expert_ffn);
                x.gate.n_off = b.off;
                x.gate.n_len = b.len;
                x.up = x.gate;
                x.up.proj = TSL_UP;
                x.down = make(TSL_DOWN, r, TSL_ROW, TSL_COMBINE_SUM, expert_ffn, hidden);
                x.down.k_off = b.off;
                x.down.k_len = b.len;
            }
            out[k++] = x;
        }
    }
    *n_out = k;
    return TSL_OK;
}

// The rows of a rank's expert products (mlxcel "MoE expert
// parallelization": every rank routes every token and runs its own
// experts): a counting sort of the slots t*k + j by expert, stable in slot
// order, over the experts the rank holds.
extern "C" tsl_status moe_dispatch(const int32_t *topk, int64_t T, int32_t k, int32_t n_experts,
                                   const int32_t *experts, int32_t n_local, int64_t *offsets,
                                   int32_t *row_slot, int32_t *slot_row) {
    if (T < 0 || k < 1 || n_experts < 1 || n_local < 0 || !offsets)
        return TSL_ERR_INVALID_ARG;
    if (T > (int64_t)(INT32_MAX - 1) / k)
        return TSL_ERR_INVALID_ARG;
    const int64_t S = T * k;
    if (S > 0 && (!topk || !row_slot || !slot_row))
        return TSL_ERR_INVALID_ARG;
    if (n_local > 0 && !experts)
        return TSL_ERR_INVALID_ARG;
    std::vector<int32_t> local(n_experts, -1); // expert -> index in `experts`
    for (int32_t i = 0; i < n_local; ++i) {
        const int32_t e = experts[i];
        if (e < 0 || e >= n_experts || local[e] >= 0)
            return TSL_ERR_INVALID_ARG;
        local[e] = i;
    }
    std::vector<int64_t> count(n_local + 1, 0);
    for (int64_t s = 0; s < S; ++s) {
        const int32_t e = topk[s];
        if (e < 0 || e >= n_experts)
            return TSL_ERR_INVALID_ARG;
        if (local[e] >= 0)
            ++count[local[e] + 1];
    }
    offsets[0] = 0;
    for (int32_t i = 0; i < n_local; ++i)
        offsets[i + 1] = offsets[i] + count[i + 1];
    std::vector<int64_t> next(offsets, offsets + n_local + 1);
    for (int64_t s = 0; s < S; ++s) {
        const int32_t li = local[topk[s]];
        if (li < 0) {
            slot_row[s] = -1;
            continue;
        }
        const int64_t r = next[li]++;
        row_slot[r] = (int32_t)s;
        slot_row[s] = (int32_t)r;
    }
    return TSL_OK;
}
