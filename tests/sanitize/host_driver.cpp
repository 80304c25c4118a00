// Host-side checks of the C ABI for the sanitizer build: plans, sizes and
// every validation path that returns before a launch, run under
// AddressSanitizer and UndefinedBehaviorSanitizer (no GPU is touched).
// Exits 0 when every call returned the status the header promises.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "tsl.h"

static int failures = 0;
#define EXPECT(cond)                                                                               \
    do {                                                                                           \
        if (!(cond)) {                                                                             \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);                             \
            ++failures;                                                                            \
        }                                                                                          \
    } while (0)

// fake device addresses: validated, never dereferenced
static void *addr(uint64_t a) { return reinterpret_cast<void *>(a); }

static void plans() {
    const tsl_dims cfgs[] = {{2048, 32, 8, 64, 8192, 4, 0},    {3584, 28, 4, 128, 18944, 4, 64},
                             {5120, 64, 8, 128, 17408, 4, 64}, {4096, 32, 4, 128, 14336, 8, 0},
                             {1024, 8, 8, 128, 4096, 1, 0}};
    for (const tsl_dims &d : cfgs) {
        std::vector<tsl_shard> s(7 * d.tp_size);
        EXPECT(plan_shards(&d, s.data(), (int64_t)s.size()) == TSL_OK);
        EXPECT(plan_shards(&d, s.data(), (int64_t)s.size() - 1) == TSL_ERR_INVALID_ARG);
        for (const tsl_shard &x : s) {
            size_t nb = 0;
            const tsl_dtype w = d.group_size ? TSL_Q4G64 : TSL_BF16;
            EXPECT(pack_shard_size(&x, w, &nb) == TSL_OK && nb > 0);
            for (int64_t M : {0, 1, 4, 16, 65, 2048}) {
                size_t ws = 0;
                EXPECT(shard_linear_workspace_size(&x, w, M, &ws) == TSL_OK);
            }
        }
    }
    // a grid of shapes, valid and not
    for (int tp = 1; tp <= 16; ++tp)
        for (int hq : {1, 4, 6, 32})
            for (int hkv : {1, 2, 3, 8}) {
                tsl_dims d = {512, hq, hkv, 64, 1024, tp, (tp & 1) ? 0 : 64};
                std::vector<tsl_shard> s(7 * tp);
                const tsl_status st = plan_shards(&d, s.data(), (int64_t)s.size());
                EXPECT(st == TSL_OK || st == TSL_ERR_NOT_DIVISIBLE || st == TSL_ERR_TP_NOT_POW2 ||
                       st == TSL_ERR_INVALID_ARG || st == TSL_ERR_GROUP_ALIGN);
            }
    EXPECT(plan_shards(nullptr, nullptr, 0) == TSL_ERR_INVALID_ARG);
    tsl_shard lin[8];
    EXPECT(plan_linear(1024, 2048, 2, TSL_COLUMN, 0, lin, 8) == TSL_OK);
    EXPECT(plan_linear(1024, 2048, 3, TSL_COLUMN, 0, lin, 8) == TSL_ERR_TP_NOT_POW2);
    EXPECT(plan_linear(1000, 2048, 8, TSL_ROW, 64, lin, 8) != TSL_OK);
    tsl_shard voc[8];
    EXPECT(plan_vocab(152064, 3584, 4, 64, voc, 8) == TSL_OK);
    EXPECT(plan_vocab(152065, 3584, 4, 64, voc, 8) == TSL_ERR_NOT_DIVISIBLE);
    std::vector<tsl_expert_shard> ex(128 * 4);
    int64_t n_out = 0;
    EXPECT(plan_experts(128, 2048, 768, 4, TSL_MOE_EXPERT_PARALLEL, 64, ex.data(),
                        (int64_t)ex.size(), &n_out) == TSL_OK && n_out == 128);
    EXPECT(plan_experts(128, 2048, 768, 4, TSL_MOE_WITHIN_EXPERT, 64, ex.data(),
                        (int64_t)ex.size(), &n_out) == TSL_OK);
    EXPECT(plan_experts(0, 2048, 768, 4, 0, 64, ex.data(), 1, &n_out) == TSL_ERR_INVALID_ARG);
}

static void validation() {
    tsl_shard s[2];
    EXPECT(plan_linear(1024, 256, 1, TSL_COLUMN, 64, s, 2) == TSL_OK);
    size_t nb = 0;
    EXPECT(pack_shard_size(&s[0], TSL_Q4G64, &nb) == TSL_OK);
    void *P = addr(1ull << 36), *X = addr(2ull << 36), *Y = addr(3ull << 36);
    // rejected before any launch
    EXPECT(shard_linear(&s[0], TSL_Q4G64, nullptr, nb, TSL_BF16, X, 1024, 8, TSL_F32, Y, 256, 0,
                        nullptr, 0, nullptr) == TSL_ERR_INVALID_ARG);
    EXPECT(shard_linear(&s[0], TSL_Q4G64, P, nb - 1, TSL_BF16, X, 1024, 8, TSL_F32, Y, 256, 0,
                        nullptr, 0, nullptr) == TSL_ERR_BUFFER_TOO_SMALL);
    EXPECT(shard_linear(&s[0], TSL_Q4G64, P, nb, TSL_BF16, addr((2ull << 36) + 2), 1024, 8,
                        TSL_F32, Y, 256, 0, nullptr, 0, nullptr) == TSL_ERR_MISALIGNED);
    EXPECT(shard_linear(&s[0], TSL_Q4G64, P, nb, TSL_F32, X, 1024, 8, TSL_F32, Y, 256, 0, nullptr,
                        0, nullptr) != TSL_OK);
    EXPECT(shard_linear(&s[0], TSL_Q4G64, P, nb, TSL_BF16, X, 1024, -1, TSL_F32, Y, 256, 0,
                        nullptr, 0, nullptr) == TSL_ERR_INVALID_ARG);
    // M = 0 enqueues nothing
    EXPECT(shard_linear(&s[0], TSL_Q4G64, P, nb, TSL_BF16, X, 1024, 0, TSL_F32, Y, 256, 0, nullptr,
                        0, nullptr) == TSL_OK);
    // a workspace the call needs but does not get
    size_t ws = 0;
    EXPECT(shard_linear_workspace_size(&s[0], TSL_Q4G64, 2048, &ws) == TSL_OK && ws > 0);
    EXPECT(shard_linear(&s[0], TSL_Q4G64, P, nb, TSL_BF16, X, 1024, 2048, TSL_F32, Y, 256, 0,
                        nullptr, 0, nullptr) == TSL_ERR_BUFFER_TOO_SMALL);
    // grouped: an output overlapping another item's input
    tsl_linear_item it[2] = {{&s[0], P, nb, X, 1024, Y, 256, TSL_F32, 0, 0, 0},
                             {&s[0], P, nb, X, 1024, X, 256, TSL_F32, 0, 0, 0}};
    EXPECT(shard_linear_group(2, it, TSL_Q4G64, TSL_BF16, 8, nullptr, 0, nullptr) ==
           TSL_ERR_INVALID_ARG);
    EXPECT(shard_linear_group(0, it, TSL_Q4G64, TSL_BF16, 8, nullptr, 0, nullptr) ==
           TSL_ERR_INVALID_ARG);
    size_t gws = 0;
    it[1].Y = addr(4ull << 36);
    it[0].sum_next = 1;
    EXPECT(shard_linear_group_workspace_size(2, it, TSL_Q4G64, 2048, &gws) == TSL_OK && gws > 0);
    EXPECT(shard_linear_group_workspace_size(2, it, TSL_Q4G64, 4, &gws) == TSL_OK);
    // the allocation-free entry point: beyond its scratch, decided on the host
    tsl_shard big[1];
    EXPECT(plan_linear(8192, 1024, 1, TSL_COLUMN, 64, big, 1) == TSL_OK);
    size_t bnb = 0;
    EXPECT(pack_shard_size(&big[0], TSL_Q4G64, &bnb) == TSL_OK);
    tsl_linear_item one = {&big[0], P, bnb, X, 8192, Y, 1024, TSL_F32, 0, 0, 0};
    EXPECT(shard_linear_group_noalloc(1, &one, TSL_Q4G64, TSL_BF16, 8192, nullptr) ==
           TSL_ERR_BUFFER_TOO_SMALL);
    // combine
    const void *parts[2] = {addr(5ull << 36), addr(6ull << 36)};
    EXPECT(combine_partials(TSL_COMBINE_SUM, 0, parts, TSL_F32, 4, 8, 8, TSL_F32, Y, 8, nullptr) ==
           TSL_ERR_INVALID_ARG);
    EXPECT(combine_partials(TSL_COMBINE_SUM, 2, parts, TSL_F32, 4, 8, 8, TSL_F32, addr(6ull << 36), 8,
                            nullptr) == TSL_ERR_INVALID_ARG);
    EXPECT(combine_partials(TSL_COMBINE_SUM, 2, parts, TSL_F32, 0, 8, 8, TSL_F32, Y, 8, nullptr) ==
           TSL_OK);
    for (int st = -8; st <= 0; ++st)
        EXPECT(tsl_status_string((tsl_status)st) != nullptr);
}

static void dispatch() {
    const int T = 257, k = 8, E = 128;
    std::vector<int32_t> topk(T * k);
    uint32_t x = 12345;
    for (int32_t &v : topk) {
        x = x * 1664525u + 1013904223u;
        v = (int32_t)((x >> 8) % E);
    }
    std::vector<int32_t> experts;
    for (int e = 1; e < E; e += 4)
        experts.push_back(e);
    std::vector<int64_t> off(experts.size() + 1);
    std::vector<int32_t> row_slot(T * k), slot_row(T * k);
    EXPECT(moe_dispatch(topk.data(), T, k, E, experts.data(), (int32_t)experts.size(), off.data(),
                        row_slot.data(), slot_row.data()) == TSL_OK);
    for (size_t i = 0; i + 1 < off.size(); ++i)
        EXPECT(off[i] <= off[i + 1]);
    for (int64_t r = 0; r < off.back(); ++r)
        EXPECT(slot_row[row_slot[r]] == r);
    experts.push_back(experts[0]); // listed twice
    off.resize(experts.size() + 1);
    EXPECT(moe_dispatch(topk.data(), T, k, E, experts.data(), (int32_t)experts.size(), off.data(),
                        row_slot.data(), slot_row.data()) == TSL_ERR_INVALID_ARG);
    EXPECT(moe_dispatch(topk.data(), 0, k, E, experts.data(), 1, off.data(), row_slot.data(),
                        slot_row.data()) == TSL_OK);
}

int main() {
    plans();
    validation();
    dispatch();
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("host driver: all checks passed\n");
    return failures ? 1 : 0;
}
