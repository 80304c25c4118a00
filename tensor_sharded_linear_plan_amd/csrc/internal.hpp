// Internal interface between the C-ABI layer (abi.cpp) and the HIP kernel
// translation units.  Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "tsl.h"

namespace tsl {

// Packed-layout geometry of one shard (see pack_shard_size in tsl.h).
struct PackGeom {
    int64_t Ks = 0, Ns = 0; // shard rows (input dim) and columns (output dim)
    int64_t Nt = 0;         // 16-column tiles
    int64_t Kpad = 0;       // Ks rounded up to the k granularity of the layout
    // F32: 16-k tiles; BF16: 32-k tiles; Q4G64: 128-k blocks
    int64_t KT = 0;
    size_t total_bytes = 0;
    // Q4G64: byte offset of the column exponents ([Nt * 16] int32 after
    // the records), see launch_pack_q4
    size_t exp_off = 0;
};

tsl_status geometry(const tsl_shard &s, tsl_dtype wdtype, PackGeom *g);

// Q4G64 packed record of 16 columns x 128 k: 1 KB of codes, then the 128
// bytes of (scale, bias) pairs of its two 64-k groups.
constexpr int kQ4Record = 1152;
constexpr int kQ4PairsAt = 1024;

// Binary16 operands of the GEMM regime.  Column n of a 4-bit shard carries
// an exponent f_n with every weight (s q + b) 2^-f_n below 2^15 in
// magnitude (ilogb of the column's largest 15 |s| + |b|, minus 14); an
// activation row m is scaled by 2^-e_m with e_m = ilogb(max |x|) - 15, so
// its largest element lies in [2^15, 2^16), below the binary16 maximum
// 65504 for every bf16 value.  The GEMM's binary32 result is multiplied
// back by 2^(e_m + f_n).
constexpr int kWeightExpBias = 14;
constexpr int kActExpBias = 15;

// ---- pack.hip ----
hipError_t launch_pack_dense(const PackGeom &g, tsl_dtype wdtype, const void *W, int64_t stride_k,
                             int64_t stride_n, int64_t k_off, int64_t n_off, void *packed,
                             hipStream_t stream);
hipError_t launch_pack_q4(const PackGeom &g, const uint8_t *codes, int64_t stride_k,
                          int64_t stride_n, const uint16_t *scales, const uint16_t *biases,
                          int64_t sb_stride_g, int64_t sb_stride_n, int64_t k_off, int64_t n_off,
                          void *packed, hipStream_t stream);

// ---- combine.hip ----
constexpr int kMaxParts = 64;
hipError_t launch_combine_sum(int n_parts, const float *const *parts, int64_t M, int64_t n_each,
                              int64_t ld_part, tsl_dtype ydtype, void *Y, int64_t ldy,
                              hipStream_t stream);
hipError_t launch_combine_concat(int n_parts, const void *const *parts, size_t elem_bytes,
                                 int64_t M, int64_t n_each, int64_t ld_part, void *Y, int64_t ldy,
                                 hipStream_t stream);
// Rank sums of several sum sets in one launch: set i adds its n_parts
// products in order into Y (row stride ldy, F32 or BF16); product r is the
// sum, in k order, of ks[r] contiguous [M_i][n] binary32 k-partials starting
// at parts[r] (ks[r] == 1: the product itself).  n_parts <= kSetParts; M is
// the largest M_i.
constexpr int kSetParts = 8;
constexpr int kMaxSets = 64;
struct SumSpec {
    const float *parts[kSetParts];
    int ks[kSetParts] = {1, 1, 1, 1, 1, 1, 1, 1};
    int n_parts = 0;
    int64_t M = 0; // rows of this set
    int64_t n = 0;
    void *Y = nullptr;
    int64_t ldy = 0;
    tsl_dtype ydtype = TSL_F32;
};
hipError_t launch_sum_sets(int n_sets, const SumSpec *sets, int64_t M, hipStream_t stream);
// Every rank's result of a collective (combine_to_ranks in tsl.h):
// scatter 0 writes the ordered sum to every output, 1 each output its row
// block; the gather copies the parts side by side into every output.
hipError_t launch_reduce_to_ranks(int n, const float *const *parts, int64_t M, int64_t n_each,
                                  int64_t ld_part, int scatter, tsl_dtype odtype,
                                  void *const *outs, int64_t ldo, hipStream_t stream);
hipError_t launch_gather_to_ranks(int n, const void *const *parts, size_t elem_bytes, int64_t M,
                                  int64_t n_each, int64_t ld_part, void *const *outs, int64_t ldo,
                                  hipStream_t stream);
// Y (+)= sum_{s < ks} P[s], P is [ks][M][N] f32 contiguous, ascending s.
hipError_t launch_splitk_reduce(const float *P, int ks, int64_t M, int64_t N, tsl_dtype ydtype,
                                void *Y, int64_t ldy, int accumulate, hipStream_t stream);

// ---- embed.hip ----
// Y[m][j] = table[(tokens[m] - k_off) * ld_table + j] when the token lies in
// [k_off, k_off + k_len), else -0.0; j < n_len.  Types F32 / BF16.
hipError_t launch_embed_lookup(tsl_dtype tdtype, const void *table, int64_t ld_table,
                               const int32_t *tokens, int64_t M, int64_t k_off, int64_t k_len,
                               int64_t n_len, tsl_dtype ydtype, void *Y, int64_t ldy,
                               hipStream_t stream);

// ---- moe.hip ----
// Y[t][j] = sum over held slots s < k of weights[t k + s] * P[slot_row[t k + s]][j],
// binary32 fused multiply-adds from -0.0, rounded once to ydtype.
hipError_t launch_moe_combine(const float *P, int64_t ldp, int64_t n_rows, const int32_t *slot_row,
                              const float *weights, int64_t T, int k, int64_t n, tsl_dtype ydtype,
                              void *Y, int64_t ldy, hipStream_t stream);

// One shard product of a (possibly grouped) shard_linear call, validated.
struct LinearItem {
    PackGeom g;
    const void *packed = nullptr;
    const void *X = nullptr;
    int64_t ldx = 0;
    void *Y = nullptr;
    int64_t ldy = 0;
    tsl_dtype ydtype = TSL_F32;
    int accumulate = 0;
    // sum sets (rank partials added in item order into the first item's
    // Y): the first item holds the set's length, the others 0, and each
    // item its position in the set
    int set_len = 1;
    int set_pos = 0;
    // token rows of this product (the call's M unless the item sets its own)
    int64_t M = 0;
    // row i of the product reads row ridx[i] of X (x_rows rows; an index
    // outside [0, x_rows) reads zeros); null: row i
    const int32_t *ridx = nullptr;
    int64_t x_rows = 0;
    // the GEMM path may not split this product's k (a member of a sum set
    // too long for one sum launch)
    bool no_split = false;
    // member fset_pos of a sum set of fset_len products that split_sets
    // turned into lone items (0: none), and the set's own output
    int fset_len = 0, fset_pos = 0;
    void *fset_Y = nullptr;
    int64_t fset_ldy = 0;
    tsl_dtype fset_ydtype = TSL_F32;
    // a sum set computed as ONE product over its members' k-ranges laid end
    // to end in set order (GEMM regime): cat members of equal k_len; g, Y,
    // ldy, ydtype describe the joined product, seg_* each member's packed
    // weights and activations (X, ldx, ridx and packed unused)
    int cat = 1;
    const void *seg_packed[kSetParts] = {};
    const void *seg_X[kSetParts] = {};
    int64_t seg_ldx[kSetParts] = {};
    const int32_t *seg_ridx[kSetParts] = {};
    int64_t seg_xrows[kSetParts] = {};
};

// Workgroups per CU of the fused 4-bit GEMM for a bm x bn tile with wm row
// waves: two when one row wave per SIMD leaves room for a second workgroup
// in half the LDS (at least four 32-k activation stages beside three
// record slots), else one.
constexpr int q4_tiles_per_cu(int bm, int bn, int wm) {
    return wm == 1 && (160 * 1024 / 2 - 3 * (bn / 16) * kQ4Record) / (bm * 64) >= 4 ? 2 : 1;
}

// ---- noalloc.hip: the fixed device scratch of shard_linear_group_noalloc ----
constexpr size_t kNoAllocScratchBytes = TSL_NOALLOC_SCRATCH_BYTES;
// The current device's copy of the scratch array (its address looked up once
// per device, on first use).
hipError_t noalloc_scratch(void **ptr);

// Items per kernel launch (the item table travels in the kernel arguments,
// up to ~13 KB of them); longer groups are launched in chunks of this size.
constexpr int kGroupMax = 128;
// ... for the prefill GEMMs and their activation pass: 256 (up to ~27 KB of
// kernel arguments, within the 32 KB this runtime launches correctly), so
// that e.g. the gate and up products of 128 experts share one launch.
constexpr int kPrefillGroupMax = 256;
// ... of them joined sum sets (their member tables ride in the kernel
// arguments too)
constexpr int kMaxJoined = 16;
// The end of the prefill launch that starts at item c0: at most
// kPrefillGroupMax items, of them at most kMaxJoined joined sets.
inline int prefill_chunk_end(const LinearItem *items, int n, int c0) {
    int c1 = c0, joined = 0;
    while (c1 < n && c1 - c0 < kPrefillGroupMax && !(items[c1].cat > 1 && joined == kMaxJoined))
        joined += items[c1++].cat > 1 ? 1 : 0;
    return c1;
}

// A dense copy [M][ldo] of rows of X [x_rows][ldx] read through an index
// (out row m = X row ridx[m], zeros when that lies outside [0, x_rows);
// columns Ks .. ldo zero), for products whose kernels read X rows directly.
struct RowGather {
    const void *X;
    int64_t ldx;
    const int32_t *ridx;
    int64_t x_rows, M, Ks;
    void *out;
    int64_t ldo;
};
// All of them, bit for bit, elem_bytes 2 or 4 (rows 16-byte aligned).
hipError_t launch_row_gathers(const std::vector<RowGather> &jobs, size_t elem_bytes,
                              hipStream_t stream);

// ---- skinny.hip: decode-sized M (streams the weights once per 64 rows) ----
struct SkinnyPlan {
    bool stream = true; // bf16 / 4-bit: streaming kernel; fp32: k-split kernel
    int mt = 1;         // 16-row m-tiles per workgroup (1, 2 or 4)
    int ntw = 1;        // 16-column tiles per wave (1 or 2)
    int cmax = 16;      // fp32 kernel: max k-chunks per wave
    bool resident = false; // streaming kernel: whole k-range of X kept in LDS
    int xstr = 0;          // ... LDS bytes per activation row
    int xsum_off = 0;      // ... LDS offset of the 4-bit group sums
    size_t lds_bytes = 0;  // dynamic LDS per workgroup
    std::vector<int64_t> m_blocks; // per item: row blocks of 16 * mt
    // per item: workgroups across its columns, k-split across workgroups
    // (partials go to the workspace) and the byte offset of its partials
    std::vector<int64_t> n_groups;
    std::vector<int> ks;
    std::vector<size_t> ws_off;
    // sum sets the streaming launch adds up itself (members unsplit, all in
    // one launch): per item its set (index into fsets) or -1; per set its
    // first item and the workspace offset of its per-tile counters
    std::vector<int> fset;
    struct FSet {
        int first = 0, len = 0;
        size_t ctr_off = 0;
    };
    std::vector<FSet> fsets;
    size_t ws_bytes = 0;
};
SkinnyPlan skinny_plan(const LinearItem *items, int n, tsl_dtype wdtype, int64_t M);
// most workgroups any one launch of the group takes (bounded by the host)
int64_t skinny_blocks(const SkinnyPlan &p, const LinearItem *items, int n);
// Enqueues the group.  A product split along k (ks > 1) leaves its binary32
// k-partials [ks][M][Ns] at workspace + ws_off[i] for the caller's sum
// launch to add in k order, unless it accumulates into Y or is a member of
// a sum set longer than kSetParts (no_split): those are finished by a
// launch of their own.
hipError_t launch_skinny(const SkinnyPlan &p, const LinearItem *items, int n, tsl_dtype wdtype,
                         int64_t M, void *workspace, hipStream_t stream);

// ---- prefill.hip: 32x32x16 MFMA GEMM, operands copied straight into LDS ----
struct PrefillPlan {
    int bm = 256, bn = 160; // block tile
    int wm = 4, wn = 1;     // wave grid
    // per item: byte offset in the workspace of its activation copy
    // (binary16 for 4-bit shards, followed by its row exponents; zero-padded
    // bf16 when K is not a multiple of 64), and the item whose copy it reads
    // (itself for the first reader of an X; -1: no copy)
    std::vector<size_t> x_off;
    std::vector<int> x_first;
    // per item: k-splits (1: none) and the byte offset of its [ks][M][Ns]
    // binary32 k-partials, which a sum launch then adds in k order
    std::vector<int> ks;
    std::vector<size_t> p_off;
    size_t ws_bytes = 0;
};
bool prefill_supported(tsl_dtype wdtype);
PrefillPlan prefill_plan(const LinearItem *items, int n, tsl_dtype wdtype, int64_t M);
// most workgroups any one launch of the group takes (bounded by the host)
int64_t prefill_blocks(const PrefillPlan &p, const LinearItem *items, int n, int64_t M);
hipError_t launch_prefill(const PrefillPlan &p, const LinearItem *items, int n, tsl_dtype wdtype,
                          int64_t M, void *workspace, hipStream_t stream);

// ---- q4gemm.hip: the fused 4-bit GEMM (records expanded in registers) ----
// Enqueues the GEMM of every item (their binary16 activation copies at
// ws + p.x_off[i], already written by the activation pass).
hipError_t launch_q4_gemm(const PrefillPlan &p, const LinearItem *items, int n, const char *ws,
                          hipStream_t stream);

// Bound (elements, exclusive) on the activation row stride and padded K of
// the prefill path, which keeps its 32-bit operand offsets in range.
constexpr int64_t kPrefillMaxStride = int64_t(1) << 22;

// Rows at or below which shard_linear takes the skinny (decode) path: 64
// for 4-bit weights (whose GEMM regime is 2x slower at 4 and 16 rows);
// 32 for bf16 weights, whose GEMM (one 64-row tile per column tile, the
// weights streamed once) is faster from about 32 rows on (gqa8 layer,
// M = 32 / 64: 111 / 113 -> 97 / 101 us; llama2k M = 64: 38 -> 35 us;
// llama2k M = 16 / 24 stay faster streamed: 26 / 30 vs 34 / 36 us).
constexpr int64_t kSkinnyMaxM = 64;
constexpr int64_t kSkinnyMaxMBf16 = 32;

} // namespace tsl
