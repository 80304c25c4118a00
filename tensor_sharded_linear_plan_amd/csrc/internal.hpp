// Internal interface between the C-ABI layer (abi.cpp) and the HIP kernel
// translation units.  Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tsl.h"

namespace tsl {

// Packed-layout geometry of one shard (see pack_shard_size in tsl.h).
struct PackGeom {
    int64_t Ks = 0, Ns = 0; // shard rows (input dim) and columns (output dim)
    int64_t Nt = 0;         // 16-column tiles
    int64_t Kpad = 0;       // Ks rounded up to the k granularity of the layout
    // F32: 16-k tiles; BF16: 32-k tiles; Q4G64: 128-k blocks
    int64_t KT = 0;
    size_t codes_bytes = 0; // Q4G64: bytes of the code region (256-byte rounded)
    size_t sb_bytes = 0;    // Q4G64: bytes of the scale/bias region
    size_t total_bytes = 0;
};

tsl_status geometry(const tsl_shard &s, tsl_dtype wdtype, PackGeom *g);

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
// Y (+)= sum_{s < ks} P[s], P is [ks][M][N] f32 contiguous, ascending s.
hipError_t launch_splitk_reduce(const float *P, int ks, int64_t M, int64_t N, tsl_dtype ydtype,
                                void *Y, int64_t ldy, int accumulate, hipStream_t stream);

// ---- skinny.hip: decode-sized M (streams the weights once per 64 rows) ----
struct SkinnyPlan {
    int mt = 1;      // 16-row m-tiles per workgroup (1, 2 or 4)
    int ntw = 1;     // 16-column n-tiles per wave (1, 2 or 4)
    int ks = 1;      // k-split across workgroups (partials go to the workspace)
    int cmax = 8;    // max k-chunks per wave (compile-time register budget)
    int64_t n_groups = 0, m_blocks = 0;
    size_t ws_bytes = 0;
};
SkinnyPlan skinny_plan(const PackGeom &g, tsl_dtype wdtype, int64_t M);
hipError_t launch_skinny(const SkinnyPlan &p, const PackGeom &g, tsl_dtype wdtype,
                         const void *packed, const void *X, int64_t ldx, int64_t M,
                         tsl_dtype ydtype, void *Y, int64_t ldy, int accumulate, void *workspace,
                         hipStream_t stream);

// ---- prefill.hip: 32x32x16 MFMA GEMM with LDS-staged tiles ----
struct PrefillPlan {
    int bm = 256, bn = 256; // block tile
    int wm = 2, wn = 2;     // wave grid
    int64_t m_blocks = 0, n_blocks = 0;
};
bool prefill_supported(tsl_dtype wdtype);
PrefillPlan prefill_plan(const PackGeom &g, int64_t M);
// workspace the prefill path needs (4-bit weights expanded to binary16)
size_t prefill_workspace_bytes(const PackGeom &g, tsl_dtype wdtype);
hipError_t launch_prefill(const PrefillPlan &p, const PackGeom &g, tsl_dtype wdtype,
                          const void *packed, const void *X, int64_t ldx, int64_t M,
                          tsl_dtype ydtype, void *Y, int64_t ldy, int accumulate, void *workspace,
                          hipStream_t stream);

// Rows at or below which shard_linear takes the skinny (decode) path.
constexpr int64_t kSkinnyMaxM = 64;

} // namespace tsl
