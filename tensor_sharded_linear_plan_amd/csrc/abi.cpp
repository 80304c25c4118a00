// The C ABI: host-side validation, packed-layout geometry and dispatch to
// the gfx950 kernels.  Every check runs before anything is enqueued, so a
// rejected call has no side effects.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"
#include "tsl.h"

namespace tsl {

namespace {

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool valid_dtype(int d) { return d == TSL_F32 || d == TSL_BF16 || d == TSL_Q4G64; }

// Shard descriptor sanity: the block lies inside W and matches its strategy.
tsl_status check_shard(const tsl_shard *s) {
    if (!s)
        return TSL_ERR_INVALID_ARG;
    if (s->K < 1 || s->N < 1 || s->k_len < 1 || s->n_len < 1 || s->k_off < 0 || s->n_off < 0)
        return TSL_ERR_INVALID_ARG;
    if (s->k_off + s->k_len > s->K || s->n_off + s->n_len > s->N)
        return TSL_ERR_INVALID_ARG;
    switch (s->strategy) {
    case TSL_COLUMN:
        if (s->k_off != 0 || s->k_len != s->K)
            return TSL_ERR_INVALID_ARG;
        break;
    case TSL_ROW:
        if (s->n_off != 0 || s->n_len != s->N)
            return TSL_ERR_INVALID_ARG;
        break;
    case TSL_REPLICATED:
        if (s->k_off != 0 || s->k_len != s->K || s->n_off != 0 || s->n_len != s->N)
            return TSL_ERR_INVALID_ARG;
        break;
    default:
        return TSL_ERR_INVALID_ARG;
    }
    return TSL_OK;
}

thread_local hipError_t g_last_hip = hipSuccess;

tsl_status from_hip(hipError_t e) {
    if (e == hipSuccess)
        return TSL_OK;
    g_last_hip = e;
    return TSL_ERR_HIP;
}

} // namespace

tsl_status geometry(const tsl_shard &s, tsl_dtype wdtype, PackGeom *g) {
    tsl_status st = check_shard(&s);
    if (st != TSL_OK)
        return st;
    if (!valid_dtype(wdtype))
        return TSL_ERR_INVALID_ARG;
    PackGeom r;
    r.Ks = s.k_len;
    r.Ns = s.n_len;
    r.Nt = (r.Ns + 15) / 16;
    const int64_t k64 = (r.Ks + 63) / 64;
    switch (wdtype) {
    case TSL_F32:
        r.KT = k64 * 4;
        r.Kpad = k64 * 64;
        r.total_bytes = (size_t)r.Nt * (size_t)r.KT * 64 * 16;
        break;
    case TSL_BF16:
        r.KT = k64 * 2;
        r.Kpad = k64 * 64;
        r.total_bytes = (size_t)r.Nt * (size_t)r.KT * 64 * 16;
        break;
    default: // TSL_Q4G64
        if (s.k_len % 64 || s.k_off % 64)
            return TSL_ERR_GROUP_ALIGN;
        r.KT = (r.Ks + 127) / 128;
        r.Kpad = r.KT * 128;
        r.codes_bytes = round_up((size_t)r.Nt * (size_t)r.KT * 64 * 16, 256);
        r.sb_bytes = round_up((size_t)r.Nt * (size_t)r.KT * 2 * 16 * 4, 256);
        r.total_bytes = r.codes_bytes + r.sb_bytes;
        break;
    }
    *g = r;
    return TSL_OK;
}

} // namespace tsl

using namespace tsl;

extern "C" tsl_status pack_shard_size(const tsl_shard *shard, tsl_dtype wdtype, size_t *bytes) {
    if (!shard || !bytes)
        return TSL_ERR_INVALID_ARG;
    PackGeom g;
    tsl_status st = geometry(*shard, wdtype, &g);
    if (st != TSL_OK)
        return st;
    *bytes = g.total_bytes;
    return TSL_OK;
}

extern "C" tsl_status pack_shard(const tsl_shard *shard, tsl_dtype wdtype, const void *W,
                                 int64_t stride_k, int64_t stride_n, const void *scales,
                                 const void *biases, int64_t sb_stride_g, int64_t sb_stride_n,
                                 void *packed, size_t packed_bytes, void *stream) {
    if (!shard || !W || !packed)
        return TSL_ERR_INVALID_ARG;
    PackGeom g;
    tsl_status st = geometry(*shard, wdtype, &g);
    if (st != TSL_OK)
        return st;
    if (stride_k < 0 || stride_n < 0)
        return TSL_ERR_INVALID_ARG;
    if (wdtype == TSL_Q4G64) {
        if (!scales || !biases || sb_stride_g < 0 || sb_stride_n < 0)
            return TSL_ERR_INVALID_ARG;
    } else if (scales || biases) {
        return TSL_ERR_INVALID_ARG;
    }
    if (packed_bytes < g.total_bytes)
        return TSL_ERR_BUFFER_TOO_SMALL;
    if (!aligned(packed, 256))
        return TSL_ERR_MISALIGNED;
    const size_t esz = wdtype == TSL_F32 ? 4 : (wdtype == TSL_BF16 ? 2 : 1);
    if (!aligned(W, esz) || (wdtype == TSL_Q4G64 && (!aligned(scales, 2) || !aligned(biases, 2))))
        return TSL_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (wdtype == TSL_Q4G64)
        e = launch_pack_q4(g, static_cast<const uint8_t *>(W), stride_k, stride_n,
                           static_cast<const uint16_t *>(scales),
                           static_cast<const uint16_t *>(biases), sb_stride_g, sb_stride_n,
                           shard->k_off, shard->n_off, packed, s);
    else
        e = launch_pack_dense(g, wdtype, W, stride_k, stride_n, shard->k_off, shard->n_off, packed,
                              s);
    return from_hip(e);
}

namespace {

// Which kernel family shard_linear uses for this call.
bool use_skinny(tsl_dtype wdtype, int64_t M) { return wdtype == TSL_F32 || M <= kSkinnyMaxM; }

} // namespace

extern "C" tsl_status shard_linear_workspace_size(const tsl_shard *shard, tsl_dtype wdtype,
                                                  int64_t M, size_t *bytes) {
    if (!shard || !bytes || M < 0)
        return TSL_ERR_INVALID_ARG;
    PackGeom g;
    tsl_status st = geometry(*shard, wdtype, &g);
    if (st != TSL_OK)
        return st;
    if (M == 0)
        *bytes = 0;
    else if (use_skinny(wdtype, M))
        *bytes = skinny_plan(g, wdtype, M).ws_bytes;
    else
        *bytes = prefill_workspace_bytes(g, wdtype);
    return TSL_OK;
}

extern "C" tsl_status shard_linear(const tsl_shard *shard, tsl_dtype wdtype, const void *packed,
                                   size_t packed_bytes, tsl_dtype xdtype, const void *X,
                                   int64_t ldx, int64_t M, tsl_dtype ydtype, void *Y, int64_t ldy,
                                   int accumulate, void *workspace, size_t ws_bytes,
                                   void *stream) {
    if (!shard || !packed || !X || !Y || M < 0)
        return TSL_ERR_INVALID_ARG;
    PackGeom g;
    tsl_status st = geometry(*shard, wdtype, &g);
    if (st != TSL_OK)
        return st;
    if (!valid_dtype(xdtype) || !valid_dtype(ydtype) || xdtype == TSL_Q4G64 || ydtype == TSL_Q4G64)
        return TSL_ERR_INVALID_ARG;
    if (accumulate != 0 && accumulate != 1)
        return TSL_ERR_INVALID_ARG;
    // (weights, activations) pairs the kernels implement
    const bool pair_ok = (wdtype == TSL_F32 && xdtype == TSL_F32) ||
                         (wdtype == TSL_BF16 && xdtype == TSL_BF16) ||
                         (wdtype == TSL_Q4G64 && xdtype == TSL_BF16);
    if (!pair_ok || (accumulate && ydtype != TSL_F32))
        return TSL_ERR_UNSUPPORTED;
    if (ldx < g.Ks || ldy < g.Ns)
        return TSL_ERR_INVALID_ARG;
    if (packed_bytes < g.total_bytes)
        return TSL_ERR_BUFFER_TOO_SMALL;
    const int64_t xa = xdtype == TSL_F32 ? 4 : 8;
    const uintptr_t ya = ydtype == TSL_F32 ? 4 : 2;
    if (!aligned(packed, 256) || !aligned(X, 16) || ldx % xa || !aligned(Y, ya))
        return TSL_ERR_MISALIGNED;
    if (M == 0)
        return TSL_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (use_skinny(wdtype, M)) {
        SkinnyPlan p = skinny_plan(g, wdtype, M);
        if (p.m_blocks > 65535 || p.n_groups > 0x7FFFFFFF)
            return TSL_ERR_UNSUPPORTED;
        if (p.ws_bytes > 0) {
            if (!workspace || ws_bytes < p.ws_bytes)
                return TSL_ERR_BUFFER_TOO_SMALL;
            if (!aligned(workspace, 256))
                return TSL_ERR_MISALIGNED;
        }
        return from_hip(launch_skinny(p, g, wdtype, packed, X, ldx, M, ydtype, Y, ldy, accumulate,
                                      workspace, s));
    }
    PrefillPlan p = prefill_plan(g, M);
    if (p.m_blocks * p.n_blocks > 0x7FFFFFFF)
        return TSL_ERR_UNSUPPORTED;
    const size_t need = prefill_workspace_bytes(g, wdtype);
    if (need > 0) {
        if (!workspace || ws_bytes < need)
            return TSL_ERR_BUFFER_TOO_SMALL;
        if (!aligned(workspace, 256))
            return TSL_ERR_MISALIGNED;
    }
    return from_hip(launch_prefill(p, g, wdtype, packed, X, ldx, M, ydtype, Y, ldy, accumulate,
                                   workspace, s));
}

extern "C" tsl_status combine_partials(tsl_combine mode, int32_t n_parts, const void *const *parts,
                                       tsl_dtype pdtype, int64_t M, int64_t n_each,
                                       int64_t ld_part, tsl_dtype ydtype, void *Y, int64_t ldy,
                                       void *stream) {
    if (!parts || !Y || n_parts < 1 || n_parts > kMaxParts || M < 0 || n_each < 0)
        return TSL_ERR_INVALID_ARG;
    for (int r = 0; r < n_parts; ++r)
        if (!parts[r])
            return TSL_ERR_INVALID_ARG;
    if (pdtype != TSL_F32 && pdtype != TSL_BF16)
        return TSL_ERR_INVALID_ARG;
    if (ydtype != TSL_F32 && ydtype != TSL_BF16)
        return TSL_ERR_INVALID_ARG;
    if (ld_part < n_each)
        return TSL_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == TSL_COMBINE_SUM) {
        if (pdtype != TSL_F32)
            return TSL_ERR_UNSUPPORTED;
        if (ldy < n_each)
            return TSL_ERR_INVALID_ARG;
        for (int r = 0; r < n_parts; ++r)
            if (!aligned(parts[r], 4))
                return TSL_ERR_MISALIGNED;
        if (!aligned(Y, ydtype == TSL_F32 ? 4 : 2))
            return TSL_ERR_MISALIGNED;
        if (M == 0 || n_each == 0)
            return TSL_OK;
        return from_hip(launch_combine_sum(n_parts, reinterpret_cast<const float *const *>(parts),
                                           M, n_each, ld_part, ydtype, Y, ldy, s));
    }
    if (mode == TSL_COMBINE_CONCAT) {
        if (pdtype != ydtype)
            return TSL_ERR_UNSUPPORTED;
        if (ldy < n_each * n_parts)
            return TSL_ERR_INVALID_ARG;
        const uintptr_t ea = pdtype == TSL_F32 ? 4 : 2;
        for (int r = 0; r < n_parts; ++r)
            if (!aligned(parts[r], ea))
                return TSL_ERR_MISALIGNED;
        if (!aligned(Y, ea))
            return TSL_ERR_MISALIGNED;
        if (M == 0 || n_each == 0)
            return TSL_OK;
        return from_hip(launch_combine_concat(n_parts, parts, ea, M, n_each, ld_part, Y, ldy, s));
    }
    return TSL_ERR_INVALID_ARG;
}

extern "C" const char *tsl_last_hip_error_string(void) { return hipGetErrorString(g_last_hip); }

extern "C" const char *tsl_status_string(tsl_status status) {
    switch (status) {
    case TSL_OK: return "ok";
    case TSL_ERR_INVALID_ARG: return "invalid argument";
    case TSL_ERR_NOT_DIVISIBLE: return "dimension does not split evenly across ranks";
    case TSL_ERR_TP_NOT_POW2: return "tp_size is not a power of two";
    case TSL_ERR_GROUP_ALIGN: return "4-bit group straddles a shard edge";
    case TSL_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case TSL_ERR_UNSUPPORTED: return "unsupported dtype combination or size";
    case TSL_ERR_MISALIGNED: return "misaligned pointer or leading dimension";
    case TSL_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}
