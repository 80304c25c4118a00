// The C ABI: host-side validation, packed-layout geometry and dispatch to
// the gfx950 kernels.  Every check runs before anything is enqueued, so a
// rejected call has no side effects.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <vector>

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
    case TSL_EXPERT:
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
        r.exp_off = round_up((size_t)r.Nt * (size_t)r.KT * kQ4Record, 256);
        r.total_bytes = r.exp_off + round_up((size_t)r.Nt * 16 * 4, 256);
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

// the item table's layout is part of the ABI
static_assert(sizeof(tsl_linear_item) == 88 && offsetof(tsl_linear_item, rows) == 68 &&
                  offsetof(tsl_linear_item, row_index) == 72 &&
                  offsetof(tsl_linear_item, x_rows) == 80,
              "tsl_linear_item layout");

namespace {

// Which kernel family serves a product of M rows.
bool use_skinny(tsl_dtype wdtype, int64_t M) {
    return wdtype == TSL_F32 || M <= (wdtype == TSL_BF16 ? kSkinnyMaxMBf16 : kSkinnyMaxM);
}

// Most items one grouped call takes.
constexpr int32_t kMaxItems = 4096;
// Workgroups per launch: the dispatch grid counts work-items in 32 bits.
constexpr int64_t kMaxBlocks = (int64_t(1) << 24) - 1;

tsl_status check_types(tsl_dtype wdtype, tsl_dtype xdtype) {
    if (!valid_dtype(wdtype) || !valid_dtype(xdtype) || xdtype == TSL_Q4G64)
        return TSL_ERR_INVALID_ARG;
    // (weights, activations) pairs the kernels implement
    const bool pair_ok = (wdtype == TSL_F32 && xdtype == TSL_F32) ||
                         (wdtype == TSL_BF16 && xdtype == TSL_BF16) ||
                         (wdtype == TSL_Q4G64 && xdtype == TSL_BF16);
    return pair_ok ? TSL_OK : TSL_ERR_UNSUPPORTED;
}

// Validates one shard product (weight and activation types already
// checked) and fills its item.
// A member of a sum set after its first item has no output of its own
// (need_y false): its Y fields are not checked.
tsl_status check_item(const tsl_shard *shard, tsl_dtype wdtype, const void *packed,
                      size_t packed_bytes, tsl_dtype xdtype, const void *X, int64_t ldx, int64_t M,
                      int ydtype, void *Y, int64_t ldy, int accumulate, LinearItem *out,
                      bool need_y = true) {
    if (!need_y) {
        Y = reinterpret_cast<void *>(uintptr_t(256));
        ydtype = TSL_F32;
        accumulate = 0;
        ldy = INT64_MAX;
    }
    if (!shard || !packed || !X || !Y)
        return TSL_ERR_INVALID_ARG;
    if (ydtype != TSL_F32 && ydtype != TSL_BF16)
        return TSL_ERR_INVALID_ARG;
    PackGeom g;
    tsl_status st = geometry(*shard, wdtype, &g);
    if (st != TSL_OK)
        return st;
    if (accumulate != 0 && accumulate != 1)
        return TSL_ERR_INVALID_ARG;
    if (accumulate && ydtype != TSL_F32)
        return TSL_ERR_UNSUPPORTED;
    if (ldx < g.Ks || ldy < g.Ns)
        return TSL_ERR_INVALID_ARG;
    if (packed_bytes < g.total_bytes)
        return TSL_ERR_BUFFER_TOO_SMALL;
    const int64_t xa = xdtype == TSL_F32 ? 4 : 8;
    const uintptr_t ya = ydtype == TSL_F32 ? 4 : 2;
    if (!aligned(packed, 256) || !aligned(X, 16) || ldx % xa || !aligned(Y, ya))
        return TSL_ERR_MISALIGNED;
    // the kernels' item tables hold shard sizes in 32 bits, and the GEMM
    // addresses a tile's operands with 32-bit offsets
    if (g.Kpad >= INT32_MAX || g.Ns >= INT32_MAX)
        return TSL_ERR_UNSUPPORTED;
    if (!use_skinny(wdtype, M) && (ldx >= kPrefillMaxStride || g.Kpad >= kPrefillMaxStride))
        return TSL_ERR_UNSUPPORTED;
    out->g = g;
    out->M = M;
    out->packed = packed;
    out->X = X;
    out->ldx = ldx;
    out->Y = Y;
    out->ldy = ldy;
    out->ydtype = (tsl_dtype)ydtype;
    out->accumulate = accumulate;
    if (!need_y) {
        out->Y = nullptr;
        out->ldy = 0;
    }
    return TSL_OK;
}

// Launch order of a group: longest k first, so the longest tiles are
// dispatched first and the short ones fill in at the end.
std::vector<LinearItem> launch_order(const std::vector<LinearItem> &items) {
    // sum sets move as units (first item, then its members in order)
    struct Unit {
        size_t first, len;
        int64_t kpad;
    };
    std::vector<Unit> units;
    for (size_t i = 0; i < items.size(); i += items[i].set_len) {
        Unit u{i, (size_t)items[i].set_len, 0};
        for (size_t r = 0; r < u.len; ++r)
            u.kpad = items[i + r].g.Kpad > u.kpad ? items[i + r].g.Kpad : u.kpad;
        units.push_back(u);
    }
    std::stable_sort(units.begin(), units.end(),
                     [](const Unit &a, const Unit &b) { return a.kpad > b.kpad; });
    std::vector<LinearItem> v;
    v.reserve(items.size());
    for (const Unit &u : units)
        for (size_t r = 0; r < u.len; ++r)
            v.push_back(items[u.first + r]);
    return v;
}

// The GEMM regime: a sum set whose members have equal k-ranges becomes one
// product over the members' k-ranges laid end to end in set order,
// Y = [X_0 X_1 ...] [W_0; W_1; ...] -- the rank sum accumulated inside the
// GEMM, with no binary32 partials and no sum launch.  4-bit weights: k-
// ranges of whole 128-k records (the activation pass writes each member's
// binary16 activations at its k offset of the joined row, and the GEMM
// reads each 128-k block's records from its member's packed buffer).
// bf16 weights: k-ranges of whole 64-k stages, activations not read through
// a row index (the GEMM reads each stage's activations, at their member's
// row stride, and weights from the member's own buffers).  The rule reads
// nothing the workspace query does not see.  Other sets, and every set of
// fp32 weights or of the decode regime, pass unchanged.
std::vector<LinearItem> concat_sets(const std::vector<LinearItem> &in, tsl_dtype wdtype,
                                    int64_t M) {
    if ((wdtype != TSL_Q4G64 && wdtype != TSL_BF16) || use_skinny(wdtype, M))
        return in;
    const int64_t unit = wdtype == TSL_Q4G64 ? 128 : 64;
    std::vector<LinearItem> out;
    out.reserve(in.size());
    for (size_t i = 0; i < in.size();) {
        const size_t len = in[i].set_len;
        bool join = len > 1 && len <= (size_t)kSetParts &&
                    (int64_t)len * in[i].g.Kpad < kPrefillMaxStride;
        for (size_t r = 0; join && r < len; ++r)
            join = in[i + r].g.Ks % unit == 0 && in[i + r].g.Ks == in[i].g.Ks &&
                   (wdtype == TSL_Q4G64 || !in[i + r].ridx);
        if (!join) {
            for (size_t r = 0; r < len; ++r)
                out.push_back(in[i + r]);
            i += len;
            continue;
        }
        LinearItem c = in[i];
        c.cat = (int)len;
        c.set_len = 1;
        c.set_pos = 0;
        c.g.Ks *= (int64_t)len;
        c.g.KT *= (int64_t)len;
        c.g.Kpad *= (int64_t)len;
        c.g.total_bytes = 0; // no packed buffer of its own
        c.packed = nullptr;
        c.X = nullptr; // never shares an activation copy
        c.ldx = 0;
        c.ridx = nullptr;
        c.x_rows = 0;
        for (size_t r = 0; r < len; ++r) {
            c.seg_packed[r] = in[i + r].packed;
            c.seg_X[r] = in[i + r].X;
            c.seg_ldx[r] = in[i + r].ldx;
            c.seg_ridx[r] = in[i + r].ridx;
            c.seg_xrows[r] = in[i + r].x_rows;
        }
        out.push_back(c);
        i += len;
    }
    return out;
}

// Sum sets: each member of a set runs into its own binary32 partial (in
// the workspace, ahead of what the plan needs), balanced with every other
// product of the group; one more launch then adds the partials of all sets
// in order.

// Rewrites every sum set of *items into lone items writing binary32
// partials at ws, ws + ...; returns the bytes used.  Call it once: the
// items it leaves are no longer sets.  With ws == nullptr the partials'
// addresses are null (for sizing; such items are never launched).
size_t split_sets(std::vector<LinearItem> *items, int64_t M, char *ws) {
    size_t off = 0;
    for (size_t i = 0; i < items->size();) {
        const size_t len = (*items)[i].set_len;
        if (len > 1) {
            void *const sY = (*items)[i].Y;
            const int64_t sldy = (*items)[i].ldy;
            const tsl_dtype sy = (*items)[i].ydtype;
            for (size_t r = 0; r < len; ++r) {
                LinearItem &L = (*items)[i + r];
                L.fset_len = (int)len;
                L.fset_pos = (int)r;
                L.fset_Y = sY;
                L.fset_ldy = sldy;
                L.fset_ydtype = sy;
                L.Y = ws ? ws + off : nullptr;
                L.ldy = L.g.Ns;
                L.ydtype = TSL_F32;
                L.accumulate = 0;
                L.set_len = 1;
                L.set_pos = 0;
                L.no_split = len > (size_t)kSetParts; // summed by launch_combine_sum

                off += ((size_t)L.M * (size_t)L.g.Ns * 4 + 255) / 256 * 256;
            }
        }
        i += len;
    }
    return off;
}

size_t span(int64_t M, int64_t n, int64_t ld, size_t elem);
bool overlaps(const void *a, size_t na, const void *b, size_t nb);

// Whether an [Ma][wa] and an [Mb][wb] row-strided matrix share a byte
// (Ma, Mb > 0).  With equal strides this is exact -- column blocks or row
// blocks of one matrix held by different owners do not overlap -- otherwise
// it compares address ranges.
bool matrices_overlap(const void *pa, int64_t Ma, int64_t wa, int64_t lda, size_t ea,
                      const void *pb, int64_t Mb, int64_t wb, int64_t ldb, size_t eb) {
    const int64_t L = lda * (int64_t)ea;
    const int64_t Wa = wa * (int64_t)ea, Wb = wb * (int64_t)eb;
    if (L != ldb * (int64_t)eb || Wa > L || Wb > L)
        return overlaps(pa, span(Ma, wa, lda, ea), pb, span(Mb, wb, ldb, eb));
    // b - a = q L + rem, 0 <= rem < L: rows r1 - r2 = q need rem < Wa, rows
    // r1 - r2 = q + 1 need L - rem < Wb, each with -Mb < r1 - r2 < Ma
    const int64_t d = (int64_t)(reinterpret_cast<uintptr_t>(pb) - reinterpret_cast<uintptr_t>(pa));
    int64_t q = d / L, rem = d % L;
    if (rem < 0) {
        rem += L;
        q -= 1;
    }
    const bool same_row = (q > -Mb && q < Ma) && rem < Wa;
    const bool next_row = (q + 1 > -Mb && q + 1 < Ma) && L - rem < Wb;
    return same_row || next_row;
}

// Rows read through an index.  The 4-bit activation pass (GEMM regime) and
// the resident streaming kernel (a few decode rows, bf16 and 4-bit
// weights) read them where they lie; the other kernels read X rows at
// fixed strides, so for them each distinct (X, ldx, k_len, row index,
// rows) is first gathered into a dense copy at the front of the workspace
// (all of a call's gathers in one launch), and the items read the copy.
// Rewrites the indexed items of *items that need a gathered copy to read
// it (ws + ...; null ws: sizing, every item its own copy) and returns the
// bytes the copies take; *jobs receives the gathers to enqueue.
size_t plan_row_gathers(std::vector<LinearItem> *items, tsl_dtype wdtype, int64_t M, char *ws,
                        std::vector<RowGather> *jobs) {
    // the 4-bit activation pass reads through the index itself, and so do
    // the streaming kernels that hold a call's rows in LDS (a few rows: the
    // plan's resident calls, decided by the items' shapes alone)
    if (wdtype == TSL_Q4G64 && !use_skinny(wdtype, M))
        return 0;
    if (wdtype != TSL_F32 && use_skinny(wdtype, M) &&
        skinny_plan(items->data(), (int)items->size(), wdtype, M).resident)
        return 0;
    const size_t e = wdtype == TSL_F32 ? 4 : 2;
    const int64_t xa = wdtype == TSL_F32 ? 4 : 8; // row strides of 16 bytes
    size_t off = 0;
    for (LinearItem &L : *items) {
        if (!L.ridx)
            continue;
        const int64_t Kc = (L.g.Ks + xa - 1) / xa * xa;
        const RowGather *same = nullptr;
        for (const RowGather &j : *jobs)
            if (ws && j.X == L.X && j.ldx == L.ldx && j.ridx == L.ridx && j.x_rows == L.x_rows &&
                j.M == L.M && j.Ks == L.g.Ks)
                same = &j;
        if (!same) {
            jobs->push_back(RowGather{L.X, L.ldx, L.ridx, L.x_rows, L.M, L.g.Ks,
                                      ws ? ws + off : nullptr, Kc});
            off += ((size_t)L.M * (size_t)Kc * e + 255) / 256 * 256;
            same = &jobs->back();
        }
        L.X = same->out;
        L.ldx = Kc;
        L.ridx = nullptr;
        L.x_rows = 0;
    }
    return off;
}

// Workspace bytes of a validated group.
size_t group_workspace(const std::vector<LinearItem> &in, tsl_dtype wdtype, int64_t M) {
    if (M == 0 || in.empty())
        return 0;
    std::vector<LinearItem> src = in;
    std::vector<RowGather> jobs;
    const size_t gathered = plan_row_gathers(&src, wdtype, M, nullptr, &jobs);
    std::vector<LinearItem> items = launch_order(concat_sets(src, wdtype, M));
    const size_t parts = split_sets(&items, M, nullptr);
    if (use_skinny(wdtype, M))
        return gathered + parts + skinny_plan(items.data(), (int)items.size(), wdtype, M).ws_bytes;
    return gathered + parts + prefill_plan(items.data(), (int)items.size(), wdtype, M).ws_bytes;
}

// Plans and enqueues a validated group.
tsl_status run_group(const std::vector<LinearItem> &in, tsl_dtype wdtype, int64_t M,
                     void *workspace, size_t ws_bytes, void *stream) {
    if (M == 0)
        return TSL_OK;
    // (a null or short workspace is rejected below, before any launch)
    char *const ws0 = static_cast<char *>(workspace);
    std::vector<LinearItem> src = in;
    std::vector<RowGather> gathers;
    const size_t gathered = plan_row_gathers(&src, wdtype, M, ws0, &gathers);
    char *ws = ws0 ? ws0 + gathered : nullptr; // the rank partials, then the plan's
    const std::vector<LinearItem> ordered = launch_order(concat_sets(src, wdtype, M));
    std::vector<LinearItem> items = ordered;
    const size_t parts = split_sets(&items, M, ws);
    const int n = (int)items.size();
    hipStream_t s = static_cast<hipStream_t>(stream);
    size_t need;
    int64_t blocks;
    SkinnyPlan sp;
    PrefillPlan pp;
    const bool skinny = use_skinny(wdtype, M);
    if (skinny) {
        sp = skinny_plan(items.data(), n, wdtype, M);
        need = gathered + parts + sp.ws_bytes;
        blocks = skinny_blocks(sp, items.data(), n);
    } else {
        pp = prefill_plan(items.data(), n, wdtype, M);
        need = gathered + parts + pp.ws_bytes;
        blocks = prefill_blocks(pp, items.data(), n, M);
    }
    if (blocks > kMaxBlocks)
        return TSL_ERR_UNSUPPORTED;
    if (need > 0) {
        if (!workspace || ws_bytes < need)
            return TSL_ERR_BUFFER_TOO_SMALL;
        if (!aligned(workspace, 256))
            return TSL_ERR_MISALIGNED;
    }
    // every product that is launched writes somewhere
    for (const LinearItem &L : items)
        if (!L.Y)
            return TSL_ERR_INVALID_ARG;
    // the rows read through an index, gathered (an index outside [0, x_rows)
    // gives a row of zeros)
    if (!gathers.empty()) {
        const hipError_t ge = launch_row_gathers(gathers, wdtype == TSL_F32 ? 4 : 2, s);
        if (ge != hipSuccess)
            return from_hip(ge);
    }
    hipError_t e = skinny ? launch_skinny(sp, items.data(), n, wdtype, M, ws + parts, s)
                          : launch_prefill(pp, items.data(), n, wdtype, M, ws + parts, s);
    if (e != hipSuccess)
        return from_hip(e);
    // k-split GEMM products: each product's k-partials, in k order
    // k-split products (decode regime: those that neither accumulate into
    // Y nor belong to a sum set too long for one sum launch; launch_skinny
    // finished the others)
    auto kcount = [&](size_t i) {
        return !skinny ? pp.ks[i]
                       : (items[i].accumulate || items[i].no_split ? 1 : sp.ks[i]);
    };
    auto kparts = [&](size_t i) {
        return kcount(i) > 1 ? reinterpret_cast<const float *>(
                                   ws + parts + (skinny ? sp.ws_off[i] : pp.p_off[i]))
                             : static_cast<const float *>(items[i].Y);
    };
    std::vector<SumSpec> sums;
    for (size_t i = 0; i < ordered.size();) {
        const size_t len = ordered[i].set_len;
        if (len == 1 && kcount(i) > 1) { // a lone product: its k-partials into its Y
            SumSpec sp1;
            sp1.parts[0] = kparts(i);
            sp1.ks[0] = kcount(i);
            sp1.n_parts = 1;
            sp1.M = items[i].M;
            sp1.n = items[i].g.Ns;
            sp1.Y = items[i].Y;
            sp1.ldy = items[i].ldy;
            sp1.ydtype = items[i].ydtype;
            sums.push_back(sp1);
        }
        i += len;
    }
    if (!parts) {
        if (!sums.empty())
            e = launch_sum_sets((int)sums.size(), sums.data(), M, s);
        return from_hip(e);
    }
    // the rank sums of the split sets, in item order: sets of up to
    // kSetParts members share one launch, longer ones get their own
    for (size_t i = 0; i < ordered.size(); i += ordered[i].set_len) {
        const LinearItem &L = ordered[i];
        if (L.set_len == 1)
            continue;
        if (skinny && sp.fset[i] >= 0)
            continue; // added up by the streaming launch itself
        if (L.set_len > kSetParts) {
            const float *p[kMaxParts];
            for (int r = 0; r < L.set_len; ++r)
                p[r] = static_cast<const float *>(items[i + r].Y);
            e = launch_combine_sum(L.set_len, p, L.M, L.g.Ns, L.g.Ns, L.ydtype, L.Y, L.ldy, s);
            if (e != hipSuccess)
                return from_hip(e);
            continue;
        }
        SumSpec sp;
        for (int r = 0; r < L.set_len; ++r) {
            sp.parts[r] = kparts(i + r);
            sp.ks[r] = kcount(i + r);
        }
        sp.n_parts = L.set_len;
        sp.M = L.M;
        sp.n = L.g.Ns;
        sp.Y = L.Y;
        sp.ldy = L.ldy;
        sp.ydtype = L.ydtype;
        sums.push_back(sp);
    }
    if (!sums.empty())
        e = launch_sum_sets((int)sums.size(), sums.data(), M, s);
    return from_hip(e);
}

// Gathers and validates the items of a grouped call.
tsl_status gather(int32_t n_items, const tsl_linear_item *items, tsl_dtype wdtype,
                  tsl_dtype xdtype, int64_t M, std::vector<LinearItem> *out) {
    if (!items || n_items < 1 || n_items > kMaxItems || M < 0)
        return TSL_ERR_INVALID_ARG;
    tsl_status st = check_types(wdtype, xdtype);
    if (st != TSL_OK)
        return st;
    out->resize(n_items);
    int32_t first = 0; // first item of the current sum set
    for (int32_t i = 0; i < n_items; ++i) {
        const tsl_linear_item &it = items[i];
        const bool member = i > first;
        if ((it.sum_next != 0 && it.sum_next != 1) || it.rows < 0 || it.rows > M)
            return TSL_ERR_INVALID_ARG;
        if (it.sum_next && i == n_items - 1)
            return TSL_ERR_INVALID_ARG;
        st = check_item(it.shard, wdtype, it.packed, it.packed_bytes, xdtype, it.X, it.ldx, M,
                        it.ydtype, it.Y, it.ldy, it.accumulate, &(*out)[i], !member);
        if (st != TSL_OK)
            return st;
        LinearItem &L = (*out)[i];
        L.set_pos = i - first;
        L.M = it.rows ? it.rows : M;
        if (it.row_index) { // rows read through an index
            if (it.x_rows < 1 || it.x_rows > INT32_MAX)
                return TSL_ERR_INVALID_ARG;
            if (!aligned(it.row_index, 4))
                return TSL_ERR_MISALIGNED;
            L.ridx = it.row_index;
            L.x_rows = it.x_rows;
        }
        if (member && (L.g.Ns != (*out)[first].g.Ns || L.M != (*out)[first].M))
            return TSL_ERR_INVALID_ARG;
        if (!it.sum_next) { // the set [first, i] is complete
            (*out)[first].set_len = i - first + 1;
            if (i > first && (*out)[first].accumulate)
                return TSL_ERR_INVALID_ARG;
            if (i - first + 1 > kMaxParts)
                return TSL_ERR_INVALID_ARG;
            for (int32_t r = first + 1; r <= i; ++r)
                (*out)[r].set_len = 0;
            first = i + 1;
        }
    }
    if (M == 0)
        return TSL_OK;
    // the products run in no particular order: no output may overlap
    // another output or any input
    const size_t xe = xdtype == TSL_F32 ? 4 : 2;
    for (int32_t i = 0; i < n_items; ++i) {
        const LinearItem &a = (*out)[i];
        if (!a.Y)
            continue; // a sum-set member writes into its set's output
        const size_t ea = a.ydtype == TSL_F32 ? 4 : 2;
        for (int32_t j = 0; j < n_items; ++j) {
            const LinearItem &b = (*out)[j];
            const size_t eb = b.ydtype == TSL_F32 ? 4 : 2;
            if (matrices_overlap(a.Y, a.M, a.g.Ns, a.ldy, ea, b.X, b.ridx ? b.x_rows : b.M, b.g.Ks,
                                 b.ldx, xe))
                return TSL_ERR_INVALID_ARG;
            if (b.ridx && overlaps(a.Y, span(a.M, a.g.Ns, a.ldy, ea), b.ridx, (size_t)b.M * 4))
                return TSL_ERR_INVALID_ARG;
            if (j > i && b.Y &&
                matrices_overlap(a.Y, a.M, a.g.Ns, a.ldy, ea, b.Y, b.M, b.g.Ns, b.ldy, eb))
                return TSL_ERR_INVALID_ARG;
        }
    }
    return TSL_OK;
}

} // namespace

extern "C" tsl_status shard_linear_workspace_size(const tsl_shard *shard, tsl_dtype wdtype,
                                                  int64_t M, size_t *bytes) {
    if (!shard || !bytes || M < 0)
        return TSL_ERR_INVALID_ARG;
    std::vector<LinearItem> items(1);
    tsl_status st = geometry(*shard, wdtype, &items[0].g);
    if (st != TSL_OK)
        return st;
    items[0].M = M;
    *bytes = group_workspace(items, wdtype, M);
    return TSL_OK;
}

extern "C" tsl_status shard_linear(const tsl_shard *shard, tsl_dtype wdtype, const void *packed,
                                   size_t packed_bytes, tsl_dtype xdtype, const void *X,
                                   int64_t ldx, int64_t M, tsl_dtype ydtype, void *Y, int64_t ldy,
                                   int accumulate, void *workspace, size_t ws_bytes,
                                   void *stream) {
    if (M < 0)
        return TSL_ERR_INVALID_ARG;
    tsl_status st = check_types(wdtype, xdtype);
    if (st != TSL_OK)
        return shard && packed && X && Y ? st : TSL_ERR_INVALID_ARG;
    std::vector<LinearItem> items(1);
    st = check_item(shard, wdtype, packed, packed_bytes, xdtype, X, ldx, M, ydtype, Y, ldy,
                    accumulate, &items[0]);
    if (st != TSL_OK)
        return st;
    return run_group(items, wdtype, M, workspace, ws_bytes, stream);
}

extern "C" tsl_status shard_linear_group_workspace_size(int32_t n_items,
                                                        const tsl_linear_item *items,
                                                        tsl_dtype wdtype, int64_t M,
                                                        size_t *bytes) {
    if (!items || !bytes || n_items < 1 || n_items > kMaxItems || M < 0)
        return TSL_ERR_INVALID_ARG;
    std::vector<LinearItem> v(n_items);
    int32_t first = 0;
    for (int32_t i = 0; i < n_items; ++i) {
        if (!items[i].shard || (items[i].sum_next != 0 && items[i].sum_next != 1) ||
            items[i].rows < 0 || items[i].rows > M)
            return TSL_ERR_INVALID_ARG;
        tsl_status st = geometry(*items[i].shard, wdtype, &v[i].g);
        if (st != TSL_OK)
            return st;
        v[i].M = items[i].rows ? items[i].rows : M;
        v[i].ridx = items[i].row_index; // only whether it is null matters here
        v[i].x_rows = 1;
        v[i].set_pos = i - first;
        if (!items[i].sum_next || i == n_items - 1) {
            v[first].set_len = i - first + 1;
            for (int32_t r = first + 1; r <= i; ++r)
                v[r].set_len = 0;
            first = i + 1;
        }
    }
    *bytes = group_workspace(v, wdtype, M);
    return TSL_OK;
}

extern "C" tsl_status shard_linear_group(int32_t n_items, const tsl_linear_item *items,
                                         tsl_dtype wdtype, tsl_dtype xdtype, int64_t M,
                                         void *workspace, size_t ws_bytes, void *stream) {
    std::vector<LinearItem> v;
    tsl_status st = gather(n_items, items, wdtype, xdtype, M, &v);
    if (st != TSL_OK)
        return st;
    return run_group(v, wdtype, M, workspace, ws_bytes, stream);
}

extern "C" tsl_status shard_linear_group_noalloc(int32_t n_items, const tsl_linear_item *items,
                                                 tsl_dtype wdtype, tsl_dtype xdtype, int64_t M,
                                                 void *stream) {
    std::vector<LinearItem> v;
    tsl_status st = gather(n_items, items, wdtype, xdtype, M, &v);
    if (st != TSL_OK)
        return st;
    // the exact workspace of this call (its items carry their X pointers, so
    // shared activation copies are counted once), checked before any device
    // call
    const size_t need = group_workspace(v, wdtype, M);
    if (need > kNoAllocScratchBytes)
        return TSL_ERR_BUFFER_TOO_SMALL;
    void *scr = nullptr;
    if (need > 0) {
        hipError_t e = noalloc_scratch(&scr);
        if (e != hipSuccess)
            return from_hip(e);
    }
    return run_group(v, wdtype, M, scr, need > 0 ? kNoAllocScratchBytes : 0, stream);
}

namespace {

// Bytes from the first to one past the last element of an [M][n] matrix
// with row stride ld (M, n > 0).
size_t span(int64_t M, int64_t n, int64_t ld, size_t elem) {
    return (size_t)((M - 1) * ld + n) * elem;
}


bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

} // namespace

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
        const size_t ye = ydtype == TSL_F32 ? 4 : 2;
        for (int r = 0; r < n_parts; ++r) {
            const bool in_place =
                r == 0 && parts[0] == Y && ydtype == TSL_F32 && ldy == ld_part;
            if (!in_place && overlaps(parts[r], span(M, n_each, ld_part, 4), Y,
                                      span(M, n_each, ldy, ye)))
                return TSL_ERR_INVALID_ARG;
        }
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
        for (int r = 0; r < n_parts; ++r)
            if (overlaps(parts[r], span(M, n_each, ld_part, ea), Y,
                         span(M, n_each * n_parts, ldy, ea)))
                return TSL_ERR_INVALID_ARG;
        return from_hip(launch_combine_concat(n_parts, parts, ea, M, n_each, ld_part, Y, ldy, s));
    }
    return TSL_ERR_INVALID_ARG;
}

extern "C" tsl_status combine_to_ranks(tsl_collective op, int32_t n, const void *const *parts,
                                       tsl_dtype pdtype, int64_t M, int64_t n_each,
                                       int64_t ld_part, tsl_dtype odtype, void *const *outs,
                                       int64_t ldo, void *stream) {
    if (!parts || !outs || n < 1 || n > kMaxParts || M < 0 || n_each < 0 || ld_part < n_each)
        return TSL_ERR_INVALID_ARG;
    if (op != TSL_ALL_REDUCE && op != TSL_REDUCE_SCATTER && op != TSL_ALL_GATHER)
        return TSL_ERR_INVALID_ARG;
    if ((pdtype != TSL_F32 && pdtype != TSL_BF16) || (odtype != TSL_F32 && odtype != TSL_BF16))
        return TSL_ERR_INVALID_ARG;
    for (int r = 0; r < n; ++r)
        if (!parts[r] || !outs[r])
            return TSL_ERR_INVALID_ARG;
    const bool gather = op == TSL_ALL_GATHER;
    if (gather ? pdtype != odtype : pdtype != TSL_F32)
        return TSL_ERR_UNSUPPORTED;
    const int64_t width = gather ? n_each * n : n_each; // columns of each output
    if (ldo < width)
        return TSL_ERR_INVALID_ARG;
    const size_t pe = pdtype == TSL_F32 ? 4 : 2, oe = odtype == TSL_F32 ? 4 : 2;
    for (int r = 0; r < n; ++r)
        if (!aligned(parts[r], pe) || !aligned(outs[r], oe))
            return TSL_ERR_MISALIGNED;
    if (M == 0 || n_each == 0)
        return TSL_OK;
    // rows of rank r's output
    auto rows = [&](int r) {
        return op == TSL_REDUCE_SCATTER ? ((int64_t)(r + 1) * M) / n - ((int64_t)r * M) / n : M;
    };
    for (int r = 0; r < n; ++r) {
        if (rows(r) == 0)
            continue;
        for (int q = 0; q < n; ++q) {
            if (matrices_overlap(outs[r], rows(r), width, ldo, oe, parts[q], M, n_each, ld_part,
                                 pe))
                return TSL_ERR_INVALID_ARG;
            if (q > r && rows(q) > 0 &&
                matrices_overlap(outs[r], rows(r), width, ldo, oe, outs[q], rows(q), width, ldo,
                                 oe))
                return TSL_ERR_INVALID_ARG;
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gather)
        return from_hip(launch_gather_to_ranks(n, parts, pe, M, n_each, ld_part, outs, ldo, s));
    return from_hip(launch_reduce_to_ranks(n, reinterpret_cast<const float *const *>(parts), M,
                                           n_each, ld_part, op == TSL_REDUCE_SCATTER, odtype, outs,
                                           ldo, s));
}

extern "C" tsl_status embed_lookup(const tsl_shard *shard, tsl_dtype tdtype, const void *table,
                                   int64_t ld_table, const int32_t *tokens, int64_t M,
                                   tsl_dtype ydtype, void *Y, int64_t ldy, void *stream) {
    tsl_status st = check_shard(shard);
    if (st != TSL_OK)
        return st;
    if (!table || !tokens || !Y || M < 0)
        return TSL_ERR_INVALID_ARG;
    if ((tdtype != TSL_F32 && tdtype != TSL_BF16) || (ydtype != TSL_F32 && ydtype != TSL_BF16))
        return TSL_ERR_INVALID_ARG;
    const int64_t n_len = shard->n_len;
    if (ld_table < n_len || ldy < n_len)
        return TSL_ERR_INVALID_ARG;
    const size_t te = tdtype == TSL_F32 ? 4 : 2, ye = ydtype == TSL_F32 ? 4 : 2;
    if (!aligned(table, te) || !aligned(tokens, 4) || !aligned(Y, ye))
        return TSL_ERR_MISALIGNED;
    if (M == 0)
        return TSL_OK;
    if (matrices_overlap(Y, M, n_len, ldy, ye, table, shard->k_len, n_len, ld_table, te) ||
        overlaps(Y, span(M, n_len, ldy, ye), tokens, (size_t)M * 4))
        return TSL_ERR_INVALID_ARG;
    return from_hip(launch_embed_lookup(tdtype, table, ld_table, tokens, M, shard->k_off,
                                        shard->k_len, n_len, ydtype, Y, ldy,
                                        static_cast<hipStream_t>(stream)));
}

extern "C" tsl_status moe_gather(const void *src, int64_t ld_src, int64_t n_src, tsl_dtype dtype,
                                 const int32_t *idx, int64_t n, int64_t width, void *out,
                                 int64_t ldo, void *stream) {
    if (!src || !idx || !out || n_src < 1 || n < 0 || width < 1 || ld_src < width || ldo < width)
        return TSL_ERR_INVALID_ARG;
    if (dtype != TSL_F32 && dtype != TSL_BF16)
        return TSL_ERR_INVALID_ARG;
    const size_t e = dtype == TSL_F32 ? 4 : 2;
    if (!aligned(src, e) || !aligned(out, e) || !aligned(idx, 4))
        return TSL_ERR_MISALIGNED;
    if (n == 0)
        return TSL_OK;
    if (matrices_overlap(out, n, width, ldo, e, src, n_src, width, ld_src, e) ||
        overlaps(out, span(n, width, ldo, e), idx, (size_t)n * 4))
        return TSL_ERR_INVALID_ARG;
    // a row gather is a lookup into a table of n_src rows that one rank owns whole
    return from_hip(launch_embed_lookup(dtype, src, ld_src, idx, n, 0, n_src, width, dtype, out,
                                        ldo, static_cast<hipStream_t>(stream)));
}

extern "C" tsl_status moe_combine(const float *P, int64_t ldp, int64_t n_rows,
                                  const int32_t *slot_row, const float *weights, int64_t T,
                                  int32_t k, int64_t n, tsl_dtype ydtype, void *Y, int64_t ldy,
                                  void *stream) {
    if (!slot_row || !weights || !Y || T < 0 || k < 1 || n < 0 || n_rows < 0 || ldy < n)
        return TSL_ERR_INVALID_ARG;
    if (n_rows > 0 && (!P || ldp < n))
        return TSL_ERR_INVALID_ARG;
    if (ydtype != TSL_F32 && ydtype != TSL_BF16)
        return TSL_ERR_INVALID_ARG;
    const size_t ye = ydtype == TSL_F32 ? 4 : 2;
    if ((P && !aligned(P, 4)) || !aligned(slot_row, 4) || !aligned(weights, 4) || !aligned(Y, ye))
        return TSL_ERR_MISALIGNED;
    if (T == 0 || n == 0)
        return TSL_OK;
    const size_t ybytes = span(T, n, ldy, ye);
    if ((n_rows > 0 && matrices_overlap(Y, T, n, ldy, ye, P, n_rows, n, ldp, 4)) ||
        overlaps(Y, ybytes, slot_row, (size_t)T * k * 4) ||
        overlaps(Y, ybytes, weights, (size_t)T * k * 4))
        return TSL_ERR_INVALID_ARG;
    return from_hip(launch_moe_combine(P, ldp, n_rows, slot_row, weights, T, k, n, ydtype, Y, ldy,
                                       static_cast<hipStream_t>(stream)));
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
