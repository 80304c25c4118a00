// combine_partials kernels: the on-device stand-ins for the collectives that
// join rank outputs (mlxcel manual "Tensor parallelism", "Communication
// patterns": all-reduce after a row-parallel layer, all-gather after a
// column-parallel one; wiki "Tensor parallel processing", "Details" §1:
// Y = sum_i Y_i and Y = [Y_1 ... Y_n]).  Every part already sits on this
// GPU, so the join is a streaming pass over HBM: 16-byte loads and stores,
// one thread per 4 columns (SUM) or per 16 bytes (CONCAT), rows over
// blockIdx.y.  The sum runs in ascending rank order in binary32.
#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

struct PartPtrs {
    const void *p[kMaxParts];
};

__device__ __forceinline__ void store4(float *y, f32x4 v) { *reinterpret_cast<f32x4 *>(y) = v; }
__device__ __forceinline__ void store4(uint16_t *y, f32x4 v) {
    u32x2 w = {pack_bf16(v.x, v.y), pack_bf16(v.z, v.w)};
    *reinterpret_cast<u32x2 *>(y) = w;
}
// Streaming (non-temporal) stores of 4 consecutive outputs: for outputs
// that the launch does not read back.  y aligned to 4 elements.
__device__ __forceinline__ void store4_nt(float *y, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(y));
}
__device__ __forceinline__ void store4_nt(uint16_t *y, f32x4 v) {
    u32x2 w = {pack_bf16(v.x, v.y), pack_bf16(v.z, v.w)};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(y));
}
__device__ __forceinline__ void store1(float *y, float v) { *y = v; }
__device__ __forceinline__ void store1(uint16_t *y, float v) {
    __bf16 b = (__bf16)v;
    *y = __builtin_bit_cast(uint16_t, b);
}

// Vector path: n_each, ld_part and ldy are multiples of 4 and every base is
// 16-byte aligned (checked on the host).
template <typename TY>
__global__ void __launch_bounds__(256) sum_vec_kernel(PartPtrs parts, int n_parts, int64_t M,
                                                      int64_t n_each, int64_t ld_part,
                                                      TY *Y, int64_t ldy) {
    const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (j >= n_each)
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const int64_t off = m * ld_part + j;
        f32x4 acc = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(parts.p[0]) + off);
        for (int r = 1; r < n_parts; ++r) {
            f32x4 v =
                *reinterpret_cast<const f32x4 *>(static_cast<const float *>(parts.p[r]) + off);
            acc.x = acc.x + v.x;
            acc.y = acc.y + v.y;
            acc.z = acc.z + v.z;
            acc.w = acc.w + v.w;
        }
        store4(Y + m * ldy + j, acc);
    }
}

template <typename TY>
__global__ void __launch_bounds__(256) sum_scalar_kernel(PartPtrs parts, int n_parts, int64_t M,
                                                         int64_t n_each, int64_t ld_part,
                                                         TY *Y, int64_t ldy) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n_each)
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const int64_t off = m * ld_part + j;
        float acc = static_cast<const float *>(parts.p[0])[off];
        for (int r = 1; r < n_parts; ++r)
            acc = acc + static_cast<const float *>(parts.p[r])[off];
        store1(Y + m * ldy + j, acc);
    }
}

// CONCAT, moving VEC-byte units (16 when every row start is 16-byte aligned).
template <int VEC>
__global__ void __launch_bounds__(256) concat_kernel(PartPtrs parts, int64_t M, int64_t row_units,
                                                     int64_t ld_part_bytes, char *__restrict__ Y,
                                                     int64_t ldy_bytes, int64_t part_bytes) {
    typedef uint8_t unit_t __attribute__((ext_vector_type(VEC)));
    const int r = blockIdx.z;
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= row_units)
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const char *src = static_cast<const char *>(parts.p[r]) + m * ld_part_bytes + u * VEC;
        char *dst = Y + m * ldy_bytes + (int64_t)r * part_bytes + u * VEC;
        *reinterpret_cast<unit_t *>(dst) = *reinterpret_cast<const unit_t *>(src);
    }
}

// Split-K finish: Y (+)= sum_s P[s], ascending s.
template <typename TY>
__global__ void __launch_bounds__(256) splitk_kernel(const float *__restrict__ P, int ks, int64_t M,
                                                     int64_t N, TY *__restrict__ Y, int64_t ldy,
                                                     int accumulate) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= N)
        return;
    const int64_t plane = M * N;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        float acc = P[m * N + j];
        for (int s = 1; s < ks; ++s)
            acc = acc + P[s * plane + m * N + j];
        TY *y = Y + m * ldy + j;
        if (accumulate)
            acc = *reinterpret_cast<float *>(y) + acc; // accumulate implies F32 output
        store1(y, acc);
    }
}

// Several sums in one launch (the rank sums of a grouped shard_linear):
// set s adds its parts (contiguous [M][n] binary32, ascending order) into
// its own output; workgroup x -> (set, 1024-column block) by binary search.
struct SumSet {
    const float *p[kSetParts];
    int32_t ks[kSetParts]; // k-partials of each product
    void *Y;
    int64_t ldy, n;
    int64_t M;           // rows of this set
    int32_t n_parts, y_bf16;
    int32_t start, pad_; // first workgroup of the set
};
struct SumSets {
    int32_t n, pad_;
    SumSet s[kMaxSets];
};

template <bool VEC>
__global__ void __launch_bounds__(256) sum_sets_kernel(SumSets g) {
    const int bid = blockIdx.x;
    int lo = 0, hi = g.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (g.s[mid].start <= bid)
            lo = mid;
        else
            hi = mid - 1;
    }
    const SumSet &st = g.s[lo];
    constexpr int E = VEC ? 4 : 1;
    const int64_t j = ((int64_t)(bid - st.start) * 256 + threadIdx.x) * E;
    if (j >= st.n)
        return;
    const int64_t plane = st.M * st.n; // one k-partial
    for (int64_t m = blockIdx.y; m < st.M; m += gridDim.y) {
        const int64_t off = m * st.n + j;
        if constexpr (VEC) {
            // product r: its k-partials added in k order
            auto product = [&](int r) {
                f32x4 v = *reinterpret_cast<const f32x4 *>(st.p[r] + off);
                for (int q = 1; q < st.ks[r]; ++q) {
                    const f32x4 w = *reinterpret_cast<const f32x4 *>(st.p[r] + q * plane + off);
                    v.x = v.x + w.x;
                    v.y = v.y + w.y;
                    v.z = v.z + w.z;
                    v.w = v.w + w.w;
                }
                return v;
            };
            f32x4 acc = product(0);
            for (int r = 1; r < st.n_parts; ++r) {
                const f32x4 v = product(r);
                acc.x = acc.x + v.x;
                acc.y = acc.y + v.y;
                acc.z = acc.z + v.z;
                acc.w = acc.w + v.w;
            }
            if (st.y_bf16)
                store4(static_cast<uint16_t *>(st.Y) + m * st.ldy + j, acc);
            else
                store4(static_cast<float *>(st.Y) + m * st.ldy + j, acc);
        } else {
            auto product = [&](int r) {
                float v = st.p[r][off];
                for (int q = 1; q < st.ks[r]; ++q)
                    v = v + st.p[r][q * plane + off];
                return v;
            };
            float acc = product(0);
            for (int r = 1; r < st.n_parts; ++r)
                acc = acc + product(r);
            if (st.y_bf16)
                store1(static_cast<uint16_t *>(st.Y) + m * st.ldy + j, acc);
            else
                store1(static_cast<float *>(st.Y) + m * st.ldy + j, acc);
        }
    }
}

// ---- every rank's result of a collective ----
struct OutPtrs {
    void *p[kMaxParts];
};

// First row of rank r's block of an [M][n] tensor split over n ranks.
__device__ __forceinline__ int64_t block_lo(int r, int64_t M, int n) {
    return ((int64_t)r * M) / n;
}

// Ordered binary32 sum of the parts at (m, j..j+V-1), written to every
// output (all-reduce) or to the owner of row m (reduce-scatter).  VST: V is
// 4 and every output row start is aligned to 4 elements, so each output
// takes one streaming vector store.
template <typename TY, int V, bool VST = false>
__global__ void __launch_bounds__(256) reduce_ranks_kernel(PartPtrs parts, int n, int64_t M,
                                                           int64_t n_each, int64_t ld_part,
                                                           OutPtrs outs, int64_t ldo,
                                                           int scatter) {
    const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
    if (j >= n_each)
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const int64_t off = m * ld_part + j;
        float acc[V];
#pragma unroll
        for (int e = 0; e < V; ++e)
            acc[e] = static_cast<const float *>(parts.p[0])[off + e];
        for (int r = 1; r < n; ++r)
#pragma unroll
            for (int e = 0; e < V; ++e)
                acc[e] = acc[e] + static_cast<const float *>(parts.p[r])[off + e];
        int r0 = 0, r1 = n;
        if (scatter) { // the rank whose block holds row m
            int r = (int)((m * n) / M);
            while (r + 1 < n && m >= block_lo(r + 1, M, n))
                ++r;
            while (r > 0 && m < block_lo(r, M, n))
                --r;
            r0 = r;
            r1 = r + 1;
        }
        for (int r = r0; r < r1; ++r) {
            const int64_t row = scatter ? m - block_lo(r, M, n) : m;
            TY *y = static_cast<TY *>(outs.p[r]) + row * ldo + j;
            if constexpr (VST) {
                store4_nt(y, f32x4{acc[0], acc[1], acc[2], acc[3]});
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    store1(y + e, acc[e]);
            }
        }
    }
}

// Row m of part q into columns [q n_each, (q+1) n_each) of row m of every
// output, in VEC-byte units (16 when every row start is 16-byte aligned):
// one load, n stores.
template <int VEC>
__global__ void __launch_bounds__(256) gather_ranks_kernel(PartPtrs parts, int n, int64_t M,
                                                           int64_t row_units, int64_t ld_part_bytes,
                                                           OutPtrs outs, int64_t ldo_bytes,
                                                           int64_t part_bytes) {
    typedef uint8_t unit_t __attribute__((ext_vector_type(VEC)));
    const int q = blockIdx.z;
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= row_units)
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const unit_t v = *reinterpret_cast<const unit_t *>(static_cast<const char *>(parts.p[q]) +
                                                           m * ld_part_bytes + u * VEC);
        const int64_t off = m * ldo_bytes + (int64_t)q * part_bytes + u * VEC;
        // streaming stores: the n copies are not read back by this launch
        for (int r = 0; r < n; ++r)
            __builtin_nontemporal_store(v, reinterpret_cast<unit_t *>(static_cast<char *>(outs.p[r]) + off));
    }
}

inline unsigned rows_grid(int64_t M) { return (unsigned)(M < 65535 ? M : 65535); }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

} // namespace

hipError_t launch_combine_sum(int n_parts, const float *const *parts, int64_t M, int64_t n_each,
                              int64_t ld_part, tsl_dtype ydtype, void *Y, int64_t ldy,
                              hipStream_t stream) {
    PartPtrs pp{};
    bool vec = (n_each % 4 == 0) && (ld_part % 4 == 0) && (ldy % 4 == 0) && aligned16(Y);
    for (int r = 0; r < n_parts; ++r) {
        pp.p[r] = parts[r];
        vec = vec && aligned16(parts[r]);
    }
    if (ydtype == TSL_BF16)
        vec = vec && ((reinterpret_cast<uintptr_t>(Y) & 7) == 0);
    if (vec) {
        dim3 grid((unsigned)((n_each / 4 + 255) / 256), rows_grid(M));
        if (ydtype == TSL_F32)
            hipLaunchKernelGGL(sum_vec_kernel<float>, grid, dim3(256), 0, stream, pp, n_parts, M,
                               n_each, ld_part, static_cast<float *>(Y), ldy);
        else
            hipLaunchKernelGGL(sum_vec_kernel<uint16_t>, grid, dim3(256), 0, stream, pp, n_parts, M,
                               n_each, ld_part, static_cast<uint16_t *>(Y), ldy);
    } else {
        dim3 grid((unsigned)((n_each + 255) / 256), rows_grid(M));
        if (ydtype == TSL_F32)
            hipLaunchKernelGGL(sum_scalar_kernel<float>, grid, dim3(256), 0, stream, pp, n_parts, M,
                               n_each, ld_part, static_cast<float *>(Y), ldy);
        else
            hipLaunchKernelGGL(sum_scalar_kernel<uint16_t>, grid, dim3(256), 0, stream, pp,
                               n_parts, M, n_each, ld_part, static_cast<uint16_t *>(Y), ldy);
    }
    return hipGetLastError();
}

hipError_t launch_combine_concat(int n_parts, const void *const *parts, size_t elem_bytes,
                                 int64_t M, int64_t n_each, int64_t ld_part, void *Y, int64_t ldy,
                                 hipStream_t stream) {
    PartPtrs pp{};
    const int64_t row_bytes = n_each * (int64_t)elem_bytes;
    const int64_t ldp_b = ld_part * (int64_t)elem_bytes, ldy_b = ldy * (int64_t)elem_bytes;
    bool vec = (row_bytes % 16 == 0) && (ldp_b % 16 == 0) && (ldy_b % 16 == 0) && aligned16(Y);
    for (int r = 0; r < n_parts; ++r) {
        pp.p[r] = parts[r];
        vec = vec && aligned16(parts[r]);
    }
    if (vec) {
        const int64_t units = row_bytes / 16;
        dim3 grid((unsigned)((units + 255) / 256), rows_grid(M), (unsigned)n_parts);
        hipLaunchKernelGGL(concat_kernel<16>, grid, dim3(256), 0, stream, pp, M, units, ldp_b,
                           static_cast<char *>(Y), ldy_b, row_bytes);
    } else if (elem_bytes == 4) {
        dim3 grid((unsigned)((n_each + 255) / 256), rows_grid(M), (unsigned)n_parts);
        hipLaunchKernelGGL(concat_kernel<4>, grid, dim3(256), 0, stream, pp, M, n_each, ldp_b,
                           static_cast<char *>(Y), ldy_b, row_bytes);
    } else {
        dim3 grid((unsigned)((n_each + 255) / 256), rows_grid(M), (unsigned)n_parts);
        hipLaunchKernelGGL(concat_kernel<2>, grid, dim3(256), 0, stream, pp, M, n_each, ldp_b,
                           static_cast<char *>(Y), ldy_b, row_bytes);
    }
    return hipGetLastError();
}

hipError_t launch_sum_sets(int n_sets, const SumSpec *sets, int64_t M, hipStream_t stream) {
    for (int c0 = 0; c0 < n_sets; c0 += kMaxSets) {
        const int cn = n_sets - c0 < kMaxSets ? n_sets - c0 : kMaxSets;
        SumSets g{};
        g.n = cn;
        bool vec = true;
        for (int i = 0; i < cn; ++i) {
            const SumSpec &sp = sets[c0 + i];
            vec = vec && sp.n % 4 == 0 && sp.ldy % 4 == 0 &&
                  (reinterpret_cast<uintptr_t>(sp.Y) & (sp.ydtype == TSL_F32 ? 15 : 7)) == 0;
            for (int r = 0; r < sp.n_parts; ++r)
                vec = vec && aligned16(sp.parts[r]);
        }
        int64_t blocks = 0;
        for (int i = 0; i < cn; ++i) {
            const SumSpec &sp = sets[c0 + i];
            SumSet &st = g.s[i];
            for (int r = 0; r < sp.n_parts; ++r) {
                st.p[r] = sp.parts[r];
                st.ks[r] = sp.ks[r];
            }
            st.Y = sp.Y;
            st.ldy = sp.ldy;
            st.n = sp.n;
            st.M = sp.M;
            st.n_parts = sp.n_parts;
            st.y_bf16 = sp.ydtype == TSL_BF16;
            st.start = (int32_t)blocks;
            blocks += (sp.n + 256 * (vec ? 4 : 1) - 1) / (256 * (vec ? 4 : 1));
        }
        dim3 grid((unsigned)blocks, rows_grid(M));
        if (vec)
            hipLaunchKernelGGL(sum_sets_kernel<true>, grid, dim3(256), 0, stream, g);
        else
            hipLaunchKernelGGL(sum_sets_kernel<false>, grid, dim3(256), 0, stream, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_reduce_to_ranks(int n, const float *const *parts, int64_t M, int64_t n_each,
                                  int64_t ld_part, int scatter, tsl_dtype odtype,
                                  void *const *outs, int64_t ldo, hipStream_t stream) {
    PartPtrs pp{};
    OutPtrs op{};
    for (int r = 0; r < n; ++r) {
        pp.p[r] = parts[r];
        op.p[r] = outs[r];
    }
    const bool vec = n_each % 4 == 0 && ld_part % 4 == 0 && ldo % 4 == 0;
    // vector stores: every output base aligned to 4 elements (rows then are too)
    bool vst = vec;
    const uintptr_t oalign = odtype == TSL_F32 ? 16 : 8;
    for (int r = 0; r < n; ++r)
        vst = vst && (reinterpret_cast<uintptr_t>(outs[r]) % oalign) == 0;
    const int V = vec ? 4 : 1;
    dim3 grid((unsigned)((n_each / V + 255) / 256), rows_grid(M));
    if (odtype == TSL_F32) {
        if (vst)
            hipLaunchKernelGGL((reduce_ranks_kernel<float, 4, true>), grid, dim3(256), 0, stream,
                               pp, n, M, n_each, ld_part, op, ldo, scatter);
        else if (vec)
            hipLaunchKernelGGL((reduce_ranks_kernel<float, 4>), grid, dim3(256), 0, stream, pp, n,
                               M, n_each, ld_part, op, ldo, scatter);
        else
            hipLaunchKernelGGL((reduce_ranks_kernel<float, 1>), grid, dim3(256), 0, stream, pp, n,
                               M, n_each, ld_part, op, ldo, scatter);
    } else {
        if (vst)
            hipLaunchKernelGGL((reduce_ranks_kernel<uint16_t, 4, true>), grid, dim3(256), 0,
                               stream, pp, n, M, n_each, ld_part, op, ldo, scatter);
        else if (vec)
            hipLaunchKernelGGL((reduce_ranks_kernel<uint16_t, 4>), grid, dim3(256), 0, stream, pp,
                               n, M, n_each, ld_part, op, ldo, scatter);
        else
            hipLaunchKernelGGL((reduce_ranks_kernel<uint16_t, 1>), grid, dim3(256), 0, stream, pp,
                               n, M, n_each, ld_part, op, ldo, scatter);
    }
    return hipGetLastError();
}

hipError_t launch_gather_to_ranks(int n, const void *const *parts, size_t elem_bytes, int64_t M,
                                  int64_t n_each, int64_t ld_part, void *const *outs, int64_t ldo,
                                  hipStream_t stream) {
    PartPtrs pp{};
    OutPtrs op{};
    for (int r = 0; r < n; ++r) {
        pp.p[r] = parts[r];
        op.p[r] = outs[r];
    }
    const int64_t row_bytes = n_each * (int64_t)elem_bytes;
    const int64_t ldp_b = ld_part * (int64_t)elem_bytes, ldo_b = ldo * (int64_t)elem_bytes;
    bool vec = (row_bytes % 16 == 0) && (ldp_b % 16 == 0) && (ldo_b % 16 == 0);
    for (int r = 0; r < n; ++r)
        vec = vec && aligned16(parts[r]) && aligned16(outs[r]);
    if (vec) {
        const int64_t units = row_bytes / 16;
        dim3 grid((unsigned)((units + 255) / 256), rows_grid(M), (unsigned)n);
        hipLaunchKernelGGL(gather_ranks_kernel<16>, grid, dim3(256), 0, stream, pp, n, M, units,
                           ldp_b, op, ldo_b, row_bytes);
    } else {
        dim3 grid((unsigned)((n_each + 255) / 256), rows_grid(M), (unsigned)n);
        if (elem_bytes == 4)
            hipLaunchKernelGGL(gather_ranks_kernel<4>, grid, dim3(256), 0, stream, pp, n, M,
                               n_each, ldp_b, op, ldo_b, row_bytes);
        else
            hipLaunchKernelGGL(gather_ranks_kernel<2>, grid, dim3(256), 0, stream, pp, n, M,
                               n_each, ldp_b, op, ldo_b, row_bytes);
    }
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *P, int ks, int64_t M, int64_t N, tsl_dtype ydtype,
                                void *Y, int64_t ldy, int accumulate, hipStream_t stream) {
    dim3 grid((unsigned)((N + 255) / 256), rows_grid(M));
    if (ydtype == TSL_F32)
        hipLaunchKernelGGL(splitk_kernel<float>, grid, dim3(256), 0, stream, P, ks, M, N,
                           static_cast<float *>(Y), ldy, accumulate);
    else
        hipLaunchKernelGGL(splitk_kernel<uint16_t>, grid, dim3(256), 0, stream, P, ks, M, N,
                           static_cast<uint16_t *>(Y), ldy, accumulate);
    return hipGetLastError();
}

} // namespace tsl
