// Vocabulary-parallel embedding lookup (mlxcel manual "Tensor
// parallelism", "Vocab Parallel": each rank owns a contiguous slice of the
// vocabulary and looks up only the tokens that fall in it).  One pass over
// the output: thread (row m, column group j) reads its token id, copies
// the table row's elements when the rank owns the token and writes -0.0
// otherwise, so the rank-ordered binary32 sum of the partials is the owned
// row exactly (x + -0.0 == x for every x, -0.0 included).
#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ void put(float *y, float v) { *y = v; }
__device__ __forceinline__ void put(uint16_t *y, float v) {
    __bf16 b = (__bf16)v;
    *y = __builtin_bit_cast(uint16_t, b);
}
// bf16 -> bf16 keeps the bits (a NaN payload included)
__device__ __forceinline__ void copy_elem(uint16_t *y, uint16_t v) { *y = v; }
__device__ __forceinline__ void copy_elem(float *y, float v) { *y = v; }
template <typename TY, typename TT> __device__ __forceinline__ void move_elem(TY *y, TT v) {
    if constexpr (sizeof(TY) == sizeof(TT))
        copy_elem(y, v);
    else
        put(y, to_f32(v));
}

template <typename TY> __device__ __forceinline__ TY neg_zero();
template <> __device__ __forceinline__ float neg_zero<float>() { return -0.0f; }
template <> __device__ __forceinline__ uint16_t neg_zero<uint16_t>() { return 0x8000u; }

// V consecutive elements per thread; V == 4 needs n_len, ld_table and ldy
// multiples of 4 and table / Y aligned to 4 elements (checked on the host).
template <typename TT, typename TY, int V>
__global__ void __launch_bounds__(256) embed_kernel(const TT *__restrict__ table, int64_t ld_table,
                                                    const int32_t *__restrict__ tokens, int64_t M,
                                                    int64_t k_off, int64_t k_len, int64_t n_len,
                                                    TY *__restrict__ Y, int64_t ldy) {
    const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
    if (j >= n_len)
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const int64_t local = (int64_t)tokens[m] - k_off;
        TY *y = Y + m * ldy + j;
        TY out[V];
        if (local >= 0 && local < k_len) {
            const TT *src = table + local * ld_table + j;
            TT in[V];
            if constexpr (V == 4) {
                typedef TT tv __attribute__((ext_vector_type(4)));
                const tv w = *reinterpret_cast<const tv *>(src);
                in[0] = w.x;
                in[1] = w.y;
                in[2] = w.z;
                in[3] = w.w;
            } else {
                in[0] = src[0];
            }
#pragma unroll
            for (int i = 0; i < V; ++i)
                move_elem(&out[i], in[i]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                out[i] = neg_zero<TY>();
        }
        if constexpr (V == 4) {
            typedef TY yv __attribute__((ext_vector_type(4)));
            yv w = {out[0], out[1], out[2], out[3]};
            *reinterpret_cast<yv *>(y) = w;
        } else {
            y[0] = out[0];
        }
    }
}

template <typename TT, typename TY>
hipError_t launch_typed(const void *table, int64_t ld_table, const int32_t *tokens, int64_t M,
                        int64_t k_off, int64_t k_len, int64_t n_len, void *Y, int64_t ldy,
                        hipStream_t stream) {
    const bool vec = n_len % 4 == 0 && ld_table % 4 == 0 && ldy % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(table) % (4 * sizeof(TT))) == 0 &&
                     (reinterpret_cast<uintptr_t>(Y) % (4 * sizeof(TY))) == 0;
    const unsigned rows = (unsigned)(M < 65535 ? M : 65535);
    const TT *t = static_cast<const TT *>(table);
    TY *y = static_cast<TY *>(Y);
    if (vec)
        hipLaunchKernelGGL((embed_kernel<TT, TY, 4>), dim3((unsigned)((n_len / 4 + 255) / 256), rows),
                           dim3(256), 0, stream, t, ld_table, tokens, M, k_off, k_len, n_len, y,
                           ldy);
    else
        hipLaunchKernelGGL((embed_kernel<TT, TY, 1>), dim3((unsigned)((n_len + 255) / 256), rows),
                           dim3(256), 0, stream, t, ld_table, tokens, M, k_off, k_len, n_len, y,
                           ldy);
    return hipGetLastError();
}

} // namespace

hipError_t launch_embed_lookup(tsl_dtype tdtype, const void *table, int64_t ld_table,
                               const int32_t *tokens, int64_t M, int64_t k_off, int64_t k_len,
                               int64_t n_len, tsl_dtype ydtype, void *Y, int64_t ldy,
                               hipStream_t stream) {
    if (tdtype == TSL_F32 && ydtype == TSL_F32)
        return launch_typed<float, float>(table, ld_table, tokens, M, k_off, k_len, n_len, Y, ldy,
                                          stream);
    if (tdtype == TSL_F32)
        return launch_typed<float, uint16_t>(table, ld_table, tokens, M, k_off, k_len, n_len, Y,
                                             ldy, stream);
    if (ydtype == TSL_F32)
        return launch_typed<uint16_t, float>(table, ld_table, tokens, M, k_off, k_len, n_len, Y,
                                             ldy, stream);
    return launch_typed<uint16_t, uint16_t>(table, ld_table, tokens, M, k_off, k_len, n_len, Y,
                                            ldy, stream);
}

} // namespace tsl
