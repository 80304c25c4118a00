// Mixture-of-experts token combine (mlxcel manual "Tensor parallelism",
// "MoE expert parallelization": each rank runs the experts it holds; a
// token's output is the router-weighted sum over its chosen experts, and
// the ranks' shares add up like row-parallel partials).  One pass over the
// output: thread (token t, 4 columns) walks the token's k slots in order
// and accumulates weight * expert row with fused multiply-adds in
// binary32, starting from -0.0.  Eight slots at a time: their rows and
// weights first, then the held slots' expert rows all in flight together,
// then the adds in slot order.
#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

template <typename TY, int V>
__global__ void __launch_bounds__(256) moe_combine_kernel(const float *__restrict__ P, int64_t ldp,
                                                          int64_t n_rows,
                                                          const int32_t *__restrict__ slot_row,
                                                          const float *__restrict__ weights,
                                                          int64_t T, int k, int64_t n,
                                                          TY *__restrict__ Y, int64_t ldy) {
    const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
    if (j >= n)
        return;
    for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i)
            acc[i] = -0.0f;
        constexpr int KU = 8;
        for (int s0 = 0; s0 < k; s0 += KU) {
            int64_t rr[KU];
            float ww[KU];
            bool held[KU];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int s = s0 + u;
                rr[u] = s < k ? slot_row[t * k + s] : -1;
                held[u] = rr[u] >= 0 && rr[u] < n_rows; // else another rank's expert
                ww[u] = held[u] ? weights[t * k + s] : 0.f;
            }
            float vv[KU][V];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                if (!held[u])
                    continue;
                const float *p = P + rr[u] * ldp + j;
                if constexpr (V == 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
                    vv[u][0] = v.x;
                    vv[u][1] = v.y;
                    vv[u][2] = v.z;
                    vv[u][3] = v.w;
                } else {
                    vv[u][0] = p[0];
                }
            }
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                if (!held[u])
                    continue;
#pragma unroll
                for (int i = 0; i < V; ++i)
                    acc[i] = __builtin_fmaf(ww[u], vv[u][i], acc[i]);
            }
        }
        TY *y = Y + t * ldy + j;
        if constexpr (sizeof(TY) == 4) {
            if constexpr (V == 4)
                *reinterpret_cast<f32x4 *>(y) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            else
                y[0] = acc[0];
        } else {
            if constexpr (V == 4) {
                const u32x2 w2 = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
                *reinterpret_cast<u32x2 *>(y) = w2;
            } else {
                const __bf16 h = (__bf16)acc[0];
                y[0] = __builtin_bit_cast(uint16_t, h);
            }
        }
    }
}

} // namespace

hipError_t launch_moe_combine(const float *P, int64_t ldp, int64_t n_rows, const int32_t *slot_row,
                              const float *weights, int64_t T, int k, int64_t n, tsl_dtype ydtype,
                              void *Y, int64_t ldy, hipStream_t stream) {
    const size_t ye = ydtype == TSL_F32 ? 4 : 2;
    const bool vec = n % 4 == 0 && ldp % 4 == 0 && ldy % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(P) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(Y) % (4 * ye)) == 0;
    const int V = vec ? 4 : 1;
    dim3 grid((unsigned)((n / V + 255) / 256), (unsigned)(T < 65535 ? T : 65535));
    if (ydtype == TSL_F32) {
        float *y = static_cast<float *>(Y);
        if (vec)
            hipLaunchKernelGGL((moe_combine_kernel<float, 4>), grid, dim3(256), 0, stream, P, ldp,
                               n_rows, slot_row, weights, T, k, n, y, ldy);
        else
            hipLaunchKernelGGL((moe_combine_kernel<float, 1>), grid, dim3(256), 0, stream, P, ldp,
                               n_rows, slot_row, weights, T, k, n, y, ldy);
    } else {
        uint16_t *y = static_cast<uint16_t *>(Y);
        if (vec)
            hipLaunchKernelGGL((moe_combine_kernel<uint16_t, 4>), grid, dim3(256), 0, stream, P,
                               ldp, n_rows, slot_row, weights, T, k, n, y, ldy);
        else
            hipLaunchKernelGGL((moe_combine_kernel<uint16_t, 1>), grid, dim3(256), 0, stream, P,
                               ldp, n_rows, slot_row, weights, T, k, n, y, ldy);
    }
    return hipGetLastError();
}

} // namespace tsl
