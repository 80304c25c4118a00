// pack_shard kernels: cut a rank's block out of the full logical W[K][N]
// (mlxcel manual "Tensor parallelism", "Column Parallel" / "Row Parallel":
// a rank holds a contiguous block of columns or of rows) and lay it out in
// the MFMA operand order the shard_linear kernels stream.  One thread
// writes one 16-byte lane chunk; out-of-shard positions are written as 0.
#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

// Dense (F32 / BF16): chunk (nt, kt, lane) holds ELEMS consecutive k of
// column nt*16 + lane%16, starting at k = kt*KTILE + (lane/16)*ELEMS.
template <typename T, int ELEMS>
__global__ void __launch_bounds__(256) pack_dense_kernel(const T *__restrict__ W, int64_t stride_k,
                                                         int64_t stride_n, int64_t k_off,
                                                         int64_t n_off, int64_t Ks, int64_t Ns,
                                                         int64_t KT, int64_t chunks,
                                                         T *__restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks)
        return;
    const int lane = (int)(c & 63);
    const int64_t tile = c >> 6; // nt * KT + kt
    const int64_t nt = tile / KT, kt = tile % KT;
    const int64_t n = nt * 16 + (lane & 15);
    const int64_t k0 = kt * (4 * ELEMS) + (int64_t)(lane >> 4) * ELEMS;
    T v[ELEMS];
#pragma unroll
    for (int j = 0; j < ELEMS; ++j) {
        const int64_t k = k0 + j;
        v[j] = (n < Ns && k < Ks) ? W[(k_off + k) * stride_k + (n_off + n) * stride_n] : T(0);
    }
    T *dst = out + c * ELEMS;
#pragma unroll
    for (int j = 0; j < ELEMS; ++j)
        dst[j] = v[j];
}

// Q4: chunk (nt, blk, lane) = 4 code words, word t covering
// k = blk*128 + t*32 + (lane/16)*8 + j, j < 8, of column nt*16 + lane%16.
__global__ void __launch_bounds__(256) pack_q4_codes_kernel(const uint8_t *__restrict__ codes,
                                                            int64_t stride_k, int64_t stride_n,
                                                            int64_t k_off, int64_t n_off,
                                                            int64_t Ks, int64_t Ns, int64_t KB,
                                                            int64_t chunks,
                                                            char *__restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks)
        return;
    const int lane = (int)(c & 63);
    const int64_t tile = c >> 6;
    const int64_t nt = tile / KB, blk = tile % KB;
    const int64_t n = nt * 16 + (lane & 15);
    uint32_t words[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t w = 0;
        const int64_t k0 = blk * 128 + t * 32 + (int64_t)(lane >> 4) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t k = k0 + j;
            uint32_t q = 0;
            if (n < Ns && k < Ks)
                q = codes[(k_off + k) * stride_k + (n_off + n) * stride_n] & 0xFu;
            const int shift = (j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1);
            w |= q << shift;
        }
        words[t] = w;
    }
    u32x4 v = {words[0], words[1], words[2], words[3]};
    *reinterpret_cast<u32x4 *>(out + tile * kQ4Record + lane * 16) = v;
}

// Q4 scale/bias pairs: entry (nt, blk, i, h) for column nt*16 + i and group
// g = 2 blk + h (the two groups of a 128-k block side by side), stored after
// the codes of record (nt, blk).
__global__ void __launch_bounds__(256) pack_q4_sb_kernel(const uint16_t *__restrict__ scales,
                                                         const uint16_t *__restrict__ biases,
                                                         int64_t sb_stride_g, int64_t sb_stride_n,
                                                         int64_t g_off, int64_t n_off,
                                                         int64_t Gs, int64_t Ns, int64_t GP,
                                                         int64_t entries,
                                                         char *__restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= entries)
        return;
    const int h = (int)(e & 1);
    const int i = (int)((e >> 1) & 15);
    const int64_t t = e >> 5;
    const int64_t KB = GP / 2;
    const int64_t nt = t / KB, g = 2 * (t % KB) + h;
    const int64_t n = nt * 16 + i;
    uint32_t v = 0;
    if (n < Ns && g < Gs) {
        const int64_t at = (g_off + g) * sb_stride_g + (n_off + n) * sb_stride_n;
        v = (uint32_t)scales[at] | ((uint32_t)biases[at] << 16);
    }
    *reinterpret_cast<uint32_t *>(out + t * kQ4Record + kQ4PairsAt + (e & 31) * 4) = v;
}

// Q4 column exponents: f_n = ilogb(max over the column's groups of
// 15 |s| + |b|) - kWeightExpBias, 0 for a column whose groups are all zero
// (or not finite).  Every weight s q + b of the column then satisfies
// |(s q + b) 2^-f_n| <= 15 |s| 2^-f_n + |b| 2^-f_n < 2^15: the binary16
// form of the GEMM regime holds the column's largest weights at full
// precision whatever the magnitude of its scales and biases.
__global__ void __launch_bounds__(256) pack_q4_exp_kernel(const uint16_t *__restrict__ scales,
                                                          const uint16_t *__restrict__ biases,
                                                          int64_t sb_stride_g, int64_t sb_stride_n,
                                                          int64_t g_off, int64_t n_off, int64_t Gs,
                                                          int64_t Ns, int64_t NP,
                                                          int32_t *__restrict__ out) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= NP)
        return;
    float m = 0.f;
    if (n < Ns) {
        for (int64_t g = 0; g < Gs; ++g) {
            const int64_t at = (g_off + g) * sb_stride_g + (n_off + n) * sb_stride_n;
            const float sc = __uint_as_float((uint32_t)scales[at] << 16);
            const float bi = __uint_as_float((uint32_t)biases[at] << 16);
            m = fmaxf(m, __builtin_fmaf(15.f, fabsf(sc), fabsf(bi)));
        }
    }
    // frexp's exponent is ilogb + 1 for finite non-zero m
    out[n] = (m > 0.f && m <= 3.4028234663852886e38f)
                 ? __builtin_amdgcn_frexp_expf(m) - 1 - kWeightExpBias
                 : 0;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

} // namespace

hipError_t launch_pack_dense(const PackGeom &g, tsl_dtype wdtype, const void *W, int64_t stride_k,
                             int64_t stride_n, int64_t k_off, int64_t n_off, void *packed,
                             hipStream_t stream) {
    const int64_t chunks = g.Nt * g.KT * 64;
    if (chunks == 0)
        return hipSuccess;
    if (wdtype == TSL_F32) {
        hipLaunchKernelGGL((pack_dense_kernel<float, 4>), dim3(blocks_for(chunks, 256)), dim3(256),
                           0, stream, static_cast<const float *>(W), stride_k, stride_n, k_off,
                           n_off, g.Ks, g.Ns, g.KT, chunks, static_cast<float *>(packed));
    } else {
        hipLaunchKernelGGL((pack_dense_kernel<uint16_t, 8>), dim3(blocks_for(chunks, 256)),
                           dim3(256), 0, stream, static_cast<const uint16_t *>(W), stride_k,
                           stride_n, k_off, n_off, g.Ks, g.Ns, g.KT, chunks,
                           static_cast<uint16_t *>(packed));
    }
    return hipGetLastError();
}

hipError_t launch_pack_q4(const PackGeom &g, const uint8_t *codes, int64_t stride_k,
                          int64_t stride_n, const uint16_t *scales, const uint16_t *biases,
                          int64_t sb_stride_g, int64_t sb_stride_n, int64_t k_off, int64_t n_off,
                          void *packed, hipStream_t stream) {
    const int64_t chunks = g.Nt * g.KT * 64;
    if (chunks == 0)
        return hipSuccess;
    char *out = static_cast<char *>(packed);
    hipLaunchKernelGGL(pack_q4_codes_kernel, dim3(blocks_for(chunks, 256)), dim3(256), 0, stream,
                       codes, stride_k, stride_n, k_off, n_off, g.Ks, g.Ns, g.KT, chunks, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t GP = g.KT * 2; // groups per column, padded to whole 128-k blocks
    const int64_t entries = g.Nt * GP * 16;
    hipLaunchKernelGGL(pack_q4_sb_kernel, dim3(blocks_for(entries, 256)), dim3(256), 0, stream,
                       scales, biases, sb_stride_g, sb_stride_n, k_off / 64, n_off, g.Ks / 64,
                       g.Ns, GP, entries, out);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t NP = g.Nt * 16;
    hipLaunchKernelGGL(pack_q4_exp_kernel, dim3(blocks_for(NP, 256)), dim3(256), 0, stream, scales,
                       biases, sb_stride_g, sb_stride_n, k_off / 64, n_off, g.Ks / 64, g.Ns, NP,
                       reinterpret_cast<int32_t *>(out + g.exp_off));
    return hipGetLastError();
}

} // namespace tsl
