// Decode-sized shard_linear (M <= 64 per block of rows): one rank's
// Y_i = X W_i (column / replicated shard) or Y_i = X_i W_i (row shard)
// (wiki "Tensor parallel processing", "Details" §1; mlxcel manual "Tensor
// parallelism", "Column Parallel" / "Row Parallel").
//
// The weights dominate the bytes, so the kernel streams every packed weight
// byte exactly once per 64 rows: each lane issues all of its 16-byte loads
// up front (contiguous 1 KB per wave instruction, the packed layout is
// already in MFMA operand order), then runs 16x16 MFMAs with the
// activations read straight from L2 as operand fragments.
//
// Work split: a workgroup = 4 waves owns NTW 16-column tiles and one of
// `ks` k-ranges; its 4 waves take consecutive quarters of that range.  The
// wave partials are summed in LDS in ascending k order; with ks > 1 the
// workgroup partials go to the workspace and a second kernel sums them in
// ascending order, so results are run-to-run deterministic.
//
// One launch serves a group of shard products with the same M and types
// (several projections, or every rank's shard of one): the item table
// rides in the kernel arguments and each workgroup finds its item by
// binary search over the items' first workgroup indices.  Large groups
// need no k-split at all, which removes the second kernel.
//
// 4-bit weights (w = s q + b per group of 64 k) are applied exactly:
// the MFMA multiplies the bf16 activations by 128 + q (an exact bf16), and
// per group the accumulator takes s * sum(x (128 + q)) + (b - 128 s) * sum(x),
// sum(x) coming from one extra MFMA against a ones operand.  This is the
// group-sum identity of the affine format, evaluated in binary32.
#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

enum { W_F32 = 0, W_BF16 = 1, W_Q4 = 2 };

struct SkinnyItem {
    const void *B;       // packed weights (codes for Q4)
    const uint32_t *SB;  // Q4 scale/bias pairs
    const void *X;
    void *Y;
    float *P;            // workspace partials [ks][M][Ns] (ks > 1)
    int64_t ldx, ldy;
    int32_t Ks, Ns, Nt;
    int32_t KC;          // chunks along k (16, 32 or 128 k each)
    int32_t GP;          // Q4: groups per column in the packed pairs
    int32_t ks, n_groups;
    int32_t start;       // first workgroup of this item
    int32_t accumulate, y_bf16;
};

struct SkinnyGroup {
    int64_t M;
    int32_t n, pad_;
    SkinnyItem it[kGroupMax];
};

// Activation fragment, bf16: 8 consecutive k of one row (zero outside).
__device__ __forceinline__ bf16x8 load_x_bf16(const uint16_t *X, int64_t ldx, int64_t row,
                                              int64_t M, int64_t k, int64_t Ks) {
    u32x4 v = {0, 0, 0, 0};
    if (row < M) {
        const uint16_t *p = X + row * ldx + k;
        if (k + 8 <= Ks) {
            v = *reinterpret_cast<const u32x4 *>(p);
        } else if (k < Ks) {
            uint16_t t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                t[j] = (k + j < Ks) ? p[j] : (uint16_t)0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = (uint32_t)t[2 * j] | ((uint32_t)t[2 * j + 1] << 16);
        }
    }
    return __builtin_bit_cast(bf16x8, v);
}

// Activation fragment, f32: 4 consecutive k of one row (zero outside).
__device__ __forceinline__ f32x4 load_x_f32(const float *X, int64_t ldx, int64_t row, int64_t M,
                                            int64_t k, int64_t Ks) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < M) {
        const float *p = X + row * ldx + k;
        if (k + 4 <= Ks) {
            v = *reinterpret_cast<const f32x4 *>(p);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = (k + j < Ks) ? p[j] : 0.f;
        }
    }
    return v;
}

template <int WT, int MT, int NTW, int CMAX>
__global__ void __launch_bounds__(256) skinny_kernel(SkinnyGroup grp) {
    constexpr int KCH = WT == W_F32 ? 16 : (WT == W_BF16 ? 32 : 128); // k per chunk
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int bid = blockIdx.x;
    int lo = 0, hi = grp.n - 1; // last item whose first workgroup is <= bid
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (grp.it[mid].start <= bid)
            lo = mid;
        else
            hi = mid - 1;
    }
    const SkinnyItem &a = grp.it[lo];
    const int64_t M = grp.M;
    const int u = bid - a.start;
    const int64_t nt0 = (int64_t)(u % a.n_groups) * NTW;
    const int ksi = (u / a.n_groups) % a.ks;
    const int64_t m0 = (int64_t)(u / a.n_groups / a.ks) * (16 * MT);

    // this wave's chunk range
    const int64_t S = (int64_t)a.ks * 4;
    const int64_t wg = (int64_t)ksi * 4 + wave;
    const int64_t c0 = wg * a.KC / S;
    const int64_t c1 = (wg + 1) * a.KC / S;
    const int nc = (int)(c1 - c0); // <= CMAX, guaranteed by the host plan

    // 1. issue every weight load of this wave
    u32x4 breg[NTW][CMAX];
    uint32_t sbreg[NTW][CMAX][2];
    const u32x4 *B = static_cast<const u32x4 *>(a.B);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int64_t nt = nt0 + j;
        const bool nt_ok = nt < a.Nt;
#pragma unroll
        for (int c = 0; c < CMAX; ++c) {
            u32x4 v = {0, 0, 0, 0};
            if (nt_ok && c < nc)
                v = B[(nt * a.KC + c0 + c) * 64 + lane];
            breg[j][c] = v;
            if (WT == W_Q4) {
                uint32_t s0 = 0, s1 = 0;
                if (nt_ok && c < nc) {
                    const uint32_t *sb = a.SB + (nt * a.GP + 2 * (c0 + c)) * 16 + (lane & 15);
                    s0 = sb[0];
                    s1 = sb[16];
                }
                sbreg[j][c][0] = s0;
                sbreg[j][c][1] = s1;
            }
        }
    }

    // 2. multiply
    f32x4 acc[MT][NTW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t arow = m0 + (lane & 15);
    const int kg = lane >> 4; // which run of k this lane feeds

#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
        if (c < nc) {
            const int64_t kb = (c0 + c) * KCH;
            if constexpr (WT == W_BF16) {
                const uint16_t *X = static_cast<const uint16_t *>(a.X);
                bf16x8 xa[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    xa[i] = load_x_bf16(X, a.ldx, arow + 16 * i, M, kb + 8 * kg, a.Ks);
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    bf16x8 b = __builtin_bit_cast(bf16x8, breg[j][c]);
#pragma unroll
                    for (int i = 0; i < MT; ++i)
                        acc[i][j] = mfma_bf16(xa[i], b, acc[i][j]);
                }
            } else if constexpr (WT == W_F32) {
                const float *X = static_cast<const float *>(a.X);
                f32x4 xa[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    xa[i] = load_x_f32(X, a.ldx, arow + 16 * i, M, kb + 4 * kg, a.Ks);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const float b = __uint_as_float(breg[j][c][t]);
#pragma unroll
                        for (int i = 0; i < MT; ++i)
                            acc[i][j] = mfma_f32(xa[i][t], b, acc[i][j]);
                    }
            } else { // W_Q4: 4 MFMA steps of 32 k = 2 groups of 64
                const uint16_t *X = static_cast<const uint16_t *>(a.X);
                const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u,
                                                                     0x3F803F80u, 0x3F803F80u});
                f32x4 xs[MT], ag[MT][NTW];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    bf16x8 xa[MT];
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        xa[i] = load_x_bf16(X, a.ldx, arow + 16 * i, M, kb + 32 * t + 8 * kg,
                                            a.Ks);
                        xs[i] = mfma_bf16(xa[i], ones,
                                          (t & 1) ? xs[i] : f32x4{0.f, 0.f, 0.f, 0.f});
                    }
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const bf16x8 b = q4_to_bf16_plus128(breg[j][c][t]);
#pragma unroll
                        for (int i = 0; i < MT; ++i)
                            ag[i][j] = mfma_bf16(xa[i], b,
                                                 (t & 1) ? ag[i][j] : f32x4{0.f, 0.f, 0.f, 0.f});
                    }
                    if (t & 1) { // end of group 2 * chunk + t / 2
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            const uint32_t sb = sbreg[j][c][t >> 1];
                            const float s = bf16_lo(sb);
                            const float cb = __builtin_fmaf(-128.f, s, bf16_hi(sb));
#pragma unroll
                            for (int i = 0; i < MT; ++i)
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    acc[i][j][r] = __builtin_fmaf(s, ag[i][j][r], acc[i][j][r]);
                                    acc[i][j][r] = __builtin_fmaf(cb, xs[i][r], acc[i][j][r]);
                                }
                        }
                    }
                }
            }
        }
    }

    // 3. sum the 4 wave partials in ascending k order (wave 0 first)
    __shared__ f32x4 red[3][MT][NTW][64];
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
                red[wave - 1][i][j][lane] = acc[i][j];
    }
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const f32x4 v = red[w][i][j][lane];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][j][r] = acc[i][j][r] + v[r];
            }

    // 4. write: lane holds rows 4 * (lane / 16) + r of column lane % 16
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int64_t col = (nt0 + j) * 16 + (lane & 15);
        if (col >= a.Ns)
            continue;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 16 * i + 4 * kg + r;
                if (row >= M)
                    continue;
                const float v = acc[i][j][r];
                if (a.ks > 1) {
                    a.P[((int64_t)ksi * M + row) * a.Ns + col] = v;
                } else if (a.y_bf16) {
                    __bf16 h = (__bf16)v;
                    static_cast<uint16_t *>(a.Y)[row * a.ldy + col] =
                        __builtin_bit_cast(uint16_t, h);
                } else {
                    float *y = static_cast<float *>(a.Y) + row * a.ldy + col;
                    *y = a.accumulate ? *y + v : v;
                }
            }
    }
}

typedef void (*SkinnyFn)(SkinnyGroup);

template <int WT, int MT>
SkinnyFn pick_ntw(int ntw) {
    switch (ntw) {
    case 1: return skinny_kernel<WT, MT, 1, 16>;
    case 2: return skinny_kernel<WT, MT, 2, 8>;
    default:
        if constexpr (MT <= 2)
            return skinny_kernel<WT, MT, 4, 4>;
        return nullptr;
    }
}

template <int WT>
SkinnyFn pick_mt(int mt, int ntw) {
    switch (mt) {
    case 1: return pick_ntw<WT, 1>(ntw);
    case 2: return pick_ntw<WT, 2>(ntw);
    default: return pick_ntw<WT, 4>(ntw);
    }
}

} // namespace

SkinnyPlan skinny_plan(const LinearItem *items, int n, tsl_dtype wdtype, int64_t M) {
    SkinnyPlan p;
    const int64_t rows = M < 64 ? M : 64;
    p.mt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
    p.m_blocks = (M + 16 * p.mt - 1) / (16 * p.mt);
    // n-tiles per wave: reuse each activation fragment over several weight
    // tiles once the fragment is as large as the weight bytes it meets
    if (wdtype == TSL_Q4G64)
        p.ntw = rows <= 2 ? 1 : (rows <= 8 ? 2 : (p.mt <= 2 ? 4 : 2));
    else if (wdtype == TSL_BF16)
        p.ntw = rows <= 16 ? 1 : 2;
    else
        p.ntw = 1;
    p.cmax = p.ntw == 1 ? 16 : (p.ntw == 2 ? 8 : 4);
    // k-split only as far as needed for ~200 workgroups over the whole group
    // (and at least as far as the register budget of a wave requires)
    int64_t base = 0;
    for (int i = 0; i < n; ++i)
        base += (items[i].g.Nt + p.ntw - 1) / p.ntw * p.m_blocks;
    const int64_t ks_want = base > 0 ? (200 + base - 1) / base : 1;
    p.ks.resize(n);
    p.ws_off.resize(n);
    size_t off = 0;
    for (int i = 0; i < n; ++i) {
        const int64_t KC = items[i].g.KT;
        const int64_t ks_min = (KC + 4 * p.cmax - 1) / (4 * p.cmax);
        const int64_t ks_cap = KC / 4 > 1 ? KC / 4 : 1;
        int64_t ks = ks_want < ks_cap ? ks_want : ks_cap;
        if (ks < ks_min)
            ks = ks_min;
        p.ks[i] = (int)ks;
        p.ws_off[i] = off;
        if (ks > 1)
            off += ((size_t)ks * (size_t)M * (size_t)items[i].g.Ns * sizeof(float) + 255) / 256 *
                   256;
    }
    p.ws_bytes = off;
    return p;
}

int64_t skinny_blocks(const SkinnyPlan &p, const LinearItem *items, int n) {
    int64_t most = 0;
    for (int c0 = 0; c0 < n; c0 += kGroupMax) {
        int64_t blocks = 0;
        for (int i = c0; i < n && i < c0 + kGroupMax; ++i)
            blocks += (items[i].g.Nt + p.ntw - 1) / p.ntw * p.ks[i] * p.m_blocks;
        most = blocks > most ? blocks : most;
    }
    return most;
}

hipError_t launch_skinny(const SkinnyPlan &p, const LinearItem *items, int n, tsl_dtype wdtype,
                         int64_t M, void *workspace, hipStream_t stream) {
    SkinnyFn fn = wdtype == TSL_F32    ? pick_mt<W_F32>(p.mt, p.ntw)
                  : wdtype == TSL_BF16 ? pick_mt<W_BF16>(p.mt, p.ntw)
                                       : pick_mt<W_Q4>(p.mt, p.ntw);
    if (!fn)
        return hipErrorInvalidValue;
    for (int c0 = 0; c0 < n; c0 += kGroupMax) {
        const int cn = n - c0 < kGroupMax ? n - c0 : kGroupMax;
        SkinnyGroup grp{};
        grp.M = M;
        grp.n = cn;
        int64_t blocks = 0;
        for (int i = 0; i < cn; ++i) {
            const LinearItem &L = items[c0 + i];
            SkinnyItem &a = grp.it[i];
            a.B = L.packed;
            a.SB = wdtype == TSL_Q4G64 ? reinterpret_cast<const uint32_t *>(
                                             static_cast<const char *>(L.packed) + L.g.codes_bytes)
                                       : nullptr;
            a.X = L.X;
            a.Y = L.Y;
            a.P = reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_off[c0 + i]);
            a.ldx = L.ldx;
            a.ldy = L.ldy;
            a.Ks = (int32_t)L.g.Ks;
            a.Ns = (int32_t)L.g.Ns;
            a.Nt = (int32_t)L.g.Nt;
            a.KC = (int32_t)L.g.KT;
            a.GP = (int32_t)(L.g.KT * 2);
            a.ks = p.ks[c0 + i];
            a.n_groups = (int32_t)((L.g.Nt + p.ntw - 1) / p.ntw);
            a.start = (int32_t)blocks;
            a.accumulate = L.accumulate;
            a.y_bf16 = L.ydtype == TSL_BF16;
            blocks += (int64_t)a.n_groups * a.ks * p.m_blocks;
        }
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0, stream, grp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        for (int i = 0; i < cn; ++i) {
            const SkinnyItem &a = grp.it[i];
            if (a.ks == 1)
                continue;
            e = launch_splitk_reduce(a.P, a.ks, M, a.Ns, items[c0 + i].ydtype, a.Y, a.ldy,
                                     a.accumulate, stream);
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

} // namespace tsl
