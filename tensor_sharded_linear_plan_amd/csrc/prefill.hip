// Prefill-sized shard_linear: one rank's Y_i = X W_i (column / replicated
// shard) or Y_i = X_i W_i (row shard) for many token rows (wiki "Tensor
// parallel processing", "Details" §1; mlxcel manual "Tensor parallelism",
// "Column Parallel" / "Row Parallel").  A dense contraction, so it runs on
// the matrix cores.
//
// Block tile BM x BN x 64 with BM = 64 * MTW rows (4 waves stacked along M,
// each 16 * MTW rows) and BN = 16 * NT columns; every wave multiplies its
// rows by all BN columns.  Both operands are staged through LDS in MFMA
// fragment order (one conflict-free 16-byte read per lane per fragment),
// double buffered: the global loads of tile k + 1 are in flight while tile
// k is multiplied, one barrier per 64 k.
//
// bf16 weights: bf16 x bf16 MFMA.  4-bit weights: each weight is
// dequantised once per workgroup, w = s q + b rounded once to binary16,
// while staging; the bf16 activations are narrowed to binary16 (exact below
// 65520 in magnitude) so the MFMA is f16 x f16 with binary32 accumulation.
//
// The grid is one workgroup per tile, ordered so that the 8 XCDs (which
// receive workgroups round-robin) each own a contiguous run of row-major
// tiles and keep those activation rows in their own L2.
#include <mutex>
#include <utility>
#include <vector>

#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

enum { P_BF16 = 1, P_Q4 = 2 };

struct PrefillArgs {
    const void *B;      // packed weights (codes for Q4)
    const uint32_t *SB; // Q4 scale/bias pairs
    const uint16_t *X;  // bf16 activations
    int64_t ldx;
    int64_t M, Ks, Ns, Nt;
    int64_t KTB;        // packed k-tiles per column tile (bf16: 32-k tiles, Q4: 128-k blocks)
    int64_t GP;         // Q4 groups per column tile
    int64_t KT64;       // 64-k steps to run
    int64_t MB, NB;     // tile grid
    void *Y;
    int64_t ldy;
    int y_bf16, accumulate;
};

template <int WT, int MTW, int NT>
struct Cfg {
    static constexpr int BM = 64 * MTW;
    static constexpr int MTILES = BM / 16;
    static constexpr int A_CHUNKS = BM * 8 / 256;                 // 16-byte A chunks per thread
    static constexpr int B_ITEMS = WT == P_BF16 ? (NT * 128 + 255) / 256 : (NT * 64 + 255) / 256;
    static constexpr int A_BYTES = MTILES * 2 * 1024;             // per stage
    static constexpr int B_BYTES = NT * 2 * 1024;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = 2 * STAGE;
};

template <int WT, int MTW, int NT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_kernel(PrefillArgs a) {
    using C = Cfg<WT, MTW, NT>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // XCD-aware tile order
    const int64_t T = a.MB * a.NB;
    int64_t tile = blockIdx.x;
    if ((T & 7) == 0)
        tile = (tile & 7) * (T >> 3) + (tile >> 3);
    const int64_t mb = tile / a.NB, nb = tile % a.NB;
    const int64_t m0 = mb * C::BM;
    const int64_t nt0 = nb * NT;

    // ---- global -> register loads ----
    u32x4 ra[C::A_CHUNKS];
    u32x4 rb[WT == P_BF16 ? C::B_ITEMS : 1];
    u32x2 rq[WT == P_Q4 ? C::B_ITEMS : 1];
    uint32_t rs[WT == P_Q4 ? C::B_ITEMS : 1];

    auto load_tile = [&](int64_t kt) {
        const int64_t k0 = kt * 64;
#pragma unroll
        for (int i = 0; i < C::A_CHUNKS; ++i) {
            const int c = tid + 256 * i;
            const int64_t row = m0 + (c >> 3);
            const int64_t k = k0 + (c & 7) * 8;
            u32x4 v = {0, 0, 0, 0};
            if (row < a.M) {
                const uint16_t *p = a.X + row * a.ldx + k;
                if (k + 8 <= a.Ks) {
                    v = *reinterpret_cast<const u32x4 *>(p);
                } else if (k < a.Ks) {
                    uint16_t t[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        t[j] = (k + j < a.Ks) ? p[j] : (uint16_t)0;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        v[j] = (uint32_t)t[2 * j] | ((uint32_t)t[2 * j + 1] << 16);
                }
            }
            ra[i] = v;
        }
        if constexpr (WT == P_BF16) {
            const u32x4 *B = static_cast<const u32x4 *>(a.B);
#pragma unroll
            for (int i = 0; i < C::B_ITEMS; ++i) {
                const int c = tid + 256 * i;
                u32x4 v = {0, 0, 0, 0};
                if (c < NT * 128) {
                    const int64_t nt = nt0 + (c >> 7);
                    const int s = (c >> 6) & 1;
                    if (nt < a.Nt)
                        v = B[(nt * a.KTB + kt * 2 + s) * 64 + (c & 63)];
                }
                rb[i] = v;
            }
        } else {
            const uint32_t *Bq = static_cast<const uint32_t *>(a.B);
#pragma unroll
            for (int i = 0; i < C::B_ITEMS; ++i) {
                const int c = tid + 256 * i;
                u32x2 v = {0, 0};
                uint32_t s = 0;
                if (c < NT * 64) {
                    const int64_t nt = nt0 + (c >> 6);
                    if (nt < a.Nt) {
                        const int l = c & 63;
                        v = *reinterpret_cast<const u32x2 *>(
                            Bq + ((nt * a.KTB + (kt >> 1)) * 64 + l) * 4 + 2 * (kt & 1));
                        s = a.SB[(nt * a.GP + kt) * 16 + (l & 15)];
                    }
                }
                rq[i] = v;
                rs[i] = s;
            }
        }
    };

    // ---- register -> LDS (fragment order) ----
    auto store_tile = [&](int stage) {
        char *As = smem + stage * C::STAGE;
        char *Bs = As + C::A_BYTES;
#pragma unroll
        for (int i = 0; i < C::A_CHUNKS; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 3, kc = c & 7;
            const int frag = (row >> 4) * 2 + (kc >> 2);
            const int l = (kc & 3) * 16 + (row & 15);
            u32x4 v = ra[i];
            if constexpr (WT == P_Q4) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = bf16pair_to_f16pair(v[j]);
            }
            *reinterpret_cast<u32x4 *>(As + (frag * 64 + l) * 16) = v;
        }
        if constexpr (WT == P_BF16) {
#pragma unroll
            for (int i = 0; i < C::B_ITEMS; ++i) {
                const int c = tid + 256 * i;
                if (c < NT * 128)
                    *reinterpret_cast<u32x4 *>(Bs + c * 16) = rb[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::B_ITEMS; ++i) {
                const int c = tid + 256 * i;
                if (c < NT * 64) {
                    const int j = c >> 6, l = c & 63;
                    const float s = bf16_lo(rs[i]);
                    const float cb = __builtin_fmaf(-1024.f, s, bf16_hi(rs[i]));
                    const f16x8 w0 = q4_dequant_f16(rq[i][0], s, cb);
                    const f16x8 w1 = q4_dequant_f16(rq[i][1], s, cb);
                    *reinterpret_cast<f16x8 *>(Bs + ((j * 2 + 0) * 64 + l) * 16) = w0;
                    *reinterpret_cast<f16x8 *>(Bs + ((j * 2 + 1) * 64 + l) * 16) = w1;
                }
            }
        }
    };

    f32x4 acc[MTW][NT];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage) {
        const char *As = smem + stage * C::STAGE;
        const char *Bs = As + C::A_BYTES;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            u32x4 af[MTW];
#pragma unroll
            for (int i = 0; i < MTW; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(
                    As + (((wave * MTW + i) * 2 + s) * 64 + lane) * 16);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const u32x4 bf = *reinterpret_cast<const u32x4 *>(Bs + ((j * 2 + s) * 64 + lane) * 16);
#pragma unroll
                for (int i = 0; i < MTW; ++i) {
                    if constexpr (WT == P_BF16)
                        acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                              __builtin_bit_cast(bf16x8, bf), acc[i][j]);
                    else
                        acc[i][j] = mfma_f16(__builtin_bit_cast(f16x8, af[i]),
                                             __builtin_bit_cast(f16x8, bf), acc[i][j]);
                }
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int64_t kt = 0; kt < a.KT64; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < a.KT64;
        if (more)
            load_tile(kt + 1);
        compute(cur);
        if (more)
            store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows 4 * (lane / 16) + r of column lane % 16 ----
    const int kg = lane >> 4;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int64_t col = (nt0 + j) * 16 + (lane & 15);
        if (col >= a.Ns)
            continue;
#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + (wave * MTW + i) * 16 + 4 * kg + r;
                if (row >= a.M)
                    continue;
                const float v = acc[i][j][r];
                if (a.y_bf16) {
                    __bf16 h = (__bf16)v;
                    static_cast<uint16_t *>(a.Y)[row * a.ldy + col] = __builtin_bit_cast(uint16_t, h);
                } else {
                    float *y = static_cast<float *>(a.Y) + row * a.ldy + col;
                    *y = a.accumulate ? *y + v : v;
                }
            }
    }
}

typedef void (*PrefillFn)(PrefillArgs);

struct Variant {
    int mtw, nt;
};
// tile shapes with a kernel instance (block rows 64 * mtw, block columns 16 * nt)
constexpr Variant kVariants[] = {{2, 1}, {2, 2}, {2, 4}, {2, 8}, {2, 17}, {2, 20},
                                 {4, 1}, {4, 2}, {4, 4}, {4, 8}, {4, 10}};

template <int WT>
PrefillFn pick(int mtw, int nt, int *lds) {
#define TSL_CASE(MW, N)                                                                            \
    if (mtw == MW && nt == N) {                                                                    \
        *lds = Cfg<WT, MW, N>::LDS;                                                                \
        return prefill_kernel<WT, MW, N>;                                                          \
    }
    TSL_CASE(2, 1) TSL_CASE(2, 2) TSL_CASE(2, 4) TSL_CASE(2, 8) TSL_CASE(2, 17) TSL_CASE(2, 20)
    TSL_CASE(4, 1) TSL_CASE(4, 2) TSL_CASE(4, 4) TSL_CASE(4, 8) TSL_CASE(4, 10)
#undef TSL_CASE
    return nullptr;
}

// Raise a kernel's dynamic-LDS limit once per (device, kernel), so that
// later launches -- including ones recorded into a graph -- only launch.
hipError_t ensure_lds(const void *fn, int lds) {
    static std::mutex mu;
    static std::vector<std::pair<int, const void *>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto &d : done)
        if (d.first == dev && d.second == fn)
            return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
        done.emplace_back(dev, fn);
    return e;
}

} // namespace

bool prefill_supported(tsl_dtype wdtype) { return wdtype == TSL_BF16 || wdtype == TSL_Q4G64; }

PrefillPlan prefill_plan(const PackGeom &g, int64_t M) {
    // Pick the tile shape with the least modelled time on 256 CUs, one
    // workgroup per CU: rounds of tiles x tile area x an LDS-read penalty
    // (each wave reads (TM + TN) x 2 bytes per k for 2 TM TN flops; the
    // CU reads LDS at 128 B/clk and retires 4096 flop/clk).
    PrefillPlan best;
    double best_cost = 1e300;
    for (const Variant &v : kVariants) {
        const int64_t BM = 64 * v.mtw, TM = 16 * v.mtw, TN = 16 * v.nt;
        const int64_t mbk = (M + BM - 1) / BM, nbk = (g.Nt + v.nt - 1) / v.nt;
        const int64_t tiles = mbk * nbk;
        const int64_t rounds = (tiles + 255) / 256;
        const double lds = 32.0 * (double)(TM + TN) / (double)(TM * TN);
        const double cost = (double)rounds * (double)(BM * TN) * (lds > 1.0 ? lds : 1.0);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best.mtw = v.mtw;
            best.nt = v.nt;
            best.m_blocks = mbk;
            best.n_blocks = nbk;
        }
    }
    return best;
}

hipError_t launch_prefill(const PrefillPlan &p, const PackGeom &g, tsl_dtype wdtype,
                          const void *packed, const void *X, int64_t ldx, int64_t M,
                          tsl_dtype ydtype, void *Y, int64_t ldy, int accumulate,
                          hipStream_t stream) {
    PrefillArgs a{};
    a.B = packed;
    a.SB = wdtype == TSL_Q4G64
               ? reinterpret_cast<const uint32_t *>(static_cast<const char *>(packed) + g.codes_bytes)
               : nullptr;
    a.X = static_cast<const uint16_t *>(X);
    a.ldx = ldx;
    a.M = M;
    a.Ks = g.Ks;
    a.Ns = g.Ns;
    a.Nt = g.Nt;
    a.KTB = g.KT;
    a.GP = g.KT * 2;
    a.KT64 = wdtype == TSL_BF16 ? g.KT / 2 : g.Ks / 64;
    a.MB = p.m_blocks;
    a.NB = p.n_blocks;
    a.Y = Y;
    a.ldy = ldy;
    a.y_bf16 = ydtype == TSL_BF16;
    a.accumulate = accumulate;

    int lds = 0;
    PrefillFn fn = wdtype == TSL_BF16 ? pick<P_BF16>(p.mtw, p.nt, &lds) : pick<P_Q4>(p.mtw, p.nt, &lds);
    if (!fn)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    const int64_t tiles = p.m_blocks * p.n_blocks;
    hipLaunchKernelGGL(fn, dim3((unsigned)tiles), dim3(256), lds, stream, a);
    return hipGetLastError();
}

} // namespace tsl
