// Decode-sized shard_linear (M <= 64 per block of rows): one rank's
// Y_i = X W_i (column / replicated shard) or Y_i = X_i W_i (row shard)
// (wiki "Tensor parallel processing", "Details" §1; mlxcel manual "Tensor
// parallelism", "Column Parallel" / "Row Parallel").
//
// The weights dominate the bytes, so every packed weight byte is streamed
// from HBM exactly once per 64 rows, as contiguous 1 KB wave loads (the
// packed layout is already in MFMA operand order), into 16x16 MFMAs.
//
// bf16 and 4-bit weights use the streaming kernel below (the 4 waves of a
// workgroup stream different column tiles over one k-range and share the
// activations through LDS).  fp32 weights, only used at small sizes, use a
// simpler kernel whose 4 waves split k and reduce in LDS.  When a call is
// too small to fill the chip, a shard's k-range is split across
// workgroups: their partials go to the workspace and a second kernel sums
// them in ascending order, so results are run-to-run deterministic.
//
// One launch serves a group of shard products with the same M and types
// (several projections, or every rank's shard of one): the item table
// rides in the kernel arguments and each workgroup finds its item by
// binary search over the items' first workgroup indices.
//
// 4-bit weights (w = s q + b per group of 64 k) are applied exactly:
// the MFMA multiplies the bf16 activations by 128 + q (an exact bf16), and
// per group the accumulator takes s * sum(x (128 + q)) + (b - 128 s) * sum(x),
// sum(x) coming from one extra MFMA against a ones operand.  This is the
// group-sum identity of the affine format, evaluated in binary32.
#include <atomic>
#include <chrono>
#include <random>
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

enum { W_F32 = 0, W_BF16 = 1, W_Q4 = 2 };

struct SkinnyItem {
    const void *B;       // packed weights
    const void *X;
    void *Y;
    float *P;            // workspace partials [ks][M][Ns] (ks > 1)
    int64_t ldx, ldy;
    int32_t Ks, Ns, Nt;
    int32_t KC;          // chunks along k (16, 32 or 128 k each)
    int32_t ks, n_groups;
    int32_t start;       // first workgroup of this item
    int32_t accumulate, y_bf16;
    int32_t fset, fpos;  // member fpos of rank-sum set fset of the launch (-1: none)
    int64_t M;           // rows of this item
    const int32_t *ridx; // row m reads X row ridx[m] (zeros outside [0, x_rows)); null: row m
    int64_t x_rows;
};

// A sum set whose rank sum the streaming launch finishes itself: member r
// (an item of the launch, ks 1) writes its binary32 product to
// P0 + r * pstride ([M][Ns], row stride Ns), and whichever wave completes
// a 16-column tile last (a counter per tile, tagged with the call's
// ticket) adds the members' tiles in rank order into Y.
struct FusedSet {
    float *P0;
    int64_t pstride;      // elements between members' products
    unsigned long long *ctr; // per 16-column tile: ticket << 16 | arrivals
    void *Y;
    int64_t ldy;
    int32_t R, y_bf16;
};
constexpr int kMaxFused = 16;

struct SkinnyGroup {
    int64_t M;
    int32_t n;
    int32_t xstr;     // streaming kernel, resident activations: LDS bytes per row
    int32_t xsum_off; // ... and LDS byte offset of the 4-bit group sums
    int32_t pad_;
    unsigned long long ticket; // 48 bits, distinct per enqueued call
    SkinnyItem it[kGroupMax];
    FusedSet fs[kMaxFused];
};

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

// ---- fp32 weights: k-split kernel ---------------------------------------
// A workgroup owns one 16-column tile and one of `ks` k-ranges; its 4 waves
// take consecutive quarters of that range, each issuing all of its weight
// loads (up to CMAX 16-k chunks) before the 16x16x4 f32 MFMAs, and the wave
// partials are summed in LDS in ascending k order.
template <int MT, int CMAX>
__global__ void __launch_bounds__(256) f32_kernel(SkinnyGroup grp) {
    constexpr int KCH = 16; // k per chunk
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
    const int64_t M = a.M;
    const int u = bid - a.start;
    const int64_t nt = u % a.n_groups;
    const int ksi = (u / a.n_groups) % a.ks;
    const int64_t m0 = (int64_t)(u / a.n_groups / a.ks) * (16 * MT);

    // this wave's chunk range
    const int64_t S = (int64_t)a.ks * 4;
    const int64_t wg = (int64_t)ksi * 4 + wave;
    const int64_t c0 = wg * a.KC / S;
    const int64_t c1 = (wg + 1) * a.KC / S;
    const int nc = (int)(c1 - c0); // <= CMAX, guaranteed by the host plan

    // 1. issue every weight load of this wave
    u32x4 breg[CMAX];
    const u32x4 *B = static_cast<const u32x4 *>(a.B);
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
        u32x4 v = {0, 0, 0, 0};
        if (c < nc)
            v = B[(nt * a.KC + c0 + c) * 64 + lane];
        breg[c] = v;
    }

    // 2. multiply
    f32x4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t arow = m0 + (lane & 15);
    const int kg = lane >> 4; // which run of k this lane feeds
    const float *X = static_cast<const float *>(a.X);
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
        if (c < nc) {
            const int64_t kb = (c0 + c) * KCH;
            f32x4 xa[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                xa[i] = load_x_f32(X, a.ldx, arow + 16 * i, M, kb + 4 * kg, a.Ks);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float b = __uint_as_float(breg[c][t]);
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[i] = mfma_f32(xa[i][t], b, acc[i]);
            }
        }
    }

    // 3. sum the 4 wave partials in ascending k order (wave 0 first)
    __shared__ f32x4 red[3][MT][64];
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
            red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const f32x4 v = red[w][i][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[i][r] = acc[i][r] + v[r];
        }

    // 4. write: lane holds rows 4 * (lane / 16) + r of column lane % 16
    const int64_t col = nt * 16 + (lane & 15);
    if (col >= a.Ns)
        return;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + 16 * i + 4 * kg + r;
            if (row >= M)
                continue;
            const float v = acc[i][r];
            if (a.ks > 1) {
                a.P[((int64_t)ksi * M + row) * a.Ns + col] = v;
            } else if (a.y_bf16) {
                __bf16 h = (__bf16)v;
                static_cast<uint16_t *>(a.Y)[row * a.ldy + col] = __builtin_bit_cast(uint16_t, h);
            } else {
                float *y = static_cast<float *>(a.Y) + row * a.ldy + col;
                *y = a.accumulate ? *y + v : v;
            }
        }
}

// ---- streaming decode kernel (bf16 and 4-bit weights) ----------------------
// A workgroup's 4 waves take 4 x NTW different 16-column tiles over one
// k-range and share the activations through LDS; every wave keeps the
// weight loads of the next two blocks (BK k each) in flight in a 3-deep
// register ring.  Each wave owns whole output tiles, so there is no
// cross-wave reduction.
//   XRES (M <= 4): the workgroup's activation rows for its whole k-range are
//     copied into LDS once; the block loop then has no barrier at all.
//   otherwise: activation blocks of 16 MT rows x BK are staged through a
//     double-buffered LDS window, loaded two blocks ahead like the weights
//     and published with one barrier per block (rows padded by 16 bytes so
//     the fragment reads do not conflict).

// Barrier that publishes LDS writes only: the compiler's __syncthreads
// also waits for every outstanding global load, which would drain the
// weight prefetch each block.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// k per block of the streaming kernel: 2 (16-byte) weight loads per tile
// per block
constexpr int stream_bk(int wt) { return wt == W_Q4 ? 256 : 64; }

// Rows whose activations stay resident in LDS for a whole k-range.
constexpr int64_t kResidentRows = 4;
// LDS a workgroup may use for resident activations.
constexpr int64_t kResidentBytes = 40 * 1024;

template <int WT, int MT>
struct SB {
    static constexpr int BK = stream_bk(WT);
    static constexpr int LPB = WT == W_Q4 ? BK / 128 : BK / 32; // 16-byte loads per tile
    static constexpr int ROWS = 16 * MT;
    static constexpr int XROW = BK * 2 + 16;                     // LDS row bytes (window)
    static constexpr int UNITS = ROWS * (BK / 8);                // 16-byte x units per block
    static constexpr int XU = (UNITS + 255) / 256;               // per thread
};

// ONE: a single token row (M == 1, resident activations): only the first
// accumulator row of each lane is ever stored, so the group epilogue
// updates that one alone.
template <int WT, int MT, int NTW, bool XRES, bool ONE = false, bool IDX = false>
__global__ void __launch_bounds__(256) stream_kernel(SkinnyGroup grp) {
    // IDX: items may read their rows through an index; only resident
    // kernels stage rows that way (once per workgroup, through xload)
    static_assert(!IDX || XRES, "rows through an index need the resident kernel");
    using S = SB<WT, MT>;
    // XRES: [M rows][xstr bytes] sized at launch; else two [ROWS][XROW] windows
    extern __shared__ __attribute__((aligned(16))) char xl[];
    const int lane = threadIdx.x & 63;
    // wave-uniform: tile and record addresses stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int64_t M = a.M;
    const int u = bid - a.start;
    const int tg = u % a.n_groups;
    const int ksi = (u / a.n_groups) % a.ks;
    const int64_t m0 = (int64_t)(u / a.n_groups / a.ks) * S::ROWS;
    const int kg = lane >> 4; // k-run of this lane in a 32-k step
    const int nblk = (a.Ks + S::BK - 1) / S::BK;
    const int b0 = (int)((int64_t)ksi * nblk / a.ks);
    const int b1 = (int)((int64_t)(ksi + 1) * nblk / a.ks);

    // this wave's tiles (clamped in range; tiles past the shard are not
    // stored): a chunk is one 16-byte load per lane, and for 4-bit weights
    // the (scale, bias) pairs of its two groups follow it in the same record
    constexpr int64_t CS = WT == W_Q4 ? kQ4Record : 1024; // bytes per chunk
    const char *wsrc[NTW];
    int64_t ntile[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        ntile[j] = ((int64_t)tg * 4 + wave) * NTW + j;
        const int64_t nt = ntile[j] < a.Nt - 1 ? ntile[j] : a.Nt - 1;
        wsrc[j] = static_cast<const char *>(a.B) + nt * (int64_t)a.KC * CS;
    }

    // weight ring: [slot][tile][load], plus scale/bias pairs for 4-bit
    u32x4 cw[3][NTW][S::LPB];
    u32x2 sbw[3][NTW][S::LPB];
    auto load_w = [&](auto SLOT, int b) __attribute__((always_inline)) {
        constexpr int s = decltype(SLOT)::value;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int l = 0; l < S::LPB; ++l) {
                const int c = b * S::LPB + l; // chunk (4-bit) or 32-k tile (bf16)
                const int cc = c < a.KC ? c : a.KC - 1;
                const char *rec = wsrc[j] + (int64_t)cc * CS;
                cw[s][j][l] = *reinterpret_cast<const u32x4 *>(rec + lane * 16);
                if constexpr (WT == W_Q4) // both groups of the chunk in one load
                    sbw[s][j][l] =
                        *reinterpret_cast<const u32x2 *>(rec + kQ4PairsAt + (lane & 15) * 8);
            }
    };

    // where row `row` of the product reads X: row ridx[row] when the item
    // reads its rows through an index (null for an index outside
    // [0, x_rows): a row of zeros)
    const uint16_t *X = static_cast<const uint16_t *>(a.X);
    auto xsrc = [&](int64_t row) __attribute__((always_inline)) -> const uint16_t * {
        const int64_t s = a.ridx[row];
        return s >= 0 && s < a.x_rows ? X + s * a.ldx : nullptr;
    };
    // 16 bytes of activations: row m0 + r, k .. k + 7 (zero past M and K)
    auto xload = [&](int64_t r, int64_t k) __attribute__((always_inline)) {
        const int64_t row = m0 + r;
        u32x4 v = {0, 0, 0, 0};
        if (row < M) {
            const uint16_t *p = X + row * a.ldx + k;
            if constexpr (IDX) {
                if (a.ridx) {
                    const uint16_t *x0 = xsrc(row);
                    if (!x0)
                        return v;
                    p = x0 + k;
                }
            }
            if (k + 8 <= a.Ks) {
                v = *reinterpret_cast<const u32x4 *>(p);
            } else if (k < a.Ks) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t l0 = k + 2 * e < a.Ks ? p[2 * e] : 0u;
                    const uint32_t h0 = k + 2 * e + 1 < a.Ks ? p[2 * e + 1] : 0u;
                    v[e] = l0 | (h0 << 16);
                }
            }
        }
        return v;
    };

    // window mode: x ring in registers, matching the weight ring slots
    constexpr int XU = XRES ? 1 : S::XU;
    u32x4 xr[3][XU];
    auto load_x = [&](auto SLOT, int b) __attribute__((always_inline)) {
        constexpr int s = decltype(SLOT)::value;
#pragma unroll
        for (int i = 0; i < XU; ++i) {
            const int unit = threadIdx.x + 256 * i;
            const int r = unit / (S::BK / 8), cu = unit % (S::BK / 8);
            xr[s][i] = unit < S::UNITS ? xload(r, (int64_t)b * S::BK + cu * 8) : u32x4{0, 0, 0, 0};
        }
    };
    // the same for a block that lies wholly inside K: every lane issues one
    // 16-byte load (rows past M and units past the window read clamped,
    // in-bounds addresses; those rows are then zero, those units unused),
    // so every steady-state step issues the same loads
    auto load_x_whole = [&](auto SLOT, int b) __attribute__((always_inline)) {
        constexpr int s = decltype(SLOT)::value;
#pragma unroll
        for (int i = 0; i < XU; ++i) {
            const int u0 = threadIdx.x + 256 * i;
            const int unit = u0 < S::UNITS ? u0 : S::UNITS - 1;
            const int r = unit / (S::BK / 8), cu = unit % (S::BK / 8);
            const int64_t row = m0 + r;
            const int64_t rr = row < M ? row : M - 1;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                X + rr * a.ldx + (int64_t)b * S::BK + cu * 8);
            xr[s][i] = row < M ? v : u32x4{0, 0, 0, 0};
        }
    };
    auto store_x = [&](auto SLOT, int buf) __attribute__((always_inline)) {
        constexpr int s = decltype(SLOT)::value;
#pragma unroll
        for (int i = 0; i < XU; ++i) {
            const int unit = threadIdx.x + 256 * i;
            if (unit < S::UNITS) {
                const int r = unit / (S::BK / 8), cu = unit % (S::BK / 8);
                *reinterpret_cast<u32x4 *>(&xl[(buf * S::ROWS + r) * S::XROW + cu * 16]) =
                    xr[s][i];
            }
        }
    };

    f32x4 acc[MT][NTW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int kr0 = b0 * S::BK;
    // resident rows past M read row M - 1 (finite; those outputs are not stored)
    const int xrow = XRES ? ((lane & 15) < M - m0 ? (lane & 15) : (int)(M - m0) - 1) : 0;
    // XRES, 4-bit: per 64-k group of the k-range, the sum of each row's
    // activations ([group][16 rows] binary32, rows past M zero)
    float *xsum = reinterpret_cast<float *>(xl + grp.xsum_off);
    auto xfrag = [&](int buf, int i, int b, int k) __attribute__((always_inline)) {
        if constexpr (XRES) {
            return *reinterpret_cast<const bf16x8 *>(
                &xl[xrow * grp.xstr + ((int64_t)b * S::BK + k + 8 * kg - kr0) * 2]);
        } else {
            const int r = 16 * i + (lane & 15);
            return *reinterpret_cast<const bf16x8 *>(
                &xl[(buf * S::ROWS + r) * S::XROW + (k + 8 * kg) * 2]);
        }
    };

    auto compute = [&](auto SLOT, int buf, int b) __attribute__((always_inline)) {
        constexpr int s = decltype(SLOT)::value;
        if constexpr (WT == W_BF16) {
#pragma unroll
            for (int l = 0; l < S::LPB; ++l) {
                bf16x8 xa[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    xa[i] = xfrag(buf, i, b, 32 * l);
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int i = 0; i < MT; ++i)
                        acc[i][j] = mfma_bf16(xa[i], __builtin_bit_cast(bf16x8, cw[s][j][l]),
                                              acc[i][j]);
            }
        } else {
            const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u,
                                                                 0x3F803F80u, 0x3F803F80u});
#pragma unroll
            for (int l = 0; l < S::LPB; ++l) { // 128-k chunk = 2 groups of 64
                if (b * S::LPB + l >= a.KC)
                    break; // odd chunk count: the block's second chunk is past K
                f32x4 xs[MT], ag[MT][NTW];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    bf16x8 xa[MT];
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        xa[i] = xfrag(buf, i, b, 128 * l + 32 * t);
                        if constexpr (XRES) { // group sums precomputed in LDS
                            if (t & 1) {
                                const int gl = (b * S::BK + 128 * l + 64 * (t >> 1) - kr0) / 64;
                                xs[i] = *reinterpret_cast<const f32x4 *>(
                                    &xsum[gl * 16 + 4 * kg]);
                            }
                        } else {
                            xs[i] = mfma_bf16(xa[i], ones,
                                              (t & 1) ? xs[i] : f32x4{0.f, 0.f, 0.f, 0.f});
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const bf16x8 bq = q4_to_bf16_plus128(cw[s][j][l][t]);
#pragma unroll
                        for (int i = 0; i < MT; ++i)
                            ag[i][j] = mfma_bf16(xa[i], bq,
                                                 (t & 1) ? ag[i][j] : f32x4{0.f, 0.f, 0.f, 0.f});
                    }
                    if (t & 1) { // end of a group: y += s sum(x (128 + q)) + (b - 128 s) sum(x)
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            const uint32_t sbp = sbw[s][j][l][t >> 1];
                            const float sc = bf16_lo(sbp);
                            const float cb = __builtin_fmaf(-128.f, sc, bf16_hi(sbp));
#pragma unroll
                            for (int i = 0; i < MT; ++i)
#pragma unroll
                                for (int r = 0; r < (ONE ? 1 : 4); ++r) {
                                    acc[i][j][r] = __builtin_fmaf(sc, ag[i][j][r], acc[i][j][r]);
                                    acc[i][j][r] = __builtin_fmaf(cb, xs[i][r], acc[i][j][r]);
                                }
                        }
                    }
                }
            }
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // one block in slot SLOT: prefetch block b + 2 into slot NEXT2, compute b,
    // (window mode) publish the activations of b + 1 from slot NEXT1
    // FULL: a steady-state step, b + 2 < b1 known -- every such step issues
    // the same loads, so the wait counts the compiler derives at the loop
    // head are exact (with a conditional prefetch it must assume the path
    // that issued none and waits for nearly every load in flight)
    auto step = [&](auto SLOT, auto NEXT1, auto NEXT2, int b, auto FULL)
                    __attribute__((always_inline)) {
        constexpr bool full = decltype(FULL)::value;
        const int buf = (b - b0) & 1;
        if (full || b + 2 < b1) {
            if constexpr (!XRES) {
                if constexpr (full)
                    load_x_whole(NEXT2, b + 2);
                else
                    load_x(NEXT2, b + 2);
            }
            load_w(NEXT2, b + 2);
        }
        compute(SLOT, buf, b);
        if constexpr (!XRES) {
            if (full || b + 1 < b1)
                store_x(NEXT1, buf ^ 1);
            lds_barrier();
        }
    };
    using Full = std::true_type;
    using Tail = std::false_type;

    if (b0 < b1) {
        if constexpr (XRES) {
            load_w(I0{}, b0);
            if (b0 + 1 < b1)
                load_w(I1{}, b0 + 1);
            // activation rows [m0, M) x [kr0, b1 BK) into LDS, 4 units per
            // thread per round, zero past K
            const int64_t rows = M - m0;
            const int per_row = (b1 - b0) * (S::BK / 8);
            const int units = (int)rows * per_row;
            for (int base = 0; base < units; base += 1024) {
                u32x4 v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int unit = base + 256 * q + threadIdx.x;
                    v[q] = unit < units ? xload(unit / per_row, kr0 + (int64_t)(unit % per_row) * 8)
                                        : u32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int unit = base + 256 * q + threadIdx.x;
                    if (unit < units)
                        *reinterpret_cast<u32x4 *>(
                            &xl[(unit / per_row) * grp.xstr + (unit % per_row) * 16]) = v[q];
                }
            }
            if constexpr (WT == W_Q4) {
                lds_barrier();
                const int groups = (b1 - b0) * (S::BK / 64);
                const int nr = (int)rows; // resident rows, 1 .. kResidentRows
                // rows past M sum to zero (their outputs are never stored)
                for (int e = threadIdx.x; e < groups * 16; e += 256)
                    if ((e & 15) >= nr)
                        xsum[e] = 0.f;
                // each (group, row) entry: 8 lanes add 8 activations each,
                // then a butterfly over those 8 lanes
                const int sub = threadIdx.x & 7;
                for (int ent = threadIdx.x >> 3; ent < groups * nr; ent += 32) {
                    const int g = ent / nr, r = ent - g * nr;
                    const u32x4 v =
                        *reinterpret_cast<const u32x4 *>(&xl[r * grp.xstr + g * 128 + sub * 16]);
                    float sum = (bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y));
                    sum += (bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w));
                    sum += __shfl_xor(sum, 1, 8);
                    sum += __shfl_xor(sum, 2, 8);
                    sum += __shfl_xor(sum, 4, 8);
                    if (sub == 0)
                        xsum[g * 16 + r] = sum;
                }
            }
        } else {
            load_x(I0{}, b0);
            load_w(I0{}, b0);
            if (b0 + 1 < b1) {
                load_x(I1{}, b0 + 1);
                load_w(I1{}, b0 + 1);
            }
            store_x(I0{}, 0);
        }
        lds_barrier();
        int b = b0;
        // steady state: the three steps prefetch blocks up to b + 4, all
        // inside the k-range and (window mode) wholly inside K.  Not for
        // 64-row tiles, where the scheduler spreads the prefetches through
        // the MFMA stream and the conditional form measured faster.
        const int bsteady = MT > 2 ? b0 : XRES ? b1 : (b1 < a.Ks / S::BK ? b1 : a.Ks / S::BK);
        for (; b + 5 <= bsteady; b += 3) {
            step(I0{}, I1{}, I2{}, b, Full{});
            step(I1{}, I2{}, I0{}, b + 1, Full{});
            step(I2{}, I0{}, I1{}, b + 2, Full{});
        }
        for (; b + 3 <= b1; b += 3) {
            step(I0{}, I1{}, I2{}, b, Tail{});
            step(I1{}, I2{}, I0{}, b + 1, Tail{});
            step(I2{}, I0{}, I1{}, b + 2, Tail{});
        }
        if (b < b1)
            step(I0{}, I1{}, I2{}, b, Tail{});
        if (b + 1 < b1)
            step(I1{}, I2{}, I0{}, b + 1, Tail{});
    }

    // acc[i][j] lane l: rows 16 i + 4 (l / 16) + r, column l % 16 of tile j
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int64_t col = ntile[j] * 16 + (lane & 15);
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
                } else if (a.fset >= 0) { // a set member's product: written through
                    __hip_atomic_store(static_cast<float *>(a.Y) + row * a.ldy + col, v,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    if (a.fset < 0)
        return;

    // Rank-sum set member: this wave's partial tiles are stored (a.Y is the
    // member's binary32 product, written with agent-scope stores, which go
    // through to the point of coherence of all XCDs); once they have
    // completed, count the arrival, and the last member to arrive at a tile
    // adds the R products in rank order, read with agent-scope loads.  (An
    // agent-scope fence would write back and invalidate the whole L2 of the
    // XCD at every member wave.)  The counter word is ticket << 16 |
    // arrivals; a word tagged with another ticket (an earlier call, or
    // never written) counts as zero, and the last arrival leaves ticket <<
    // 16 | 0, so a replay of the same enqueued call starts from zero too.
    //
    // Ordering, on gfx950's instructions rather than C++ acquire/release
    // (which would cost the L2 write-back and invalidate above): the
    // partials are "global_store_dword ... sc1" (written through to the
    // device-coherent level); "s_waitcnt vmcnt(0)" below returns only once
    // those stores are acknowledged there; the counter update is a device-
    // scope "global_atomic_cmpswap_x2", performed at that same level after
    // the wait; the last arrival's reads are "global_load_dword ... sc1"
    // (they miss the non-coherent L2) and issue only after its swap has
    // returned, behind a branch on the swap's result.  So every member's
    // stores are visible before the count that admits the last arrival,
    // and that arrival's reads come after it.
    const FusedSet &fs = grp.fs[a.fset];
    const unsigned long long tag = grp.ticket << 16;
    const int64_t mb = m0 / (16 * MT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): the product stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        if (ntile[j] >= a.Nt)
            continue; // a clamped duplicate tile of the last column group
        unsigned long long *ctr = fs.ctr + mb * a.Nt + ntile[j];
        int last = 0;
        if (lane == 0) {
            // A failed swap means another member's swap on this word
            // succeeded in between (the word changes only by a member's
            // increment or the last arrival's reset, which follows every
            // increment of this call), so the loop ends after at most R - 1
            // failures; it never gives up, since a lost arrival would leave
            // the tile's sum unwritten.
            unsigned long long old = __hip_atomic_load(ctr, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            for (;;) {
                const unsigned long long base = (old & ~0xFFFFull) == tag ? old : tag;
                if (__hip_atomic_compare_exchange_strong(ctr, &old, base + 1, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)) {
                    last = (int)((base + 1) & 0xFFFF) == fs.R;
                    break;
                }
            }
        }
        last = __builtin_amdgcn_readfirstlane(__shfl(last, 0));
        if (!last)
            continue;
        const int64_t col = ntile[j] * 16 + (lane & 15);
        if (col < a.Ns) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = m0 + 16 * i + 4 * kg + r;
                    if (row >= M)
                        continue;
                    float *p = fs.P0 + row * a.Ns + col;
                    float v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    for (int q = 1; q < fs.R; ++q)
                        v = v + __hip_atomic_load(p + q * fs.pstride, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                    if (fs.y_bf16) {
                        __bf16 h = (__bf16)v;
                        static_cast<uint16_t *>(fs.Y)[row * fs.ldy + col] =
                            __builtin_bit_cast(uint16_t, h);
                    } else {
                        static_cast<float *>(fs.Y)[row * fs.ldy + col] = v;
                    }
                }
        }
        if (lane == 0)
            __hip_atomic_store(ctr, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

typedef void (*SkinnyFn)(SkinnyGroup);

// 48-bit tickets, distinct for every enqueued streaming launch of the
// process (a random start, then consecutive)
unsigned long long next_ticket() {
    static std::atomic<unsigned long long> next{[] {
        std::random_device rd;
        return ((unsigned long long)rd() << 32) ^ (unsigned long long)rd() ^
               (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    }()};
    return next.fetch_add(1) & ((1ull << 48) - 1);
}

// fp32 weights: the k-split kernel (4 waves split k, LDS reduction)
SkinnyFn pick_f32(int mt) {
    switch (mt) {
    case 1: return f32_kernel<1, 16>;
    case 2: return f32_kernel<2, 16>;
    default: return f32_kernel<4, 16>;
    }
}

template <int WT, int MT>
SkinnyFn pick_stream_ntw(int ntw) {
    return ntw == 1 ? stream_kernel<WT, MT, 1, false> : stream_kernel<WT, MT, 2, false>;
}

template <int WT>
SkinnyFn pick_stream(int mt, int ntw, bool resident, bool one, bool idx) {
    if (resident && idx) // some item reads its rows through an index
        return one && ntw == 1 ? stream_kernel<WT, 1, 1, true, true, true>
               : ntw == 1      ? stream_kernel<WT, 1, 1, true, false, true>
                               : stream_kernel<WT, 1, 2, true, false, true>;
    if (resident && one && ntw == 1)
        return stream_kernel<WT, 1, 1, true, true>;
    if (resident)
        return ntw == 1 ? stream_kernel<WT, 1, 1, true> : stream_kernel<WT, 1, 2, true>;
    switch (mt) {
    case 1: return pick_stream_ntw<WT, 1>(ntw);
    case 2: return pick_stream_ntw<WT, 2>(ntw);
    default: return pick_stream_ntw<WT, 4>(ntw);
    }
}

} // namespace

SkinnyPlan skinny_plan(const LinearItem *items, int n, tsl_dtype wdtype, int64_t M) {
    SkinnyPlan p;
    const int64_t rows = M < 64 ? M : 64;
    p.mt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
    p.m_blocks.resize(n);
    for (int i = 0; i < n; ++i)
        p.m_blocks[i] = (items[i].M + 16 * p.mt - 1) / (16 * p.mt);
    p.stream = wdtype != TSL_F32;
    p.ks.resize(n);
    p.ws_off.resize(n);
    p.n_groups.resize(n);
    if (p.stream) {
        // 4 waves x NTW tiles per workgroup, each wave over the whole k-range;
        // k split across workgroups only when the group is too small to put
        // ~2 workgroups on every CU.  Two tiles per wave halve the
        // activation reads per weight byte: for more than 16 rows always,
        // for 5..16 rows when the group still has >= 8 workgroups per CU
        int64_t wg1 = 0;
        for (int i = 0; i < n; ++i)
            wg1 += (items[i].g.Nt + 3) / 4 * p.m_blocks[i];
        p.ntw = rows > 16 || (rows > 4 && wg1 >= 2048) ? 2 : 1;
        const int bk = stream_bk(wdtype == TSL_Q4G64 ? W_Q4 : W_BF16);
        int64_t base = 0;
        for (int i = 0; i < n; ++i) {
            p.n_groups[i] = (items[i].g.Nt + 4 * p.ntw - 1) / (4 * p.ntw);
            base += p.n_groups[i] * p.m_blocks[i];
        }
        const int64_t ks_want = base > 0 ? (512 + base - 1) / base : 1;
        for (int i = 0; i < n; ++i) {
            const int64_t nblk = (items[i].g.Ks + bk - 1) / bk;
            const int64_t cap = nblk / 2 > 1 ? nblk / 2 : 1;
            p.ks[i] = (int)(ks_want < cap ? ks_want : cap);
        }
        // few rows: each workgroup keeps its activations for its whole
        // k-range in LDS (no barrier in the block loop)
        int64_t span = 0;
        for (int i = 0; i < n; ++i) {
            const int64_t nblk = (items[i].g.Ks + bk - 1) / bk;
            const int64_t per = (nblk + p.ks[i] - 1) / p.ks[i] + 1; // blocks of a k-range
            span = per * bk > span ? per * bk : span;
        }
        const int64_t xstr = span * 2 + 16;
        const int64_t xsum = wdtype == TSL_Q4G64 ? span / 64 * 16 * 4 : 0;
        if (M <= kResidentRows && M * xstr + xsum <= kResidentBytes) {
            p.resident = true;
            p.xstr = (int)xstr;
            p.xsum_off = (int)((M * xstr + 15) / 16 * 16);
            p.lds_bytes = (size_t)p.xsum_off + (size_t)xsum;
        } else {
            p.lds_bytes = 2 * (size_t)(16 * p.mt) * (size_t)(bk * 2 + 16);
        }
    } else {
        // fp32: a workgroup owns one 16-column tile and one k-range split
        // over its 4 waves; k split further for ~1024 workgroups (and as far
        // as the register budget of a wave requires)
        p.ntw = 1;
        p.cmax = 16;
        int64_t base = 0;
        for (int i = 0; i < n; ++i) {
            p.n_groups[i] = items[i].g.Nt;
            base += p.n_groups[i] * p.m_blocks[i];
        }
        const int64_t ks_want = base > 0 ? (1024 + base - 1) / base : 1;
        for (int i = 0; i < n; ++i) {
            const int64_t KC = items[i].g.KT;
            const int64_t ks_min = (KC + 4 * p.cmax - 1) / (4 * p.cmax);
            const int64_t ks_cap = KC / 4 > 1 ? KC / 4 : 1;
            int64_t ks = ks_want < ks_cap ? ks_want : ks_cap;
            p.ks[i] = (int)(ks < ks_min ? ks_min : ks);
        }
    }
    size_t off = 0;
    for (int i = 0; i < n; ++i) {
        p.ws_off[i] = off;
        if (p.ks[i] > 1)
            off += ((size_t)p.ks[i] * (size_t)items[i].M * (size_t)items[i].g.Ns * sizeof(float) +
                    255) / 256 * 256;
    }
    // sum sets the streaming launch finishes: resident launches (a few token
    // rows; with more rows the written-through products and their reads
    // cost more than the separate sum launch, measured), every member
    // unsplit and in the same launch, at most kMaxFused per launch; a
    // counter per (row block, 16-column tile)
    p.fset.assign(n, -1);
    int in_chunk = 0, chunk = -1;
    for (int i = 0; p.stream && p.resident && i < n;) {
        const int len = items[i].fset_len;
        if (len < 2 || items[i].fset_pos != 0) {
            ++i;
            continue;
        }
        bool ok = i + len <= n && len <= kSetParts && i / kGroupMax == (i + len - 1) / kGroupMax;
        for (int r = 0; ok && r < len; ++r)
            ok = p.ks[i + r] == 1 && items[i + r].fset_pos == r;
        if (i / kGroupMax != chunk) {
            chunk = i / kGroupMax;
            in_chunk = 0;
        }
        if (ok && in_chunk < kMaxFused) {
            SkinnyPlan::FSet f;
            f.first = i;
            f.len = len;
            f.ctr_off = off;
            off += ((size_t)p.m_blocks[i] * (size_t)items[i].g.Nt * 8 + 255) / 256 * 256;
            for (int r = 0; r < len; ++r)
                p.fset[i + r] = (int)p.fsets.size();
            p.fsets.push_back(f);
            ++in_chunk;
        }
        i += len;
    }
    p.ws_bytes = off;
    return p;
}

int64_t skinny_blocks(const SkinnyPlan &p, const LinearItem *items, int n) {
    (void)items;
    int64_t most = 0;
    for (int c0 = 0; c0 < n; c0 += kGroupMax) {
        int64_t blocks = 0;
        for (int i = c0; i < n && i < c0 + kGroupMax; ++i)
            blocks += p.n_groups[i] * p.ks[i] * p.m_blocks[i];
        most = blocks > most ? blocks : most;
    }
    return most;
}

hipError_t launch_skinny(const SkinnyPlan &p, const LinearItem *items, int n, tsl_dtype wdtype,
                         int64_t M, void *workspace, hipStream_t stream) {
    // items read through a row index only in resident calls (the caller
    // gathers the rows of the others)
    bool idx = false;
    for (int i = 0; i < n; ++i)
        idx = idx || items[i].ridx != nullptr;
    if (idx && (!p.stream || !p.resident))
        return hipErrorInvalidValue;
    SkinnyFn fn = wdtype == TSL_F32    ? pick_f32(p.mt)
                  : wdtype == TSL_BF16 ? pick_stream<W_BF16>(p.mt, p.ntw, p.resident, M == 1, idx)
                                       : pick_stream<W_Q4>(p.mt, p.ntw, p.resident, M == 1, idx);
    if (!fn)
        return hipErrorInvalidValue;
    for (int c0 = 0; c0 < n; c0 += kGroupMax) {
        const int cn = n - c0 < kGroupMax ? n - c0 : kGroupMax;
        SkinnyGroup grp{};
        grp.M = M;
        grp.n = cn;
        grp.xstr = p.xstr;
        grp.xsum_off = p.xsum_off;
        grp.ticket = next_ticket();
        // this launch's finished sum sets, in plan order
        int nfs = 0, fs0 = -1;
        for (size_t f = 0; f < p.fsets.size(); ++f) {
            const SkinnyPlan::FSet &F = p.fsets[f];
            if (F.first < c0 || F.first >= c0 + cn)
                continue;
            if (fs0 < 0)
                fs0 = (int)f;
            const LinearItem &L0 = items[F.first];
            FusedSet &d = grp.fs[nfs++];
            d.P0 = static_cast<float *>(L0.Y);
            d.pstride = F.len > 1 ? (static_cast<const float *>(items[F.first + 1].Y) -
                                     static_cast<const float *>(L0.Y))
                                  : 0;
            d.ctr = reinterpret_cast<unsigned long long *>(static_cast<char *>(workspace) +
                                                           F.ctr_off);
            d.Y = L0.fset_Y;
            d.ldy = L0.fset_ldy;
            d.R = F.len;
            d.y_bf16 = L0.fset_ydtype == TSL_BF16;
            // the members' products lie at equal strides (split_sets)
            for (int r = 1; r < F.len; ++r)
                if (static_cast<const float *>(items[F.first + r].Y) !=
                    d.P0 + r * d.pstride)
                    return hipErrorInvalidValue;
        }
        int64_t blocks = 0;
        for (int i = 0; i < cn; ++i) {
            const LinearItem &L = items[c0 + i];
            SkinnyItem &a = grp.it[i];
            a.B = L.packed;
            a.X = L.X;
            a.ridx = L.ridx;
            a.x_rows = L.x_rows;
            a.Y = L.Y;
            a.P = reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_off[c0 + i]);
            a.ldx = L.ldx;
            a.ldy = L.ldy;
            a.Ks = (int32_t)L.g.Ks;
            a.Ns = (int32_t)L.g.Ns;
            a.Nt = (int32_t)L.g.Nt;
            a.KC = (int32_t)L.g.KT;
            a.ks = p.ks[c0 + i];
            a.n_groups = (int32_t)p.n_groups[c0 + i];
            a.accumulate = L.accumulate;
            a.y_bf16 = L.ydtype == TSL_BF16;
            a.M = L.M;
            a.fset = p.fset[c0 + i] < 0 ? -1 : p.fset[c0 + i] - fs0;
            a.fpos = L.fset_pos;
            a.start = (int32_t)blocks;
            blocks += (int64_t)a.n_groups * a.ks * p.m_blocks[c0 + i];
        }
        if (p.lds_bytes > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)p.lds_bytes);
            if (e != hipSuccess)
                return e;
        }
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), p.lds_bytes, stream, grp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        // k-partials of products that accumulate into Y or belong to a sum
        // set too long for one sum launch; the others' are added by the
        // caller's one sum launch
        for (int i = 0; i < cn; ++i) {
            const SkinnyItem &a = grp.it[i];
            if (a.ks == 1 || !(a.accumulate || items[c0 + i].no_split))
                continue;
            e = launch_splitk_reduce(a.P, a.ks, a.M, a.Ns, items[c0 + i].ydtype, a.Y, a.ldy,
                                     a.accumulate, stream);
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

} // namespace tsl
