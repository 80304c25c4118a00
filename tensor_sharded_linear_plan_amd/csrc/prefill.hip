// Prefill-sized shard_linear: one rank's Y_i = X W_i (column / replicated
// shard) or Y_i = X_i W_i (row shard) for many token rows (wiki "Tensor
// parallel processing", "Details" §1; mlxcel manual "Tensor parallelism",
// "Column Parallel" / "Row Parallel").  A dense contraction, so it runs on
// the matrix cores with the full-rate 32x32x16 MFMA.
//
// Block tile BM x BN x 64, 4 waves arranged WM x WN, wave tile
// (BM/WM) x (BN/WN) made of 32x32 accumulator tiles.  Both operands are
// staged through LDS in MFMA fragment order (one 1 KB fragment = 32 rows or
// columns x 16 k; a lane reads its 16 bytes with one ds_read_b128), double
// buffered, one barrier per 64 k.  Inside a stage the fragments of the next
// 16-k step are read while the MFMAs of the current one run; the next
// stage's LDS writes and the global loads of the stage after it are issued
// between the MFMA groups.  Activation fragments are XOR-swizzled by k so
// that both the row-coalesced global->LDS writes and the fragment reads hit
// distinct LDS banks.
//
// Operands: bf16 x bf16, or f16 x f16 for 4-bit weights -- those are first
// dequantised into binary16 fragments (w = s q + b rounded once) by a
// pre-pass, and the bf16 activations are narrowed to binary16 while they
// are staged (exact below 65536 in magnitude).  Accumulation is binary32.
//
// The grid is one workgroup per tile, ordered so that each of the 8 XCDs
// (which receive workgroups round-robin) works on a contiguous run of
// row-major tiles and keeps those activation rows in its own L2.
#include <mutex>
#include <utility>
#include <vector>

#include "device.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

enum { OP_BF16 = 0, OP_F16 = 1 };

struct GemmArgs {
    const u32x4 *B;    // dense fragment-packed weights [Nt16][KT32][64] x 16 B
    const uint16_t *X; // bf16 activations
    int64_t ldx;
    int64_t M, Ks, Ns, Nt16;
    int64_t KT32;      // 32-k tiles per column tile in B
    int64_t KT64;      // 64-k stages to run
    int64_t MB, NB;    // tile grid
    void *Y;
    int64_t ldy;
    int y_bf16, accumulate;
};

template <int OP, int BM, int BN, int WM, int WN>
struct G {
    static constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    static constexpr int MT = TM / 32, NT = TN / 32; // 32x32 tiles per wave
    static constexpr int A_CH = BM * 8 / 256;        // 16-byte A chunks per thread per stage
    static constexpr int B_CH = (BN * 8 + 255) / 256;
    static constexpr int A_BYTES = BM * 128;          // BM x 64 k x 2 bytes
    static constexpr int B_BYTES = BN * 128;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 tiles");
    static_assert((BM * 8) % 256 == 0, "A chunks must divide over 256 threads");
};

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c, int op) {
    if (op == OP_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// LDS slot of activation chunk (row, kc) inside its fragment: logical slot
// row%32 + 32*(kc%2) XOR 2*kc (kc = 8-k chunk index 0..7 within the stage).
__device__ __forceinline__ int a_lds_offset(int row, int kc) {
    const int frag = (row >> 5) * 4 + (kc >> 1);
    const int slot = ((row & 31) + 32 * (kc & 1)) ^ (2 * kc);
    return (frag * 64 + slot) * 16;
}

template <int OP, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_kernel(GemmArgs a) {
    using C = G<OP, BM, BN, WM, WN>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const int64_t T = a.MB * a.NB;
    int64_t tile = blockIdx.x;
    if ((T & 7) == 0)
        tile = (tile & 7) * (T >> 3) + (tile >> 3);
    const int64_t mb = tile / a.NB, nb = tile % a.NB;
    const int64_t m0 = mb * BM, n0 = nb * BN;

    // ---- global -> registers ----
    // Rows past M and column tiles past the shard are clamped to the last
    // valid one: the loads stay in bounds and those outputs are never
    // stored.  Only a stage reaching past K (K % 64 != 0) takes the
    // element-wise guarded path, so every other load is unconditional.
    u32x4 ra[C::A_CH], rb[C::B_CH];
    const int64_t last_row = a.M - 1;
    auto gload = [&](int64_t kt) {
        const int64_t k0 = kt * 64;
        if (k0 + 64 <= a.Ks) {
#pragma unroll
            for (int i = 0; i < C::A_CH; ++i) {
                const int c = tid + 256 * i;
                int64_t row = m0 + (c >> 3);
                row = row < last_row ? row : last_row;
                ra[i] = *reinterpret_cast<const u32x4 *>(a.X + row * a.ldx + k0 + (c & 7) * 8);
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::A_CH; ++i) {
                const int c = tid + 256 * i;
                int64_t row = m0 + (c >> 3);
                row = row < last_row ? row : last_row;
                const int64_t k = k0 + (c & 7) * 8;
                const uint16_t *p = a.X + row * a.ldx + k;
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = (k + 2 * j < a.Ks) ? p[2 * j] : 0u;
                    const uint32_t hi = (k + 2 * j + 1 < a.Ks) ? p[2 * j + 1] : 0u;
                    w[j] = lo | (hi << 16);
                }
                ra[i] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
#pragma unroll
        for (int i = 0; i < C::B_CH; ++i) {
            const int c = tid + 256 * i;
            if (c < BN * 8) {
                int64_t t16 = (n0 >> 4) + (c >> 7); // 16-column packed tile
                t16 = t16 < a.Nt16 - 1 ? t16 : a.Nt16 - 1;
                const int64_t kt32 = kt * 2 + ((c >> 6) & 1);
                rb[i] = a.B[(t16 * a.KT32 + kt32) * 64 + (c & 63)];
            }
        }
    };
    // ---- registers -> LDS (fragment order) ----
    auto lwrite_a = [&](int stage, int i) {
        char *As = smem + stage * C::STAGE;
        const int c = tid + 256 * i;
        u32x4 v = ra[i];
        if constexpr (OP == OP_F16) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = bf16pair_to_f16pair(v[j]);
        }
        *reinterpret_cast<u32x4 *>(As + a_lds_offset(c >> 3, c & 7)) = v;
    };
    auto lwrite_b = [&](int stage, int i) {
        char *Bs = smem + stage * C::STAGE + C::A_BYTES;
        const int c = tid + 256 * i;
        if (c < BN * 8) {
            const int l16 = c & 63;
            const int n = (c >> 7) * 16 + (l16 & 15);       // column within the block
            const int kr = ((c >> 6) & 1) * 4 + (l16 >> 4); // 8-k chunk within the stage
            const int frag = (n >> 5) * 4 + (kr >> 1);
            const int slot = (n & 31) + 32 * (kr & 1);
            *reinterpret_cast<u32x4 *>(Bs + (frag * 64 + slot) * 16) = rb[i];
        }
    };
    auto lwrite = [&](int stage) {
#pragma unroll
        for (int i = 0; i < C::A_CH; ++i)
            lwrite_a(stage, i);
#pragma unroll
        for (int i = 0; i < C::B_CH; ++i)
            lwrite_b(stage, i);
    };

    f32x16 acc[C::MT][C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    // fragment readers: A fragment (mt32, s16) lane l reads logical slot l
    const int a_slot_h = lane >> 5; // k half of this lane
    auto read_frags = [&](int stage, int s, u32x4 (&af)[C::MT], u32x4 (&bf)[C::NT]) {
        const char *As = smem + stage * C::STAGE;
        const char *Bs = As + C::A_BYTES;
        const int kc = 2 * s + a_slot_h;
#pragma unroll
        for (int i = 0; i < C::MT; ++i) {
            const int frag = (wm * C::MT + i) * 4 + s;
            af[i] = *reinterpret_cast<const u32x4 *>(As + (frag * 64 + (lane ^ (2 * kc))) * 16);
        }
#pragma unroll
        for (int j = 0; j < C::NT; ++j) {
            const int frag = (wn * C::NT + j) * 4 + s;
            bf[j] = *reinterpret_cast<const u32x4 *>(Bs + (frag * 64 + lane) * 16);
        }
    };

    u32x4 af[2][C::MT], bfr[2][C::NT];
    // One 64-k stage from LDS buffer `cur`.  With `more`, the registers
    // (holding the next stage) are written to the other buffer in slices
    // between the MFMA groups of steps 1 and 2, and the stage after next is
    // fetched from memory during step 3.
    auto stage_body = [&](int cur, bool more, int64_t next2) {
        read_frags(cur, 0, af[0], bfr[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3)
                read_frags(cur, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
            int w = 0; // LDS-write slices handed out between this step's MFMAs
#pragma unroll
            for (int i = 0; i < C::MT; ++i)
#pragma unroll
                for (int j = 0; j < C::NT; ++j) {
                    acc[i][j] = mfma32(af[s & 1][i], bfr[s & 1][j], acc[i][j], OP);
                    if (more && (s == 1 || s == 2)) {
                        // spread the A+B chunk writes over steps 1 and 2
                        const int total = C::A_CH + C::B_CH;
                        const int per = (total + 2 * C::MT * C::NT - 1) / (2 * C::MT * C::NT);
                        for (int q = 0; q < per; ++q) {
                            const int idx = (s - 1) * C::MT * C::NT * per + w * per + q;
                            if (idx < C::A_CH)
                                lwrite_a(cur ^ 1, idx);
                            else if (idx < total)
                                lwrite_b(cur ^ 1, idx - C::A_CH);
                        }
                        ++w;
                    }
                }
            if (more && s == 3)
                gload(next2);
        }
    };

    gload(0);
    lwrite(0);
    if (a.KT64 > 1)
        gload(1);
    __syncthreads();

    for (int64_t kt = 0; kt + 1 < a.KT64; ++kt) {
        const int64_t next2 = kt + 2 < a.KT64 ? kt + 2 : a.KT64 - 1; // re-fetch of the last stage is harmless
        stage_body((int)(kt & 1), true, next2);
        __syncthreads();
    }
    stage_body((int)((a.KT64 - 1) & 1), false, 0);

    // ---- epilogue: acc reg r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32 ----
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        const int64_t col = n0 + (wn * C::NT + j) * 32 + (lane & 31);
        if (col >= a.Ns)
            continue;
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row =
                    m0 + (wm * C::MT + i) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
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

// 4-bit -> binary16 fragments: one thread per packed 16-byte code chunk
// (16 columns x 128 k per 64 lanes), writing the four 32-k fragments it
// covers in the dense packed layout.
__global__ void __launch_bounds__(256) dequant_f16_kernel(const u32x4 *__restrict__ codes,
                                                          const uint32_t *__restrict__ sb,
                                                          int64_t KB, int64_t GP, int64_t Gs,
                                                          int64_t chunks, u32x4 *__restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks)
        return;
    const int lane = (int)(c & 63);
    const int64_t t = c >> 6;
    const int64_t nt = t / KB, blk = t % KB;
    const u32x4 w = codes[c];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t g = 2 * blk + h;
        if (g >= Gs)
            break; // pad group of a half-filled last block: its fragments are never read
        const uint32_t p = sb[(nt * GP + g) * 16 + (lane & 15)];
        const float s = bf16_lo(p);
        const float cb = __builtin_fmaf(-1024.f, s, bf16_hi(p));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = 2 * h + q;
            const f16x8 v = q4_dequant_f16(w[tt], s, cb);
            out[((nt * (KB * 4) + blk * 4 + tt) * 64) + lane] = __builtin_bit_cast(u32x4, v);
        }
    }
}

typedef void (*GemmFn)(GemmArgs);

struct Variant {
    int bm, bn, wm, wn;
};
// tile shapes with a kernel instance
constexpr Variant kVariants[] = {{256, 160, 4, 1}, {256, 128, 2, 2}, {128, 256, 2, 2},
                                 {128, 128, 2, 2}, {256, 64, 4, 1},  {128, 64, 2, 2},
                                 {64, 64, 2, 2}};

template <int OP>
GemmFn pick(const Variant &v, int *lds) {
#define TSL_CASE(BM_, BN_, WM_, WN_)                                                               \
    if (v.bm == BM_ && v.bn == BN_ && v.wm == WM_ && v.wn == WN_) {                                \
        *lds = G<OP, BM_, BN_, WM_, WN_>::LDS;                                                     \
        return gemm_kernel<OP, BM_, BN_, WM_, WN_>;                                                \
    }
    TSL_CASE(256, 160, 4, 1) TSL_CASE(256, 128, 2, 2)
    TSL_CASE(128, 256, 2, 2) TSL_CASE(128, 128, 2, 2) TSL_CASE(256, 64, 4, 1)
    TSL_CASE(128, 64, 2, 2) TSL_CASE(64, 64, 2, 2)
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

size_t prefill_workspace_bytes(const PackGeom &g, tsl_dtype wdtype) {
    // 4-bit weights are expanded to binary16 fragments: 16 columns x 32 k
    // per KiB, k padded to whole 128-k blocks
    return wdtype == TSL_Q4G64 ? (size_t)g.Nt * (size_t)g.KT * 4 * 1024 : 0;
}

PrefillPlan prefill_plan(const PackGeom &g, int64_t M) {
    // Least modelled time on 256 CUs, one workgroup per CU: rounds of
    // tiles x padded tile area x an LDS-read penalty.  A wave reads
    // (TM + TN) x 2 bytes per k for 2 TM TN flops; a CU reads LDS at
    // 128 B/clk and retires 4096 flop/clk, so the penalty is
    // max(1, 64 (TM + TN) / (TM TN)) with 20% headroom for the LDS writes.
    PrefillPlan best;
    double best_cost = 1e300;
    const int64_t N = g.Nt * 16;
    for (const Variant &v : kVariants) {
        const int64_t TM = v.bm / v.wm, TN = v.bn / v.wn;
        const int64_t mbk = (M + v.bm - 1) / v.bm, nbk = (N + v.bn - 1) / v.bn;
        const int64_t rounds = (mbk * nbk + 255) / 256;
        const double lds = 1.2 * 64.0 * (double)(TM + TN) / (double)(TM * TN);
        const double cost = (double)rounds * (double)(v.bm * v.bn) * (lds > 1.0 ? lds : 1.0);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best.bm = v.bm;
            best.bn = v.bn;
            best.wm = v.wm;
            best.wn = v.wn;
            best.m_blocks = mbk;
            best.n_blocks = nbk;
        }
    }
    return best;
}

hipError_t launch_prefill(const PrefillPlan &p, const PackGeom &g, tsl_dtype wdtype,
                          const void *packed, const void *X, int64_t ldx, int64_t M,
                          tsl_dtype ydtype, void *Y, int64_t ldy, int accumulate, void *workspace,
                          hipStream_t stream) {
    GemmArgs a{};
    const void *B = packed;
    int op = OP_BF16;
    if (wdtype == TSL_Q4G64) {
        // expand the 4-bit shard to binary16 fragments in the workspace
        const int64_t chunks = g.Nt * g.KT * 64;
        const uint32_t *sb =
            reinterpret_cast<const uint32_t *>(static_cast<const char *>(packed) + g.codes_bytes);
        hipLaunchKernelGGL(dequant_f16_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256),
                           0, stream, static_cast<const u32x4 *>(packed), sb, g.KT, g.KT * 2,
                           g.Ks / 64, chunks, static_cast<u32x4 *>(workspace));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        B = workspace;
        op = OP_F16;
    }
    a.B = static_cast<const u32x4 *>(B);
    a.X = static_cast<const uint16_t *>(X);
    a.ldx = ldx;
    a.M = M;
    a.Ks = g.Ks;
    a.Ns = g.Ns;
    a.Nt16 = g.Nt;
    a.KT32 = wdtype == TSL_Q4G64 ? g.KT * 4 : g.KT;
    a.KT64 = (g.Ks + 63) / 64;
    a.MB = p.m_blocks;
    a.NB = p.n_blocks;
    a.Y = Y;
    a.ldy = ldy;
    a.y_bf16 = ydtype == TSL_BF16;
    a.accumulate = accumulate;

    const Variant v{p.bm, p.bn, p.wm, p.wn};
    int lds = 0;
    GemmFn fn = op == OP_BF16 ? pick<OP_BF16>(v, &lds) : pick<OP_F16>(v, &lds);
    if (!fn)
        return hipErrorInvalidValue;
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)(p.m_blocks * p.n_blocks)), dim3(256), lds, stream, a);
    return hipGetLastError();
}

} // namespace tsl
