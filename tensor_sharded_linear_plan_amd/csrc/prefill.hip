// Prefill-sized shard_linear: one rank's Y_i = X W_i (column / replicated
// shard) or Y_i = X_i W_i (row shard) for many token rows (wiki "Tensor
// parallel processing", "Details" §1; mlxcel manual "Tensor parallelism",
// "Column Parallel" / "Row Parallel").  A dense contraction, so it runs on
// the matrix cores with the full-rate 32x32x16 MFMA.
//
// Block tile BM x BN, 4 waves arranged WM x WN, wave tile (BM/WM) x
// (BN/WN) made of 32x32 accumulator tiles.  Operands move from global
// memory straight into LDS with gfx950's global_load_lds_dwordx4 (a wave
// instruction fills 1 KB of LDS, lane l at byte 16 l), so staging costs no
// VGPRs and no LDS write instructions:
//   - activations: one instruction fetches whole 128- or 64-byte row
//     segments into an LDS block whose 16-byte chunks are XOR-swizzled by
//     row, which keeps the MFMA fragment reads bank-conflict free;
//   - weights: the packed layout already holds 16 columns x 8 k per
//     16-byte chunk, so a 32-column x 16-k MFMA fragment is two 512-byte
//     runs.
// A stage covers 64 k (32 k when three 64-k stages would not fit in 160 KB)
// and stages rotate through S <= 4 LDS slots (5 of 32 k).  Fragment reads run one 16-k
// step ahead of the MFMAs.  The barrier that publishes stage k + 1 sits
// before the last 16-k step of stage k: each wave first waits for its own
// copies of stage k + 1 and for its own reads of stage k; after the barrier
// it reads the first fragments of stage k + 1 and, between the MFMAs of the
// last step of stage k, issues the copies of stage k + S into the slot of
// stage k, which no wave reads any more.
//
// Operands: bf16 x bf16, accumulated in binary32.  bf16 activations are
// copied, zero-padded, only when K is not a multiple of 64.  4-bit weights
// run in q4gemm.hip's fused kernel; this file also holds what the two share:
// the activation pass (which for 4-bit weights writes each distinct
// activation matrix once as binary16, every row scaled by a power of two),
// the tile-shape cost model and the launch sequence.
//
// One launch serves a group of shard products of the same types, each over
// its own rows; the item table rides in the kernel arguments.  Each item's
// tiles take a run of workgroups right after the previous item's.
// Workgroups reach the 8 XCDs round-robin, so an item's workgroups go on
// round the XCDs from where the previous item's ended (items of a few tiles
// spread over all XCDs instead of piling onto the first), and the
// workgroups of one XCD take a contiguous run of the item's tiles in band
// order (bands of up to 8 m-blocks, m fastest), a compact patch whose
// activation rows and weight columns stay in that XCD's L2 (the fused 4-bit
// kernel uses bands of 2 m-blocks).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <unordered_map>
#include <vector>

#include "device.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

struct GemmItem {
    const u32x4 *B;    // fragment-packed bf16 weights [Nt16][KT32][64] x 16 B
    const uint16_t *X; // bf16 activations, K padded to 64
    void *Y;
    int64_t ldx, ldy;
    int32_t Ns, Nt16;
    int32_t KT32;      // 32-k tiles per column tile in B
    int32_t KT64;      // 64-k stages
    int32_t MB, NB;    // tile grid
    int32_t R;         // members of a joined sum set (1: a lone product)
    int32_t start;     // first workgroup
    int32_t accumulate;
    int32_t flags;     // bit 0: bf16 output
    int64_t M;         // rows of this item
    float *P;          // ks > 1: binary32 k-partials [ks][M][Ns]
    int32_t ks;        // k-splits: tile t of split q covers stages [q nst / ks, (q+1) nst / ks)
    int32_t seg;       // R > 1: the set's row of the member tables
};
static_assert(sizeof(GemmItem) == 104, "item table size");
constexpr int kYBf16 = 1;

struct GemmGroup {
    int64_t M;
    int32_t n, pad_;
    GemmItem it[kPrefillGroupMax];
    // joined sum set j, member r: its packed weights, its activations and
    // their row stride
    const char *segb[kMaxJoined][kSetParts];
    const char *segx[kMaxJoined][kSetParts];
    int32_t segld[kMaxJoined][kSetParts];
};

// Tile geometry.  A stage covers BK k: 64, or 32 when three 64-k stages do
// not fit in LDS (then four 32-k stages do).  Activation rows are copied in
// 1 KB LDS blocks of RPB rows (RPB x BK x 2 bytes); weight blocks are 32
// columns x 16 k.
template <int BM, int BN, int WM, int WN>
struct G {
    static constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    static constexpr int MT = TM / 32, NT = TN / 32; // 32x32 tiles per wave
    static constexpr int BK = 3 * (BM + BN) * 128 <= kLdsLimit ? 64 : 32;
    static constexpr int S16 = BK / 16;             // 16-k MFMA steps per stage
    static constexpr int CPR = BK / 8;              // 16-byte chunks per activation row
    static constexpr int RPB = 64 / CPR;            // activation rows per 1 KB block
    static constexpr int AF = BM / RPB;             // activation blocks per stage
    static constexpr int BF = (BN / 32) * S16;      // weight blocks per stage
    static constexpr int NW = WM * WN;              // waves
    static constexpr int FPW = (AF + BF) / NW;      // copy instructions per wave per stage
    static constexpr int STAGE = (AF + BF) * 1024;
    // slots: up to four 64-k stages, or five 32-k ones (the 256 x 256 tile:
    // its weight copies, read from HBM, then start four stages ahead of
    // their use -- gqa8 layer M = 512: 342-353 -> 333-338 us)
    static constexpr int NSMAX = BK == 32 ? 5 : 4;
    static constexpr int NS = kLdsLimit / STAGE >= NSMAX ? NSMAX : kLdsLimit / STAGE;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 tiles");
    static_assert(AF % NW == 0 && BF % NW == 0, "LDS blocks must divide over the waves");
    static_assert(NW % S16 == 0, "a wave's weight blocks keep one 16-k step");
    static_assert(NS >= 2, "two stages must fit in LDS");
    static_assert(S16 % 2 == 0, "fragment buffers alternate by step parity");
    static_assert(FPW * (NS - 2) < 64, "vmcnt range");
};

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
    __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) gemm_kernel(GemmGroup grp) {
    using C = G<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(1024))) char lds[C::NS * C::STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // scalar
    const int wm = wave / WN, wn = wave % WN;

    const int bid = blockIdx.x;
    int lo = 0, hi = grp.n - 1; // last item whose first workgroup is <= bid
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (grp.it[mid].start <= bid)
            lo = mid;
        else
            hi = mid - 1;
    }
    const GemmItem &a = grp.it[lo];
    const int64_t M = a.M;
    const int local = bid - a.start;
    // (split, tile) in band order: block b runs on XCD b mod 8, an item's
    // blocks go on round the XCDs from where the previous item's ended, and
    // the blocks of one XCD take a contiguous run of the order
    const int tiles = a.MB * a.NB;
    const int nk = tiles * a.ks, x = local & 7, q8 = nk >> 3, r8 = nk & 7;
    const int tk = x * q8 + (x < r8 ? x : r8) + (local >> 3);
    const int ksi = tk / tiles, t = tk - ksi * tiles;
    const int band = t / (8 * a.NB);
    const int first_m = band * 8;
    const int bm_cnt = a.MB - first_m < 8 ? a.MB - first_m : 8;
    const int in_band = t - band * 8 * a.NB;
    const int64_t mb = first_m + in_band % bm_cnt, nb = in_band / bm_cnt;
    const int64_t m0 = mb * BM, n0 = nb * BN;
    const int nst_all = a.KT64 * (64 / C::BK); // stages of the whole k-range
    const int kb = ksi * nst_all / a.ks;       // this split's first stage
    const int nst = (ksi + 1) * nst_all / a.ks - kb;

    // Sources of this wave's LDS blocks: block f = wave + NW j < AF holds
    // activation rows RPB f .. RPB f + RPB - 1 of the tile, the others weight
    // blocks g = f - AF (columns 32 (g / S16) of the tile, 16-k step g % S16;
    // f < AF exactly when j < AF / NW).  Each is a per-lane byte offset from a
    // tile base that advances by a constant per stage; the offsets are
    // recomputed at every issue (a few VALU ops) rather than held in
    // registers.  Rows past M and columns past the shard are clamped to the
    // last valid ones: in bounds, and those outputs are never stored.
    // Offsets stay below 2^32 because a lane's row, clamped to the tile's
    // last valid one before it meets the row stride, is below 256 and the
    // activation row stride and K are below 2^22 elements (checked by the
    // caller).
    const int64_t t0 = n0 >> 4;
    // Where stage g of the product reads.  A joined sum set (R members of
    // equal k-range, spm stages each) runs the members' k-ranges end to
    // end: stage g is stage g - r spm of member r.  Lane r of xr / br / xl
    // holds member r's activation and record bases for this tile and its
    // activation row stride (lane 0 a lone product's), picked per stage
    // with v_readlane, so the block loop reads no table from memory.
    const int spm = a.R > 1 ? nst_all / a.R : nst_all;
    uint32_t xr[2], br[2], xl;
    {
        const int seg = a.R > 1 ? a.seg : 0;
        const int r = lane < a.R ? lane : 0;
        const char *xm = a.R > 1 ? grp.segx[seg][r] : reinterpret_cast<const char *>(a.X);
        const char *wm0 = a.R > 1 ? grp.segb[seg][r] : reinterpret_cast<const char *>(a.B);
        const int64_t ld = a.R > 1 ? (int64_t)grp.segld[seg][r] : a.ldx;
        const uint64_t xv = (uint64_t)(uintptr_t)(xm + m0 * ld * 2);
        const uint64_t bv = (uint64_t)(uintptr_t)(wm0 + t0 * (int64_t)a.KT32 * 1024);
        xr[0] = (uint32_t)xv;
        xr[1] = (uint32_t)(xv >> 32);
        br[0] = (uint32_t)bv;
        br[1] = (uint32_t)(bv >> 32);
        xl = (uint32_t)ld;
    }
    // the activation and record bases and the activation row stride of
    // stage kt of this split
    auto src = [&](int kt, const char *&xs, const char *&bs, uint32_t &xld)
                   __attribute__((always_inline)) {
        int r = 0, gl = kt + kb;
        while (gl >= spm) { // uniform, at most R - 1 + NS / spm steps
            gl -= spm;
            ++r;
        }
        xld = (uint32_t)__builtin_amdgcn_readlane((int)xl, r);
        const uint64_t xv = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)xr[0], r) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)xr[1], r) << 32);
        const uint64_t bv = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)br[0], r) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)br[1], r) << 32);
        xs = reinterpret_cast<const char *>((uintptr_t)xv) + gl * (C::BK * 2);
        bs = reinterpret_cast<const char *>((uintptr_t)bv) + gl * (C::BK / 32 * 1024);
    };
    const int arow = lane / C::CPR; // row of this lane in its block
    const uint32_t chunk = 8 * ((lane % C::CPR) ^ swz<C::CPR>(arow));
    const uint32_t arow0 = (uint32_t)(C::RPB * wave + arow); // in copy 0
    const uint32_t last_row = (uint32_t)(M - 1 - m0 < BM - 1 ? M - 1 - m0 : BM - 1);
    const int kr = 2 * (wave % C::S16) + (lane >> 5); // 8-k run of this wave's weight blocks
    const uint32_t boff0 = ((uint32_t)((kr >> 2) * 64 + (kr & 3) * 16 + (lane & 15))) * 16;
    const uint32_t tstep = (uint32_t)a.KT32 * 1024; // one 16-column tile
    const int tmax = (int)(a.Nt16 - 1 - t0);
    const int tfirst = 2 * (wave / C::S16) + ((lane & 31) >> 4);
    constexpr int TPJ = 2 * (C::NW / C::S16); // 16-column tiles per weight block step
    const uint32_t lds0 = (uint32_t)(uintptr_t)(void __attribute__((address_space(3))) *)lds;
    // copy j (0 <= j < FPW) of this wave for the stage whose bases are xs,
    // bs (activation row stride xld) into LDS slot `slot`
    auto issue1 = [&](const char *xs, const char *bs, uint32_t xld, int slot, int j)
                      __attribute__((always_inline)) {
        const uint32_t dst = lds0 + slot * C::STAGE + wave * 1024 + C::NW * j * 1024;
        uint32_t a0 = arow0, b0 = boff0;
        asm volatile("" : "+v"(a0), "+v"(b0)); // keep the per-j offsets out of registers
        if (j < C::AF / C::NW) {
            const uint32_t row = a0 + (uint32_t)(j * C::NW * C::RPB);
            dma16(xs, ((row < last_row ? row : last_row) * xld + chunk) * 2, dst);
        } else {
            const int tt = tfirst + TPJ * (j - C::AF / C::NW);
            dma16(bs, b0 + (uint32_t)(tt < tmax ? tt : tmax) * tstep, dst);
        }
    };
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
        const char *xs, *bs;
        uint32_t xld;
        src(kt, xs, bs, xld);
#pragma unroll
        for (int j = 0; j < C::FPW; ++j)
            issue1(xs, bs, xld, slot, j);
    };

    f32x16 acc[C::MT][C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    // fragments of 16-k step s of the stage in `slot`
    u32x4 af[2][C::MT], bfr[2][C::NT];
    auto rd = [&](int slot, int s, u32x4 (&x)[C::MT], u32x4 (&y)[C::NT]) __attribute__((always_inline)) {
        const char *As = lds + slot * C::STAGE;
        const char *Bs = As + C::AF * 1024;
#pragma unroll
        for (int i = 0; i < C::MT; ++i) {
            const int r = (wm * C::MT + i) * 32 + (lane & 31); // row in the block tile
            const int k8 = 2 * s + (lane >> 5);                // 8-k run in the stage
            const int rb = r % C::RPB;
            x[i] = *reinterpret_cast<const u32x4 *>(As + (r / C::RPB) * 1024 + rb * (C::BK * 2) +
                                                    ((k8 ^ swz<C::CPR>(rb)) * 16));
        }
#pragma unroll
        for (int j = 0; j < C::NT; ++j)
            y[j] = *reinterpret_cast<const u32x4 *>(
                Bs + (((wn * C::NT + j) * C::S16 + s) * 64 + lane) * 16);
    };
    // this wave's copies of stage kt are done once only the younger stages'
    // copies (at most NS - 2) may still be in flight
    auto wait_stage = [&](int kt) __attribute__((always_inline)) {
        const int younger = nst - 1 - kt < C::NS - 2 ? nst - 1 - kt : C::NS - 2;
        if (C::NS >= 5 && younger >= 3)
            wait_vmcnt<C::FPW * 3>();
        else if (C::NS >= 4 && younger >= 2)
            wait_vmcnt<C::FPW * 2>();
        else if (C::NS >= 3 && younger >= 1)
            wait_vmcnt<C::FPW>();
        else
            wait_vmcnt<0>();
    };

    for (int k = 0; k < C::NS && k < nst; ++k)
        issue(k, k);
    wait_stage(0);
    barrier();
    rd(0, 0, af[0], bfr[0]);
    int slot = 0;
    for (int kt = 0; kt < nst; ++kt) {
        const int next = slot + 1 == C::NS ? 0 : slot + 1;
        const char *cxs = nullptr, *cbs = nullptr; // stage kt + NS's bases
        uint32_t cxld = 0;
#pragma unroll
        for (int s = 0; s < C::S16; ++s) {
            const int b = s & 1; // S16 is even, so step parity is s parity
            bool copies = false;
            if (s + 1 < C::S16) {
                rd(slot, s + 1, af[b ^ 1], bfr[b ^ 1]);
            } else {
                // this wave's reads of stage kt have landed (on every path,
                // so that the MFMAs below wait for nothing newer)
                wait_lgkm0();
                if (kt + 1 < nst) {
                    wait_stage(kt + 1);
                    barrier();
                    rd(next, 0, af[b ^ 1], bfr[b ^ 1]);
                    copies = kt + C::NS < nst;
                    if (copies)
                        src(kt + C::NS, cxs, cbs, cxld);
                }
            }
            // the copies of stage kt + NS go into the slot of stage kt,
            // spread between the MFMAs of the last step so that they issue
            // in their shadow
#pragma unroll
            for (int q = 0; q < C::MT * C::NT; ++q) {
                const int i = q / C::NT, j = q % C::NT;
                acc[i][j] = mfma32(af[b][i], bfr[b][j], acc[i][j]);
                if (s + 1 == C::S16) {
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int f = q * C::FPW / (C::MT * C::NT); f < (q + 1) * C::FPW / (C::MT * C::NT); ++f)
                        if (copies)
                            issue1(cxs, cbs, cxld, slot, f);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // keep the steps in this order: the scheduler would otherwise
            // sink MFMAs below the waits and the barrier of the next step
            __builtin_amdgcn_sched_barrier(0);
        }
        slot = next;
    }

    // ---- epilogue: acc reg r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32 ----
    // One base address per lane; every store is that base plus a
    // compile-time row/column step times the (uniform) row stride.
    const int64_t row0 = m0 + wm * C::MT * 32 + 4 * (lane >> 5);
    const int64_t col0 = n0 + wn * C::NT * 32 + (lane & 31);
    // a k-split writes its binary32 partial, [M][Ns] at split ksi
    const bool part = a.ks > 1;
    const bool ybf = part ? false : (a.flags & kYBf16) != 0;
    const bool accu = part ? false : a.accumulate;
    const int64_t ldy = part ? a.Ns : a.ldy;
    char *yb0 = part ? reinterpret_cast<char *>(a.P + (int64_t)ksi * M * a.Ns)
                     : static_cast<char *>(a.Y);
    const int esz = ybf ? 2 : 4;
    char *ybase = yb0 + (row0 * ldy + col0) * esz;
    const int64_t rstride = ldy * esz;
    bool colok[C::NT];
#pragma unroll
    for (int j = 0; j < C::NT; ++j)
        colok[j] = col0 + 32 * j < a.Ns;
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = i * 32 + 8 * (r >> 2) + (r & 3); // row step from row0
            if (row0 + rr >= M)
                continue;
            char *yr = ybase + rr * rstride;
#pragma unroll
            for (int j = 0; j < C::NT; ++j) {
                if (!colok[j])
                    continue;
                const float v = acc[i][j][r];
                if (ybf) {
                    __bf16 h = (__bf16)v;
                    *reinterpret_cast<uint16_t *>(yr + j * 64) = __builtin_bit_cast(uint16_t, h);
                } else {
                    float *y = reinterpret_cast<float *>(yr + j * 128);
                    *y = accu ? *y + v : v;
                }
            }
        }
}

// ---- prep: activation copies ----------------------------------------------
// One job per distinct activation matrix of a launch: a product's X, or the
// members' blocks X_0, X_1, ... of a joined sum set side by side.  A
// workgroup of four waves takes one row of a wide job (rows of 4096
// columns and more) and four rows, a wave each, of a narrow one, so that
// rows of a few hundred columns still keep every lane busy.  Binary16
// copies (4-bit weights): the row's largest magnitude fixes e_m
// (kActExpBias below its ilogb), every element becomes x 2^-e_m rounded to
// nearest binary16, and e_m goes to rexp[m].  Plain copies (bf16 weights
// with ragged K) only zero-pad.  Segment r is the piece at pos r of the
// job; columns past its Ks up to Kw are zero.  A segment with a row index
// reads its row m from row ridx[m] of x_in (a row of zeros when that lies
// outside [0, x_rows)).
struct XPiece {
    const uint16_t *x_in;
    const int32_t *ridx; // null: row m of x_in
    int64_t x_rows;
    uint16_t *x_out;  // this segment's first output column
    int32_t *rexp;    // row exponents (binary16 copy), null for a plain copy
    int64_t ldx_in;
    int32_t x_ld;     // output row stride (elements)
    int32_t Ks, Kw;   // columns read / written by this segment
    int32_t R, pos;   // segments of the job, this one's place
    int32_t M;        // rows
    int32_t start;    // first workgroup of the job (the same for its pieces)
    int32_t wide;     // the job's rows take a workgroup each (else a wave each)
};

struct XPrepGroup {
    int32_t n, pad_;
    XPiece it[kPrefillGroupMax];
};
constexpr int kXPrepWideColumns = 4096;

// |x| of a bf16 pair, bit patterns (magnitude order is integer order)
__device__ __forceinline__ uint32_t pair_max_abs(uint32_t m, uint32_t v) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    const us2 a = __builtin_bit_cast(us2, m), b = __builtin_bit_cast(us2, v & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// The rows of one launch: its jobs' pieces in grp.it[0 .. grp.n).
template <class Group>
__device__ __forceinline__ void xprep_rows(const Group &grp, uint32_t *red) {
    const int bid = blockIdx.x;
    int lo = 0, hi = grp.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (grp.it[mid].start <= bid)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int first = lo - grp.it[lo].pos;
    const XPiece &j0 = grp.it[first];
    // the whole workgroup on one row (wide jobs), or a wave on each of four
    const bool wide = j0.wide != 0;
    const int tid = wide ? (int)threadIdx.x : (int)(threadIdx.x & 63);
    const int nthr = wide ? 256 : 64;
    const int64_t m = wide ? (int64_t)(bid - j0.start)
                           : (int64_t)(bid - j0.start) * 4 +
                                 __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (m >= j0.M)
        return; // narrow jobs only (a wide job's workgroups are its rows): no barrier follows
    const bool to_f16 = j0.rexp != nullptr;
    // the source row of segment p (null: a row of zeros)
    auto src_row = [&](const XPiece &p) -> const uint16_t * {
        int64_t row = m;
        if (p.ridx) {
            row = p.ridx[m];
            if (row < 0 || row >= p.x_rows)
                return nullptr;
        }
        return p.x_in + row * p.ldx_in;
    };
    int e = 0;
    // a narrow lone row of up to 2048 columns: read once into registers,
    // then its largest magnitude and its binary16 copy from them
    if (to_f16 && !wide && j0.R == 1 && j0.Kw <= 4 * 64 * 8) {
        const uint16_t *src = src_row(j0);
        const int ks = src ? j0.Ks : 0; // columns read
        u32x4 v[4];
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = tid * 8 + i * 64 * 8;
            v[i] = u32x4{0, 0, 0, 0};
            if (k + 8 <= ks) {
                v[i] = *reinterpret_cast<const u32x4 *>(src + k);
            } else if (k < ks) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo2 = (k + 2 * q < ks) ? src[k + 2 * q] : 0u;
                    const uint32_t hi2 = (k + 2 * q + 1 < ks) ? src[k + 2 * q + 1] : 0u;
                    v[i][q] = lo2 | (hi2 << 16);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mx = pair_max_abs(mx, v[i][q]); // zero columns leave it as it is
        }
        uint32_t h = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const uint32_t x = __shfl_xor(h, o, 64);
            h = x > h ? x : h;
        }
        if (h != 0 && h < 0x7F80u)
            e = __builtin_amdgcn_frexp_expf(__uint_as_float(h << 16)) - 1 - kActExpBias;
        if (tid == 0)
            j0.rexp[m] = e;
        uint16_t *dst = j0.x_out + m * (int64_t)j0.x_ld;
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = tid * 8 + i * 64 * 8;
            if (k < j0.Kw) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    h2 o;
                    o.x = (_Float16)__builtin_amdgcn_ldexpf(bf16_lo(v[i][q]), -e);
                    o.y = (_Float16)__builtin_amdgcn_ldexpf(bf16_hi(v[i][q]), -e);
                    v[i][q] = __builtin_bit_cast(uint32_t, o);
                }
                *reinterpret_cast<u32x4 *>(dst + k) = v[i];
            }
        }
        return;
    }
    if (to_f16) {
        uint32_t mx = 0;
        for (int r = 0; r < j0.R; ++r) {
            const XPiece &p = grp.it[first + r];
            const uint16_t *src = src_row(p);
            if (!src)
                continue;
            for (int k = tid * 8; k < p.Ks; k += nthr * 8) {
                if (k + 8 <= p.Ks) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(src + k);
                    mx = pair_max_abs(mx, v.x);
                    mx = pair_max_abs(mx, v.y);
                    mx = pair_max_abs(mx, v.z);
                    mx = pair_max_abs(mx, v.w);
                } else {
                    for (int q = k; q < p.Ks; ++q)
                        mx = pair_max_abs(mx, src[q]);
                }
            }
        }
        uint32_t h = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const uint32_t x = __shfl_xor(h, o, 64);
            h = x > h ? x : h;
        }
        if (wide) { // the row's four waves agree
            if ((threadIdx.x & 63) == 0)
                red[threadIdx.x >> 6] = h;
            __syncthreads();
            h = red[0];
#pragma unroll
            for (int w = 1; w < 4; ++w)
                h = red[w] > h ? red[w] : h;
        }
        // a row of zeros (or non-finite values) keeps e = 0
        if (h != 0 && h < 0x7F80u)
            e = __builtin_amdgcn_frexp_expf(__uint_as_float(h << 16)) - 1 - kActExpBias;
        if (tid == 0)
            j0.rexp[m] = e;
    }
    for (int r = 0; r < j0.R; ++r) {
        const XPiece &p = grp.it[first + r];
        const uint16_t *src = src_row(p);
        const int ks = src ? p.Ks : 0; // columns read
        uint16_t *dst = p.x_out + m * (int64_t)p.x_ld;
        for (int k = tid * 8; k < p.Kw; k += nthr * 8) {
            u32x4 v = {0, 0, 0, 0};
            if (k + 8 <= ks) {
                v = *reinterpret_cast<const u32x4 *>(src + k);
            } else if (k < ks) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo2 = (k + 2 * q < ks) ? src[k + 2 * q] : 0u;
                    const uint32_t hi2 = (k + 2 * q + 1 < ks) ? src[k + 2 * q + 1] : 0u;
                    v[q] = lo2 | (hi2 << 16);
                }
            }
            if (to_f16) {
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    h2 o;
                    o.x = (_Float16)__builtin_amdgcn_ldexpf(bf16_lo(v[q]), -e);
                    o.y = (_Float16)__builtin_amdgcn_ldexpf(bf16_hi(v[q]), -e);
                    v[q] = __builtin_bit_cast(uint32_t, o);
                }
            }
            *reinterpret_cast<u32x4 *>(dst + k) = v;
        }
    }
}

__global__ void __launch_bounds__(256) xprep_kernel(XPrepGroup grp) {
    __shared__ uint32_t red[4];
    xprep_rows(grp, red);
}

// Row gathers (plain copies through a row index) take a short job table:
// a call has few distinct gathers, and a launch's arguments are copied
// whole whatever the table holds.
constexpr int kGatherJobs = 16;
struct GatherGroup {
    int32_t n, pad_;
    XPiece it[kGatherJobs];
};

__global__ void __launch_bounds__(256) gather_rows_kernel(GatherGroup grp) {
    __shared__ uint32_t red[4];
    xprep_rows(grp, red);
}

typedef void (*GemmFn)(GemmGroup);

struct Variant {
    int bm, bn, wm, wn;
};
// tile shapes with a kernel instance: bf16 operands, and the fused 4-bit
// kernel (waves WM x 4; two workgroups per CU where they fit)
constexpr Variant kVariants[] = {{256, 256, 2, 4}, {256, 160, 4, 1}, {256, 128, 4, 2},
                                 {128, 256, 2, 4}, {128, 128, 2, 2}, {256, 64, 4, 1},
                                 {128, 64, 2, 2},  {64, 64, 2, 2}};
constexpr Variant kQ4Variants[6] = {{256, 256, 2, 4}, {256, 128, 1, 4}, {128, 256, 2, 4},
                                    {128, 128, 1, 4}, {64, 256, 1, 4},  {64, 128, 1, 4}};
// workgroups of a 4-bit tile shape per CU
int q4_per_cu(const Variant &v) { return q4_tiles_per_cu(v.bm, v.bn, v.wm); }

GemmFn pick(const Variant &v) {
#define TSL_CASE(BM_, BN_, WM_, WN_)                                                               \
    if (v.bm == BM_ && v.bn == BN_ && v.wm == WM_ && v.wn == WN_)                                  \
        return gemm_kernel<BM_, BN_, WM_, WN_>;
    TSL_CASE(256, 256, 2, 4) TSL_CASE(256, 160, 4, 1) TSL_CASE(256, 128, 4, 2)
    TSL_CASE(128, 256, 2, 4) TSL_CASE(128, 128, 2, 2) TSL_CASE(256, 64, 4, 1)
    TSL_CASE(128, 64, 2, 2) TSL_CASE(64, 64, 2, 2)
#undef TSL_CASE
    return nullptr;
}

inline int64_t kpad64(int64_t k) { return (k + 63) / 64 * 64; }

// Modelled time of a variant over a group: greedy list scheduling of the
// tiles (in launch order) on 256 CUs, one workgroup each, times the larger
// of two per-CU penalties relative to the 4096 flop/clk the MFMAs retire:
// LDS traffic (fragment reads of (TM + TN) x 2 bytes per k per wave plus
// the (BM + BN) x 2 bytes the copies write, at 128 B/clk) and L2 delivery
// ((BM + BN) x 2 bytes per 2 BM BN flops at a sustained ~40 B/clk).
// k-splits of the products of launch [c0, c1): each long product's k-range
// in `factor` parts (at least 8 stages of 64 k each, at most 8 parts);
// products that accumulate into Y or belong to a sum set too long for one
// sum launch are not split.
void split_ks(const LinearItem *items, int c0, int c1, int factor, int *ks) {
    for (int i = c0; i < c1; ++i) {
        ks[i - c0] = 1;
        if (factor <= 1 || items[i].accumulate || items[i].no_split)
            continue;
        const int64_t cap = kpad64(items[i].g.Ks) / 64 / 8;
        const int64_t k = factor < cap ? factor : cap;
        ks[i - c0] = (int)(k < 1 ? 1 : (k > 8 ? 8 : k));
    }
}

// ... or each long product's k-range into as many parts as bring it to at
// most `len` stages of 64 k (same limits), so that a launch of products of
// unequal k-ranges (a joined sum set among single products) splits only
// its longest ones.
void split_to_length(const LinearItem *items, int c0, int c1, int64_t len, int *ks) {
    for (int i = c0; i < c1; ++i) {
        ks[i - c0] = 1;
        if (items[i].accumulate || items[i].no_split)
            continue;
        const int64_t st = kpad64(items[i].g.Ks) / 64;
        int64_t k = (st + len - 1) / len;
        const int64_t cap = st / 8;
        k = k < cap ? k : cap;
        ks[i - c0] = (int)(k < 1 ? 1 : (k > 8 ? 8 : k));
    }
}

// A launch with fewer tiles than this -- a quarter of the CUs -- splits the
// k-range of its long products toward one tile per CU.
constexpr int64_t kSplitBelow = 64;

// Modelled cost of one launch [c0, c1) whose items are split ks[i - c0]
// ways along k.
double chunk_cost(const Variant &v, double pen, const LinearItem *items, int c0, int c1,
                  const int *ks, int per_cu) {
    auto mbk = [&](int i) { return (items[i].M + v.bm - 1) / v.bm; };
    double span = 0.0, extra = 0.0;
    int64_t tiles = 0;
    for (int i = c0; i < c1; ++i) {
        tiles += mbk(i) * ((items[i].g.Ns + v.bn - 1) / v.bn) * ks[i - c0];
        if (ks[i - c0] > 1) // partials written and read once, ~3.3 KB per clock
            extra += 2.0 * ks[i - c0] * (double)items[i].M * (double)items[i].g.Ns * 4 / 3333.0;
    }
    if (tiles > 16384) { // large: every CU busy to the end, to a tile
        double work = 0.0, longest = 0.0;
        for (int i = c0; i < c1; ++i) {
            const double len = (double)kpad64(items[i].g.Ks) / 64.0 / ks[i - c0];
            work += (double)(mbk(i) * ((items[i].g.Ns + v.bn - 1) / v.bn) * ks[i - c0]) * len;
            longest = len > longest ? len : longest;
        }
        span = work / 256.0 + longest;
    } else {
        // per_cu workgroups share a CU, each at 1 / per_cu of its rate
        std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
        for (int i = 0; i < 256 * per_cu; ++i)
            cu.push(0.0);
        for (int i = c0; i < c1; ++i) {
            const double len = (double)kpad64(items[i].g.Ks) / 64.0 / ks[i - c0] * per_cu;
            const int64_t T = mbk(i) * ((items[i].g.Ns + v.bn - 1) / v.bn) * ks[i - c0];
            for (int64_t t = 0; t < T; ++t) {
                const double f = cu.top() + len;
                cu.pop();
                cu.push(f);
                span = f > span ? f : span;
            }
        }
    }
    // a stage of a bm x bn tile is bm bn / 32 clocks of MFMA
    return span * (double)(v.bm * v.bn) * pen + extra * 32.0;
}

// Launches of fewer tiles than this -- four per CU -- try k-split factors
// up to 8, and splits of the products longer than each k-range the launch
// holds down to it, and keep the one the list schedule models shortest
// (the partials' traffic included): a launch of one or two waves of long
// tiles otherwise ends with most CUs idle.
constexpr int64_t kSplitSearchBelow = 1024;

// Modelled cost of a variant over a group, each launch (kPrefillGroupMax items;
// every launch drains before the next starts) with its k-splits, which
// *ks receives per item: a launch of fewer than kSplitBelow tiles splits
// its long products toward one tile per CU; a launch of fewer than
// kSplitSearchBelow tiles takes the modelled best factor.
double variant_cost(const Variant &v, const LinearItem *items, int n, std::vector<int> *ks,
                    bool q4) {
    const double TM = v.bm / v.wm, TN = v.bn / v.wn;
    const double flops = 2.0 * v.bm * v.bn; // per k
    double pen;
    if (!q4) {
        const double lds = 4096.0 * (4.0 * (TM + TN) * 2 + (v.bm + v.bn) * 2) / flops / 128.0;
        const double l2 = 4096.0 * (v.bm + v.bn) * 2 / flops / 40.0;
        pen = lds > l2 ? lds : l2;
    } else {
        // the fused 4-bit kernel: LDS reads of binary16 activations by the
        // four column waves and of code words, copies of activations and
        // records; L2 delivery of both
        const double lds = 4096.0 * (4.0 * v.bm * 2 + v.bn * 0.5 + v.bm * 2 + v.bn * 0.5625) /
                           flops / 128.0;
        const double l2 = 4096.0 * (v.bm * 2 + v.bn * 0.5625) / flops / 40.0;
        pen = lds > l2 ? lds : l2;
        pen = pen > 1.0 ? pen : 1.0;
        // plus the issue cycles every 16-k step costs a wave besides its
        // MFMAs (reads, expansion, copies, waits: ~120), against the SIMD's
        // bm bn / 4096 MFMAs of 32 clocks per step; a second wave per SIMD
        // (two row waves, or two workgroups per CU) covers half of it
        const int waves = v.wm * q4_per_cu(v);
        pen += 120.0 / ((v.bm / 32) * (v.bn / 4 / 32) * 32.0) / (waves > 1 ? 2.0 : 1.0);
    }
    pen = pen > 1.0 ? pen : 1.0;
    double total = 0.0;
    ks->assign(n, 1);
    for (int c0 = 0; c0 < n;) {
        const int c1 = prefill_chunk_end(items, n, c0);
        const int per_cu = q4 ? q4_per_cu(v) : 1;
        int64_t tiles = 0;
        for (int i = c0; i < c1; ++i)
            tiles += ((items[i].M + v.bm - 1) / v.bm) * ((items[i].g.Ns + v.bn - 1) / v.bn);
        int *kc = &(*ks)[c0];
        if (tiles < kSplitBelow)
            split_ks(items, c0, c1, (int)((256 + tiles - 1) / tiles), kc);
        double best = chunk_cost(v, pen, items, c0, c1, kc, per_cu);
        if (tiles >= kSplitBelow && tiles < kSplitSearchBelow) {
            int trial[kPrefillGroupMax];
            auto consider = [&]() {
                const double c = chunk_cost(v, pen, items, c0, c1, trial, per_cu);
                if (c < best * 0.98) {
                    best = c;
                    std::memcpy(kc, trial, sizeof(int) * (c1 - c0));
                }
            };
            for (int f : {2, 3, 4, 6, 8}) {
                split_ks(items, c0, c1, f, trial);
                consider();
            }
            std::vector<int64_t> lens;
            for (int i = c0; i < c1; ++i)
                lens.push_back(kpad64(items[i].g.Ks) / 64);
            std::sort(lens.begin(), lens.end());
            lens.erase(std::unique(lens.begin(), lens.end()), lens.end());
            for (size_t q = 0; q + 1 < lens.size(); ++q) { // the longest splits nothing
                split_to_length(items, c0, c1, lens[q], trial);
                consider();
            }
        }
        total += best;
        c0 = c1;
    }
    return total;
}

// The tile shape and k-splits of a group's geometry, remembered: the cost
// model (a list schedule per variant and split factor) runs once per
// distinct geometry, and repeated calls of one layer's group reuse it.
struct PlanChoice {
    Variant v;
    std::vector<int> ks;
};
std::mutex g_plan_mu;
std::unordered_map<std::string, PlanChoice> g_plans;
constexpr size_t kPlanCacheMax = 256;

// what the choice depends on: weight type, and per item rows, k, columns
// and whether it may be split
std::string plan_key(const LinearItem *items, int n, tsl_dtype wdtype) {
    std::string key(sizeof(int32_t) + (size_t)n * 25, '\0');
    char *p = &key[0];
    const int32_t w = (int32_t)wdtype;
    std::memcpy(p, &w, 4);
    p += 4;
    for (int i = 0; i < n; ++i) {
        const int64_t f[3] = {items[i].M, items[i].g.Ks, items[i].g.Ns};
        std::memcpy(p, f, 24);
        p[24] = (char)((items[i].accumulate ? 1 : 0) | (items[i].no_split ? 2 : 0));
        p += 25;
    }
    return key;
}

} // namespace

bool prefill_supported(tsl_dtype wdtype) { return wdtype == TSL_BF16 || wdtype == TSL_Q4G64; }

PrefillPlan prefill_plan(const LinearItem *items, int n, tsl_dtype wdtype, int64_t M) {
    (void)M;
    PrefillPlan best;
    const bool q4 = wdtype == TSL_Q4G64;
    const std::string key = plan_key(items, n, wdtype);
    PlanChoice choice;
    bool cached = false;
    {
        std::lock_guard<std::mutex> lock(g_plan_mu);
        auto it = g_plans.find(key);
        if (it != g_plans.end()) {
            choice = it->second;
            cached = true;
        }
    }
    if (!cached) {
        double best_cost = 1e300;
        std::vector<int> ks;
        const Variant *vs = q4 ? kQ4Variants : kVariants;
        const int nv = q4 ? (int)(sizeof(kQ4Variants) / sizeof(Variant))
                          : (int)(sizeof(kVariants) / sizeof(Variant));
        for (int vi = 0; vi < nv; ++vi) {
            const double cost = variant_cost(vs[vi], items, n, &ks, q4);
            if (cost < best_cost - 1e-9) {
                best_cost = cost;
                choice.v = vs[vi];
                choice.ks = ks;
            }
        }
        std::lock_guard<std::mutex> lock(g_plan_mu);
        if (g_plans.size() >= kPlanCacheMax)
            g_plans.clear();
        g_plans.emplace(key, choice);
    }
    best.bm = choice.v.bm;
    best.bn = choice.v.bn;
    best.wm = choice.v.wm;
    best.wn = choice.v.wn;
    // workspace: activation copies (binary16 for 4-bit items, with their
    // row exponents; zero-padded bf16 for ragged-K bf16 items), one per
    // distinct (X, ldx, K, rows) -- items without a known X (sizing, joined
    // sets) never share; the 4-bit weights are read from their records
    best.x_off.assign(n, 0);
    best.x_first.assign(n, -1);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return at;
    };
    for (int i = 0; i < n; ++i) {
        const PackGeom &g = items[i].g;
        const bool q4 = wdtype == TSL_Q4G64;
        if (q4 || g.Ks % 64 != 0) {
            int first = i;
            for (int j = 0; j < i && items[i].X; ++j)
                if (items[j].X == items[i].X && items[j].ldx == items[i].ldx &&
                    items[j].ridx == items[i].ridx && items[j].x_rows == items[i].x_rows &&
                    items[j].g.Ks == g.Ks && items[j].M == items[i].M && best.x_first[j] == j) {
                    first = j;
                    break;
                }
            best.x_first[i] = first;
            // the copy, then (binary16) its row exponents, padded to whole
            // 256-row tiles (the GEMM reads them by the tile)
            best.x_off[i] = first == i ? take((size_t)items[i].M * (size_t)kpad64(g.Ks) * 2 +
                                              (q4 ? (size_t)(items[i].M + 255) / 256 * 256 * 4
                                                  : 0))
                                       : best.x_off[first];
        }
    }
    // k-splits (as modelled), their binary32 partials after the other
    // copies
    best.ks = choice.ks;
    best.p_off.assign(n, 0);
    for (int i = 0; i < n; ++i)
        if (best.ks[i] > 1) {
            best.p_off[i] = off;
            off += ((size_t)best.ks[i] * (size_t)items[i].M * (size_t)items[i].g.Ns * 4 + 255) /
                   256 * 256;
        }
    best.ws_bytes = off;
    return best;
}

// The activation pass of items [c0, c1): a job per distinct X (a joined
// set's job has a piece per member), launched in groups of whole jobs.
hipError_t launch_xprep(const PrefillPlan &p, const LinearItem *items, int c0, int c1, bool q4,
                        char *ws, hipStream_t stream) {
    std::vector<XPiece> xp;
    for (int i = c0; i < c1; ++i) {
        const LinearItem &L = items[i];
        if (p.x_first[i] != i)
            continue;
        const PackGeom &g = L.g;
        const int R = L.cat;
        const int64_t kseg = g.Ks / R;
        for (int r = 0; r < R; ++r) {
            XPiece x{};
            x.x_in = static_cast<const uint16_t *>(R > 1 ? L.seg_X[r] : L.X);
            x.ldx_in = R > 1 ? L.seg_ldx[r] : L.ldx;
            x.ridx = R > 1 ? L.seg_ridx[r] : L.ridx;
            x.x_rows = R > 1 ? L.seg_xrows[r] : L.x_rows;
            x.x_out = reinterpret_cast<uint16_t *>(ws + p.x_off[i]) + r * kseg;
            // row exponents right after the copy's M rows
            x.rexp = q4 ? reinterpret_cast<int32_t *>(reinterpret_cast<uint16_t *>(ws + p.x_off[i]) +
                                                      L.M * kpad64(g.Ks))
                        : nullptr;
            x.x_ld = (int32_t)kpad64(g.Ks);
            x.Ks = (int32_t)kseg;
            x.Kw = (int32_t)(R > 1 ? kseg : kpad64(g.Ks));
            x.R = R;
            x.pos = r;
            x.M = (int32_t)L.M;
            xp.push_back(x);
        }
    }
    for (size_t q0 = 0; q0 < xp.size();) {
        XPrepGroup xg{};
        int64_t blocks = 0;
        size_t q = q0;
        while (q < xp.size() && q - q0 + xp[q].R <= (size_t)kPrefillGroupMax) {
            int64_t width = 0;
            for (int r = 0; r < xp[q].R; ++r)
                width += xp[q + r].Kw;
            const bool wide = width >= kXPrepWideColumns;
            for (int r = 0; r < xp[q].R; ++r) {
                XPiece &x = xg.it[xg.n++];
                x = xp[q + r];
                x.start = (int32_t)blocks;
                x.wide = wide ? 1 : 0;
            }
            blocks += wide ? xp[q].M : (xp[q].M + 3) / 4;
            q += xp[q].R;
        }
        if (blocks > 0) {
            hipLaunchKernelGGL(xprep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, xg);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        q0 = q;
    }
    return hipSuccess;
}

// Row gathers: plain copies (no binary16) through the activation pass's
// row code, a 16-bit word of the copy per element half of fp32 data.  Jobs
// that continue one another -- the same X, the next run of the index, the
// next rows of one copy (the per-expert runs of a routing's row layout) --
// merge into one.
hipError_t launch_row_gathers(const std::vector<RowGather> &jobs, size_t elem_bytes,
                              hipStream_t stream) {
    const int64_t h = (int64_t)elem_bytes / 2; // 16-bit words per element
    std::vector<RowGather> merged;
    for (const RowGather &g : jobs) {
        if (!merged.empty()) {
            RowGather &m = merged.back();
            if (m.X == g.X && m.ldx == g.ldx && m.x_rows == g.x_rows && m.Ks == g.Ks &&
                m.ldo == g.ldo && m.ridx + m.M == g.ridx &&
                static_cast<char *>(m.out) + m.M * m.ldo * (int64_t)elem_bytes == g.out &&
                m.M + g.M <= INT32_MAX) {
                m.M += g.M;
                continue;
            }
        }
        merged.push_back(g);
    }
    for (size_t q0 = 0; q0 < merged.size();) {
        GatherGroup xg{};
        int64_t blocks = 0;
        size_t q = q0;
        for (; q < merged.size() && xg.n < kGatherJobs; ++q) {
            const RowGather &g = merged[q];
            XPiece &x = xg.it[xg.n++];
            x.x_in = static_cast<const uint16_t *>(g.X);
            x.ridx = g.ridx;
            x.x_rows = g.x_rows;
            x.ldx_in = g.ldx * h;
            x.x_out = static_cast<uint16_t *>(g.out);
            x.rexp = nullptr;
            x.x_ld = (int32_t)(g.ldo * h);
            x.Ks = (int32_t)(g.Ks * h);
            x.Kw = (int32_t)(g.ldo * h);
            x.R = 1;
            x.pos = 0;
            x.M = (int32_t)g.M;
            x.start = (int32_t)blocks;
            x.wide = x.Kw >= kXPrepWideColumns ? 1 : 0;
            blocks += x.wide ? g.M : (g.M + 3) / 4;
        }
        if (blocks > 0) {
            hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                               xg);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        q0 = q;
    }
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillPlan &p, const LinearItem *items, int n, tsl_dtype wdtype,
                          int64_t M, void *workspace, hipStream_t stream) {
    (void)M;
    char *ws = static_cast<char *>(workspace);
    if (wdtype == TSL_Q4G64) {
        // the activation pass for every item, then the fused 4-bit GEMM
        hipError_t e = launch_xprep(p, items, 0, n, true, ws, stream);
        return e != hipSuccess ? e : launch_q4_gemm(p, items, n, ws, stream);
    }
    GemmFn fn = pick(Variant{p.bm, p.bn, p.wm, p.wn});
    if (!fn)
        return hipErrorInvalidValue;
    for (int c0 = 0; c0 < n;) {
        const int c1 = prefill_chunk_end(items, n, c0);
        // 1. zero-padded copies of ragged-K activations
        hipError_t e = launch_xprep(p, items, c0, c1, false, ws, stream);
        if (e != hipSuccess)
            return e;
        // 2. the GEMM over every item's tiles
        GemmGroup grp{};
        grp.M = M;
        grp.n = c1 - c0;
        int joined = 0;
        int64_t blocks = 0;
        for (int i = 0; i < c1 - c0; ++i) {
            const LinearItem &L = items[c0 + i];
            const PackGeom &g = L.g;
            GemmItem &a = grp.it[i];
            const bool copied = p.x_first[c0 + i] >= 0;
            a.R = L.cat;
            a.seg = 0;
            if (L.cat > 1) { // members never need a copy: whole 64-k stages
                a.seg = joined++;
                for (int r = 0; r < L.cat; ++r) {
                    grp.segb[a.seg][r] = static_cast<const char *>(L.seg_packed[r]);
                    grp.segx[a.seg][r] = static_cast<const char *>(L.seg_X[r]);
                    grp.segld[a.seg][r] = (int32_t)L.seg_ldx[r];
                }
                a.B = static_cast<const u32x4 *>(L.seg_packed[0]);
                a.X = static_cast<const uint16_t *>(L.seg_X[0]);
                a.ldx = L.seg_ldx[0];
            } else {
                a.B = static_cast<const u32x4 *>(L.packed);
                a.X = copied ? reinterpret_cast<const uint16_t *>(ws + p.x_off[c0 + i])
                             : static_cast<const uint16_t *>(L.X);
                a.ldx = copied ? kpad64(g.Ks) : L.ldx;
            }
            a.Y = L.Y;
            a.ldy = L.ldy;
            a.Ns = (int32_t)g.Ns;
            a.Nt16 = (int32_t)g.Nt;
            a.KT32 = (int32_t)(g.KT / L.cat); // a member's
            a.KT64 = (int32_t)(kpad64(g.Ks) / 64);
            a.M = L.M;
            a.MB = (int32_t)((L.M + p.bm - 1) / p.bm);
            a.NB = (int32_t)((g.Ns + p.bn - 1) / p.bn);
            a.ks = p.ks[c0 + i];
            a.P = reinterpret_cast<float *>(ws + p.p_off[c0 + i]);
            a.start = (int32_t)blocks;
            a.accumulate = L.accumulate;
            a.flags = L.ydtype == TSL_BF16 ? kYBf16 : 0;
            blocks += (int64_t)a.MB * a.NB * a.ks;
        }
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * p.wm * p.wn), 0, stream, grp);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        c0 = c1;
    }
    return hipSuccess;
}

int64_t prefill_blocks(const PrefillPlan &p, const LinearItem *items, int n, int64_t M) {
    (void)M;
    int64_t most = 0;
    for (int c0 = 0; c0 < n;) {
        const int c1 = prefill_chunk_end(items, n, c0);
        int64_t blocks = 0;
        for (int i = c0; i < c1; ++i)
            blocks += ((items[i].M + p.bm - 1) / p.bm) * ((items[i].g.Ns + p.bn - 1) / p.bn) *
                      p.ks[i];
        most = blocks > most ? blocks : most;
        c0 = c1;
    }
    return most;
}

} // namespace tsl
