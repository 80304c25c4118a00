// Prefill-sized shard products with 4-bit weights: one rank's Y_i = X W_i
// (column / replicated shard) or Y_i = X_i W_i (row shard), many token rows
// (wiki "Tensor parallel processing", "Details" §1; mlxcel manual "Tensor
// parallelism", "Column Parallel" / "Row Parallel"), with the affine 4-bit
// groups expanded inside the GEMM.
//
// The weights stay in their packed 4-bit records all the way into LDS:
// whole 128-k records of the block's BN columns are copied global -> LDS
// (0.5625 bytes per weight, a third of a binary16 copy), and each wave
// expands the codes of its own columns in registers, s q + b per 16-k MFMA
// step.  Activations are the binary16 copy of the activation pass (each row
// scaled by a power of two), copied global -> LDS in 32-k stages as in the
// bf16 GEMM.  The epilogue multiplies each result by 2^(e_m + f_n), the
// row's and the column's exponents (exact), and stores bf16 or binary32.
//
// Waves are laid out WM x 4 (WM = 2 for 256 x 256 and 128 x 256 tiles,
// two waves per SIMD; else 1, with two workgroups per CU where half the LDS
// holds a tile's pipeline): wave (wm, wn) owns rows [wm BM/WM, (wm+1) BM/WM) and
// columns [wn BN/4, (wn+1) BN/4) of the block tile, so each weight is
// expanded by WM waves (once per row half).  A wave's 32x32x16 f16 MFMA B
// fragment is one 32-bit code word per lane (8 consecutive k of the lane's
// column); the expansion is, per pair of codes, one v_and_or_b32 (plus one
// shift per two pairs), one v_pk_add_f16 and one v_pk_fma_f16 -- 1024 + q
// (or 64 + q) becomes q exactly, then q s' + b' rounds once to binary16,
// where s' = s 2^-f and b' = b 2^-f are the group's scale and bias scaled by
// the column exponent f (exact unless they fall out of binary16 range, far
// below the column's largest weight).
//
// Pipeline: NS activation stages of 32 k and three record slots of 128 k
// rotate through LDS; the copies of a record block travel in the same batch
// as the activation stage that first uses it, ahead of its activation
// copies, so the one per-wave vmcnt wait before the barrier that publishes a
// stage covers both.  Fragment reads and the expansion run one 16-k step
// ahead of the MFMAs; the copies of stage k + NS are issued between the
// MFMAs of the last step of stage k.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace tsl {
namespace {

// One product of a launch (96 bytes; the table rides in the kernel
// arguments).
struct Q4Item {
    const char *W;     // packed records [Nt16][KBm] of 1152 bytes, then the column exponents
    const uint16_t *X; // binary16 activation copy [M][ldx]; row exponents follow its M rows
    void *Y;
    float *P;          // ks > 1: binary32 k-partials [ks][M][Ns]
    int64_t ldy;
    int32_t ldx;       // elements, below 2^22
    int32_t M;
    int32_t Ns, Nt16;
    int32_t KBm;       // 128-k records per column tile of one member
    int32_t nst;       // 32-k activation stages of the whole k-range
    int32_t MB, NB;    // tile grid
    int32_t pad0_, start; // first workgroup
    int32_t flags, ks; // flags: bit 0 bf16 output, bit 1 accumulate
    int32_t seg, R;    // joined sum set: member table row (-1: none) and member count
};
static_assert(sizeof(Q4Item) == 96, "item table size");
constexpr int kQ4YBf16 = 1, kQ4Accumulate = 2;

// Joined sum sets of a launch: member r's records (the product runs over the
// members' k-ranges laid end to end).

struct Q4Group {
    int32_t n, pad_;
    Q4Item it[kPrefillGroupMax];
    const char *segw[kMaxJoined][kSetParts];
};

// Block tile BM x BN, waves WM x WN (WM WN / 4 per SIMD): wave (wm, wn)
// owns rows [wm BM/WM, (wm+1) BM/WM) and columns [wn BN/WN, (wn+1) BN/WN).
template <int BM, int BN, int WM, int WN>
struct Q4G {
    static constexpr int NW = WM * WN;               // waves
    static constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    static constexpr int MT = TM / 32, NT = TN / 32; // 32x32 tiles per wave
    static constexpr int ASLOT = BM * 64;            // a 32-k stage: BM rows x 64 bytes
    static constexpr int AF = BM / 16;               // its 1 KB blocks (16 rows each)
    static constexpr int ACW = AF / NW;              // activation copies per wave per stage
    static constexpr int NR = BN / 16;               // records per 128-k block
    static constexpr int BSLOT = NR * kQ4Record;     // codes [NR][1 KB], then pairs [NR][128 B]
    static constexpr int CCW = NR / NW;              // code copies (1 KB) per wave per block
    static constexpr int PCW = NR / 2 / NW;          // pair copies (256 B, two records) per wave
    static constexpr int BCW = CCW + PCW;
    static constexpr int NBS = 3;                    // record slots
    // two workgroups per CU where they fit (each within half the LDS), so
    // that one's pipeline fill and epilogue overlap the other's MFMAs
    static constexpr int WPC = q4_tiles_per_cu(BM, BN, WM);
    static constexpr int NSA = (kLdsLimit / WPC - NBS * BSLOT) / ASLOT;
    static constexpr int NS = NSA > 8 ? 8 : NSA;     // activation slots
    static_assert(MT >= 2 && NT >= 1 && TN % 32 == 0, "whole 32x32 tiles, two or more per step");
    static_assert(AF % NW == 0 && NR % (2 * NW) == 0, "copies divide over the waves");
    static_assert(NS >= 4, "activation stages in flight");
    static_assert((NS - 2) * ACW + 2 * BCW < 64, "vmcnt range");
};

// s 2^-f and b 2^-f of a (scale, bias) bf16 pair, each rounded to nearest
// binary16 and repeated in both halves of a word.
__device__ __forceinline__ void q4_pair(uint32_t sb, int f, uint32_t &ss, uint32_t &bb) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v;
    v.x = (_Float16)__builtin_amdgcn_ldexpf(bf16_lo(sb), -f);
    v.y = (_Float16)__builtin_amdgcn_ldexpf(bf16_hi(sb), -f);
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    ss = (u & 0xFFFFu) * 0x10001u;
    bb = (u >> 16) * 0x10001u;
}

// Tile order of an item: bands of kBandM row tiles, each band column tile by
// column tile (row tiles fastest); the workgroups of one XCD take a
// contiguous run of this order, so an XCD's concurrent tiles share kBandM
// row tiles' activations and a few column tiles' records in its L2.
constexpr int kBandM = 2;

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
    __attribute__((amdgpu_waves_per_eu(WM * WN / 4 * q4_tiles_per_cu(BM, BN, WM),
                                       WM * WN / 4 * q4_tiles_per_cu(BM, BN, WM))))
    q4_gemm_kernel(Q4Group grp) {
    using C = Q4G<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(1024))) char lds[C::NS * C::ASLOT + C::NBS * C::BSLOT];
    __shared__ const char *mtab[kSetParts];
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
    const Q4Item &a = grp.it[lo];
    const int64_t M = a.M;
    const int local = bid - a.start;
    // (split, tile) in band order: block b runs on XCD b mod 8, an item's
    // blocks go on round the XCDs from where the previous item's ended, and
    // the blocks of one XCD take a contiguous run of the order
    const int tiles = a.MB * a.NB;
    const int nk = tiles * a.ks, x = local & 7, q8 = nk >> 3, r8 = nk & 7;
    const int tk = x * q8 + (x < r8 ? x : r8) + (local >> 3);
    const int ksi = tk / tiles, t = tk - ksi * tiles;
    const int band = t / (kBandM * a.NB);
    const int first_m = band * kBandM;
    const int bm_cnt = a.MB - first_m < kBandM ? a.MB - first_m : kBandM;
    const int in_band = t - band * kBandM * a.NB;
    const int64_t mb = first_m + in_band % bm_cnt, nb = in_band / bm_cnt;
    const int64_t m0 = mb * BM, n0 = nb * BN;
    // this split's k-range, in whole 128-k record blocks
    const int nblk = (a.nst + 3) / 4;
    const int blk0 = ksi * nblk / a.ks;
    const int blk1 = (ksi + 1) * nblk / a.ks;
    const int st0 = 4 * blk0;
    const int nst = (4 * blk1 < a.nst ? 4 * blk1 : a.nst) - st0;

    // ---- activation copies (as the bf16 GEMM's, 32-k stages) ----
    // block f = wave + NW j of a stage holds rows 16 f .. 16 f + 15; rows past
    // M read the last valid row (never stored)
    const char *xbase = reinterpret_cast<const char *>(a.X + m0 * a.ldx);
    const int arow = lane >> 2;
    const uint32_t chunk = 8 * ((lane & 3) ^ swz<4>(arow));
    const uint32_t aoff0 = ((uint32_t)(16 * wave + arow) * (uint32_t)a.ldx + chunk) * 2;
    const uint32_t astep = 16 * C::NW * (uint32_t)a.ldx * 2;
    const int64_t last_row = M - 1 - m0 < BM - 1 ? M - 1 - m0 : BM - 1;
    const uint32_t alim = ((uint32_t)last_row * (uint32_t)a.ldx + chunk) * 2;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(void __attribute__((address_space(3))) *)lds;
    const uint32_t ldsb = lds0 + C::NS * C::ASLOT;
    // copy j of stage kt into activation slot aslot
    auto copy_a = [&](int kt, int aslot, int j) __attribute__((always_inline)) {
        uint32_t o = aoff0;
        asm volatile("" : "+v"(o)); // recomputed per issue, not held
        o += (uint32_t)j * astep;
        dma16(xbase + (int64_t)(st0 + kt) * 64, o < alim ? o : alim,
              lds0 + aslot * C::ASLOT + (wave + C::NW * j) * 1024);
    };

    // ---- record copies: block b of the split (global block blk0 + b) ----
    // The members' record bases sit in an LDS table (a lone product: one
    // entry), so the block loop never reads the kernel arguments (a scalar
    // load there would drain the LDS reads in flight); the copies address
    // records with full 64-bit per-lane addresses.
    int KBm = a.KBm, tmax = a.Nt16 - 1;
    asm volatile("" : "+s"(KBm), "+s"(tmax));
    if (threadIdx.x < kSetParts)
        mtab[threadIdx.x] = a.R > 1 ? grp.segw[a.seg][threadIdx.x < a.R ? threadIdx.x : 0] : a.W;
    __syncthreads();
    const int t0 = (int)(n0 >> 4);
    // where block b's records start: the member holding global block
    // blk0 + b and the block's index within it
    auto block_src = [&](int b, int &lb) __attribute__((always_inline)) {
        const int gb = blk0 + b;
        const int r = gb / KBm;
        lb = gb - r * KBm;
        return mtab[r];
    };
    // copy c < BCW of this wave for a block into record slot bslot: the
    // first CCW copy the codes (1 KB) of records wave + NW c, the others the
    // (scale, bias) pairs of records 2 p, 2 p + 1 with p = wave + NW (c - CCW)
    auto copy_b = [&](const char *base, int lb, int bslot, int c) __attribute__((always_inline)) {
        const uint32_t dst = ldsb + bslot * C::BSLOT;
        if (c < C::CCW) {
            const int rr = wave + C::NW * c;
            const int nt = t0 + rr < tmax ? t0 + rr : tmax;
            const uint32_t off = (uint32_t)((nt * KBm + lb) * kQ4Record) + 16 * (uint32_t)lane;
            dma16_at(base + off, dst + rr * 1024);
        } else {
            const int p = wave + C::NW * (c - C::CCW);
            const int rr = 2 * p + (lane >> 5);
            const int nt = t0 + rr < tmax ? t0 + rr : tmax;
            const uint32_t off = (uint32_t)((nt * KBm + lb) * kQ4Record) + kQ4PairsAt +
                                 4 * (uint32_t)(lane & 31);
            dma4_at(base + off, dst + C::NR * 1024 + p * 256);
        }
    };
    // the batch of stage kt (the first NS stages): its record block's copies
    // when it opens one, then its activation copies
    auto issue = [&](int kt) __attribute__((always_inline)) {
        if ((kt & 3) == 0) {
            int lb;
            const char *base = block_src(kt >> 2, lb);
#pragma unroll
            for (int c = 0; c < C::BCW; ++c)
                copy_b(base, lb, (kt >> 2) % C::NBS, c);
        }
#pragma unroll
        for (int j = 0; j < C::ACW; ++j)
            copy_a(kt, kt % C::NS, j);
    };
    // wait until this wave's copies of stage kt have landed: batches kt + 1
    // .. last may still be in flight (in-order vmcnt); batch s holds ACW
    // copies, and BCW more when s = 0 mod 4
    auto wait_for = [&](int kt, int last) __attribute__((always_inline)) {
        const int y = last - kt;
        const int nbk = y > 0 ? (last >> 2) - (kt >> 2) : 0;
        const int code = y * 4 + nbk;
#define TSL_W(Y_, B_)                                                                              \
    case (Y_)*4 + (B_): wait_vmcnt<(Y_)*C::ACW + (B_)*C::BCW>(); break;
        switch (code) {
            TSL_W(0, 0) TSL_W(1, 0) TSL_W(1, 1) TSL_W(2, 0) TSL_W(2, 1) TSL_W(3, 0) TSL_W(3, 1)
            TSL_W(4, 1) TSL_W(5, 1) TSL_W(5, 2) TSL_W(6, 1) TSL_W(6, 2)
        default: wait_vmcnt<0>(); break;
        }
#undef TSL_W
    };

    // ---- column exponents (a joined set's: the largest of its members') ----
    int fcol[C::NT];
    {
        const size_t eoff = ((size_t)a.Nt16 * a.KBm * kQ4Record + 255) / 256 * 256;
#pragma unroll
        for (int j = 0; j < C::NT; ++j) {
            int64_t n = n0 + C::TN * wn + 32 * j + (lane & 31);
            n = n < (int64_t)a.Nt16 * 16 ? n : (int64_t)a.Nt16 * 16 - 1;
            int f = -1000;
            for (int r = 0; r < a.R; ++r) {
                const char *base = a.R > 1 ? grp.segw[a.seg][r] : a.W;
                const int fr = reinterpret_cast<const int32_t *>(base + eoff)[n];
                f = fr > f ? fr : f;
            }
            fcol[j] = f;
        }
    }

    f32x16 acc[C::MT][C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    // Fragments of a 16-k step: activations read from LDS, code words read
    // from LDS and expanded in registers.  Step g of the split is in stage
    // g / 2 and record block g / 8.
    u32x4 af[2][C::MT], bfr[2][C::NT];
    // bq[h][j]: column tile j's code words for the block's steps of parity
    // h (word t serves step 2 t + h), read once per block
    u32x4 bq[2][C::NT];
    uint32_t praw[C::NT], ss[C::NT], bb[C::NT];
    // the constants of the expansion, held opaquely so that each code pair
    // takes one v_and_or_b32 (gfx9 VOP3 encodings take no literal): nibble
    // pairs 0 and 2 of a word land on binary16 1024 + q (0x6400 | q), pairs
    // 1 and 3 on 64 + q (0x5400 | q << 4, the mantissa's unit there being
    // 1/16), so only pairs 2 and 3 need a shift, one for both
    uint32_t cmask, cmask4, cbias, cbias4;
    asm("v_mov_b32 %0, 0x000f000f" : "=v"(cmask));
    asm("v_mov_b32 %0, 0x00f000f0" : "=v"(cmask4));
    asm("s_mov_b32 %0, 0x64006400" : "=s"(cbias));
    asm("s_mov_b32 %0, 0x54005400" : "=s"(cbias4));
    // LDS reads for the step at position pos (0..7) of its record block,
    // from activation slot aslot and record slot bslot: at positions 0 and 1
    // the code words of the block's even / odd steps (one 16-byte read per
    // column tile: lanes 16 bytes apart, no bank conflicts), at positions 0
    // and 4 the columns' scale/bias pairs of the 64-k group the step opens,
    // then the activation fragments.  Lane parts of the read addresses are re-made opaque at
    // each use, so that the compiler does not hoist one address per unrolled
    // step out of the loop and run out of registers.
    const int rl = (lane & 31) >> 4;
    const uint32_t bw_lane = ((C::TN / 16) * wn + rl) * 1024 + ((lane >> 5) * 16 + (lane & 15)) * 16;
    const uint32_t bp_lane = C::NR * 1024 + ((C::TN / 16) * wn + rl) * 128 + (lane & 15) * 8;
    const int rb = lane & 15;
    uint32_t a_lane[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
        a_lane[s2] = (wm * C::MT * 2 + ((lane & 31) >> 4)) * 1024 + rb * 64 +
                     (((2 * s2 + (lane >> 5)) ^ swz<4>(rb)) * 16);
    auto read = [&](int pos, int aslot, int bslot, u32x4 (&x)[C::MT]) __attribute__((always_inline)) {
        uint32_t bw = bw_lane, bp = bp_lane, al = a_lane[pos & 1];
        asm volatile("" : "+v"(bw), "+v"(bp), "+v"(al));
        const char *Bs = lds + C::NS * C::ASLOT + bslot * C::BSLOT;
        if (pos < 2) {
#pragma unroll
            for (int j = 0; j < C::NT; ++j)
                bq[pos][j] = *reinterpret_cast<const u32x4 *>(Bs + bw + j * 2048 + pos * 512);
        }
        if ((pos & 3) == 0) {
#pragma unroll
            for (int j = 0; j < C::NT; ++j)
                praw[j] = *reinterpret_cast<const uint32_t *>(Bs + bp + j * 256 + (pos >> 2) * 4);
        }
        const char *As = lds + aslot * C::ASLOT;
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
            x[i] = *reinterpret_cast<const u32x4 *>(As + al + i * 2048);
    };
    // code word of column tile j for the step at position pos
    auto word = [&](int pos, int j) __attribute__((always_inline)) {
        const u32x4 v = (pos & 1) ? bq[1][j] : bq[0][j];
        const int t = pos >> 1;
        return t == 0 ? v[0] : t == 1 ? v[1] : t == 2 ? v[2] : v[3];
    };
    // part c of the expansion of the step at position pos: c == 0 converts
    // the group's scale/bias pairs (when the step opens a 64-k group),
    // c = 1 + 2 j + h expands code pairs
    // 2 h and 2 h + 1 of column tile j, interleaved; each result is pinned
    // where it is computed (otherwise the compiler sinks the expansion to
    // its first use, behind the MFMAs)
    constexpr int NC = 1 + 2 * C::NT;
    auto expand = [&](int pos, int c, u32x4 (&y)[C::NT]) __attribute__((always_inline)) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        if (c == 0) {
            if ((pos & 3) == 0) {
#pragma unroll
                for (int j = 0; j < C::NT; ++j) {
                    q4_pair(praw[j], fcol[j], ss[j], bb[j]);
                    asm volatile("" : "+v"(ss[j]), "+v"(bb[j]));
                }
            }
        } else {
            const int j = (c - 1) >> 1, h = (c - 1) & 1;
            const uint32_t wd = word(pos, j);
            const uint32_t w = h ? wd >> 8 : wd;
            const uint32_t v0 = (w & cmask) | cbias, v1 = (w & cmask4) | cbias4;
            const h2 o0 = {(_Float16)-1024.f, (_Float16)-1024.f};
            const h2 o1 = {(_Float16)-64.f, (_Float16)-64.f};
            const h2 q0 = __builtin_bit_cast(h2, v0) + o0, q1 = __builtin_bit_cast(h2, v1) + o1;
            const h2 s2 = __builtin_bit_cast(h2, ss[j]), b2 = __builtin_bit_cast(h2, bb[j]);
            uint32_t e0 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q0, s2, b2));
            uint32_t e1 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q1, s2, b2));
            asm volatile("" : "+v"(e0), "+v"(e1));
            y[j][2 * h] = e0;
            y[j][2 * h + 1] = e1;
        }
    };

    auto wrap = [](int x, int n) __attribute__((always_inline)) { return x >= n ? x - n : x; };
    const char *nbase = nullptr; // record source of the next block to copy
    int nlb = 0;
    // Stage kt: its two 16-k steps.  as_cur / as_nxt: activation slots of
    // stages kt and kt + 1; bs_cur / bs_nxt: their record slots; bdst: the
    // record slot of block (kt + NS) / 4.  P: kt mod 4 when known at
    // compile time (-1: not); COPY: the copies of stage kt + NS are issued
    // (into the slot of stage kt and, BCOPY, opening a block, record slot
    // bdst -- slots no wave reads any more).
    // (with P = -1 the copy flags are the run-time rcopy, rbcopy)
    auto stage = [&](int kt, int as_cur, int as_nxt, int bs_cur, int bs_nxt, int bdst, auto P,
                     auto COPY, auto BCOPY, bool rcopy, bool rbcopy) __attribute__((always_inline)) {
        constexpr int p = decltype(P)::value;
        const bool copy = p >= 0 ? decltype(COPY)::value : rcopy;
        const bool bcopy = p >= 0 ? decltype(BCOPY)::value : rbcopy;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // (step g = 2 kt + s) position of step g + 1 in its record block (a constant
            // in the steady state)
            const int pos1 = p >= 0 ? (2 * p + s + 1) & 7 : (2 * kt + s + 1) & 7;
            const int cur = s, nxt = s ^ 1; // buffers alternate by step parity
            if (s == 1) {
                // this wave's reads of stage kt have landed; stage kt + 1
                // (if any) is published
                wait_lgkm0();
                if constexpr (p >= 0) {
                    // steady state: NS - 2 younger batches, of which these
                    // open a record block
                    constexpr int nb = (p + C::NS - 1) / 4 - (p + 1) / 4;
                    wait_vmcnt<(C::NS - 2) * C::ACW + nb * C::BCW>();
                } else {
                    const int last = kt + C::NS - 1 < nst - 1 ? kt + C::NS - 1 : nst - 1;
                    wait_for(kt + 1, last);
                }
                barrier();
            }
            // the next block's source, one step ahead of its copies (an LDS
            // read, awaited with the stage's other reads)
            if (s == 0 && bcopy)
                nbase = block_src((kt + C::NS) >> 2, nlb);
            // the reads and expansion of step g + 1 -- after the last step
            // too, where they read stale LDS (in range) and their values go
            // unused, so that no step branches on them
            read(pos1, s == 0 ? as_cur : as_nxt, s == 0 ? bs_cur : bs_nxt, af[nxt]);
            // the MFMAs of step g; between them, the expansion of step g + 1
            // (starting one MFMA in, so that its LDS reads have landed) and,
            // at the last step of a stage, the copies
            constexpr int NMF = C::MT * C::NT;
            constexpr int TOT = C::BCW + C::ACW;
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                const int i = q / C::NT, j = q % C::NT;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, af[cur][i]), __builtin_bit_cast(f16x8, bfr[cur][j]),
                    acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (q >= 1) {
#pragma unroll
                    for (int c = (q - 1) * NC / (NMF - 1); c < q * NC / (NMF - 1); ++c)
                        expand(pos1, c, bfr[nxt]);
                }
                if (s == 1 && copy) {
#pragma unroll
                    for (int f = q * TOT / NMF; f < (q + 1) * TOT / NMF; ++f) {
                        if (f < C::BCW) {
                            if (bcopy)
                                copy_b(nbase, nlb, bdst, f);
                        } else {
                            copy_a(kt + C::NS, as_cur, f - C::BCW);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (nst > 0) {
        for (int k = 0; k < C::NS && k < nst; ++k)
            issue(k);
        wait_for(0, (C::NS < nst ? C::NS : nst) - 1);
        barrier();
        read(0, 0, 0, af[0]);
#pragma unroll
        for (int c = 0; c < NC; ++c)
            expand(0, c, bfr[0]);
        using T = std::true_type;
        using F = std::false_type;
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using IN = std::integral_constant<int, -1>;
        // record blocks opened by the copies at each position of a block
        constexpr bool B0 = (0 + C::NS) % 4 == 0, B1 = (1 + C::NS) % 4 == 0;
        constexpr bool B2 = (2 + C::NS) % 4 == 0, B3 = (3 + C::NS) % 4 == 0;
        int kt = 0, as0 = 0, bs0 = 0; // stage, its activation slot, its record slot
        // steady state: whole record blocks whose four stages all issue the
        // copies of stage kt + NS
        for (; kt + 3 + C::NS < nst; kt += 4) {
            const int a1 = wrap(as0 + 1, C::NS), a2 = wrap(as0 + 2, C::NS);
            const int a3 = wrap(as0 + 3, C::NS), a4 = wrap(as0 + 4, C::NS);
            const int bn = wrap(bs0 + 1, C::NBS);
            const int d0 = wrap(bs0 + (0 + C::NS) / 4, C::NBS), d1 = wrap(bs0 + (1 + C::NS) / 4, C::NBS);
            const int d2 = wrap(bs0 + (2 + C::NS) / 4, C::NBS), d3 = wrap(bs0 + (3 + C::NS) / 4, C::NBS);
            stage(kt, as0, a1, bs0, bs0, d0, I0{}, T{}, std::integral_constant<bool, B0>{}, true,
                  true);
            stage(kt + 1, a1, a2, bs0, bs0, d1, I1{}, T{}, std::integral_constant<bool, B1>{}, true,
                  true);
            stage(kt + 2, a2, a3, bs0, bs0, d2, I2{}, T{}, std::integral_constant<bool, B2>{}, true,
                  true);
            stage(kt + 3, a3, a4, bs0, bn, d3, I3{}, T{}, std::integral_constant<bool, B3>{}, true,
                  true);
            as0 = a4;
            bs0 = bn;
        }
        // the rest, one stage at a time
        for (; kt < nst; ++kt) {
            const int a1 = wrap(as0 + 1, C::NS);
            const int bn = (kt & 3) == 3 ? wrap(bs0 + 1, C::NBS) : bs0;
            const int bd = ((kt + C::NS) >> 2) % C::NBS;
            const bool cp = kt + C::NS < nst;
            stage(kt, as0, a1, bs0, bn, bd, IN{}, F{}, F{}, cp, cp && ((kt + C::NS) & 3) == 0);
            as0 = a1;
            bs0 = bn;
        }
    }

    // ---- epilogue: acc reg r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32 ----
    const int64_t row0 = m0 + wm * C::TM + 4 * (lane >> 5);
    const int64_t col0 = n0 + C::TN * wn + (lane & 31);
    const bool part = a.ks > 1;
    const bool ybf = part ? false : (a.flags & kQ4YBf16) != 0;
    const bool accu = part ? false : (a.flags & kQ4Accumulate) != 0;
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
    // row exponents: per 32-row block one load (lane l takes row l of the
    // block; the exponents are padded to whole 256-row tiles), issued before
    // the first store (vmcnt counts stores too); each lane then reads its
    // rows, 4 (lane / 32) apart, from the lanes that hold them
    int rblk[C::MT];
    {
        const int32_t *re = reinterpret_cast<const int32_t *>(a.X + M * a.ldx);
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
            rblk[i] = re[m0 + wm * C::TM + i * 32 + (lane & 31)];
    }
    const bool hi_half = (lane >> 5) != 0;
#pragma unroll
    for (int i = 0; i < C::MT; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = i * 32 + 8 * (r >> 2) + (r & 3); // row step from row0
            if (row0 + rr >= M)
                continue;
            char *yr = ybase + rr * rstride;
            const int q = 8 * (r >> 2) + (r & 3);
            const int lo_e = __builtin_amdgcn_readlane(rblk[i], q);
            const int hi_e = __builtin_amdgcn_readlane(rblk[i], q + 4);
            const int rexp = hi_half ? hi_e : lo_e;
#pragma unroll
            for (int j = 0; j < C::NT; ++j) {
                if (!colok[j])
                    continue;
                // undo the operand scales: one exact power-of-two step
                // (rounded only where the result leaves the normal range)
                const float v = __builtin_amdgcn_ldexpf(acc[i][j][r], rexp + fcol[j]);
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
}

typedef void (*Q4Fn)(Q4Group);

// the kernel of a tile shape and its workgroup size: 256 x 256 and
// 128 x 256 tiles run eight waves (two per SIMD, so that one covers the
// other's stalls), the others four (two workgroups per CU where the LDS
// holds them)
Q4Fn pick_q4(int bm, int bn, int *threads) {
#define TSL_Q4(BM_, BN_, WM_, WN_)                                                                 \
    if (bm == BM_ && bn == BN_) {                                                                  \
        *threads = 64 * WM_ * WN_;                                                                 \
        return q4_gemm_kernel<BM_, BN_, WM_, WN_>;                                                 \
    }
    TSL_Q4(256, 256, 2, 4) TSL_Q4(256, 128, 1, 4) TSL_Q4(128, 256, 2, 4) TSL_Q4(128, 128, 1, 4)
    TSL_Q4(64, 256, 1, 4) TSL_Q4(64, 128, 1, 4)
#undef TSL_Q4
    return nullptr;
}

} // namespace

hipError_t launch_q4_gemm(const PrefillPlan &p, const LinearItem *items, int n, const char *ws,
                          hipStream_t stream) {
    int threads = 0;
    Q4Fn fn = pick_q4(p.bm, p.bn, &threads);
    if (!fn)
        return hipErrorInvalidValue;
    for (int c0 = 0; c0 < n;) {
        Q4Group grp{};
        int joined = 0;
        int64_t blocks = 0;
        const int c1 = prefill_chunk_end(items, n, c0);
        int c = c0;
        for (; c < c1; ++c) {
            const LinearItem &L = items[c];
            const PackGeom &g = L.g;
            Q4Item &a = grp.it[grp.n++];
            a.R = L.cat;
            a.seg = -1;
            if (L.cat > 1) {
                a.seg = joined++;
                for (int r = 0; r < L.cat; ++r)
                    grp.segw[a.seg][r] = static_cast<const char *>(L.seg_packed[r]);
            } else {
                a.W = static_cast<const char *>(L.packed);
            }
            a.X = reinterpret_cast<const uint16_t *>(ws + p.x_off[c]);
            a.ldx = (int32_t)((g.Ks + 63) / 64 * 64);
            a.Y = L.Y;
            a.ldy = L.ldy;
            a.M = (int32_t)L.M;
            a.Ns = (int32_t)g.Ns;
            a.Nt16 = (int32_t)g.Nt;
            a.KBm = (int32_t)(g.KT / L.cat);
            a.nst = (int32_t)(g.Ks / 32);
            a.MB = (int32_t)((L.M + p.bm - 1) / p.bm);
            a.NB = (int32_t)((g.Ns + p.bn - 1) / p.bn);
            a.ks = p.ks[c];
            a.P = reinterpret_cast<float *>(const_cast<char *>(ws) + p.p_off[c]);
            a.start = (int32_t)blocks;
            a.flags = (L.ydtype == TSL_BF16 ? kQ4YBf16 : 0) | (L.accumulate ? kQ4Accumulate : 0);
            blocks += (int64_t)a.MB * a.NB * a.ks;
        }
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(threads), 0, stream, grp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        c0 = c;
    }
    return hipSuccess;
}

} // namespace tsl
