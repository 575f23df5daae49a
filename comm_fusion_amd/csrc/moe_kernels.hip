// moe_kernels.hip -- gfx950 (MI355X) kernels of the MoE expert path with the
// Combine exchange fused into the Linear-2 epilogue.
//
// Method (X-Stage paper, arXiv 2607.23264; arXiv abstract page, Abstract;
// pith.science review page, "If this is right" and Figs. 4, 8, 9): a rank
// runs its local experts' Linear-1 and Linear-2 on the tokens routed to it;
// the owner of each Linear-2 output tile stores it into the Combine slots of
// the tokens' source ranks (on one GPU: P regions of one buffer) and moves
// on.  The schedule -- which tiles run between those store bursts -- is set
// by the host (moe_launch): Expert-Wave runs each wave's Linear-1 tiles, then
// its Linear-2 tiles; the interleaved schedule runs wave w's Linear-2 tiles
// interleaved with wave w+1's Linear-1 tiles in one launch.
//
// Design for CDNA4:
//  * one kernel for both layers: a workgroup of 8 wave64s (two per SIMD)
//    computes a tile of 256 output features x 256 token rows, each wave
//    128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (six operand reads
//    per eight MFMAs), over k-steps of 64 (four substeps of 16);
//  * outputs are computed transposed, C^T = W X^T: the weight rows are the A
//    operand and the token rows the B operand, so every lane holds one token
//    row and 16 of its features per block (runs of 4 consecutive features);
//  * operand tiles go global -> LDS directly (buffer loads into the LDS, no
//    VGPR staging, no vector instruction per copy): weight tiles
//    (mostly from HBM) through three stages, copied two k-steps ahead, token
//    tiles (mostly L2 hits) through two, one step ahead; one barrier per
//    step of 32 MFMAs per wave; the operand reads are explicit LDS
//    instructions issued a k-substep ahead;
//  * Linear-1 tiles take 128 gate rows and the 128 matching up rows of W1,
//    arranged so that each wave's feature blocks hold gate and up of the
//    same intermediate columns: SiLU(gate) * up is formed in registers;
//  * token rows are gathered through row_slot (slot / k is the token), so the
//    dispatch exchange's receive side is read in place;
//  * the Linear-2 epilogue multiplies each row by its routing weight, rounds
//    to bf16, stages the tile in the LDS and stores whole 512-byte row
//    segments (16 bytes per lane) into each row's Combine slot;
//  * a wave skips the MFMAs and operand reads of its 32-row token blocks
//    that lie past its expert's last row (a partial tile still copies its
//    weight slice and meets every barrier);
//  * the persistent form runs a whole schedule in one launch: workgroups
//    take tiles in schedule order from a device queue, and a Linear-2 tile
//    first waits (bounded) until the Linear-1 tiles of its token rows have
//    counted themselves done (moe_persist, below).
#include "moe_internal.h"
#include "ua_internal.h"

#include <algorithm>
#include <type_traits>
#include <utility>
#include <vector>

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

constexpr int BM = 256;                 // token rows per tile
constexpr int BF = 256;                 // feature rows per tile (Linear-1: 128 gate + 128 up)
constexpr int BK = 64;                  // k per step
constexpr int NSTAGE_W = 3;             // weight tile stages: copies run two steps ahead
constexpr int NSTAGE_X = 2;             // token tile stages: copies run one step ahead
constexpr int NW = 8;                   // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int TILE = 256 * BK * 2;      // bytes of one operand tile (32 KiB)
constexpr int LDS_BYTES = (NSTAGE_W + NSTAGE_X) * TILE;  // 160 KiB
constexpr int NCPW = TILE / 1024 / NW;  // 1 KiB copies per wave per operand tile
constexpr int L1_COLS = 128;            // intermediate columns per Linear-1 tile
constexpr int L2_COLS = 256;            // hidden columns per Linear-2 tile

typedef __attribute__((address_space(3))) void lds_void;
// word 3 of a raw buffer descriptor (gfx9: 32-bit data format, no swizzle)
constexpr int kBufferFlags = 0x00020000;

// One expert's tiles of one kind in a launch.
struct Seg {
    int32_t kind;    // 0: Linear-1 (+ activation), 1: Linear-2 (+ Combine)
    int32_t expert;  // local expert
    int32_t row0;    // its first receive row
    int32_t rows;    // its receive rows
    int32_t mtiles;  // token tiles, ceil(rows / BM)
    int32_t ntiles;  // feature tiles
    int32_t tile0;   // first tile of the segment among its kind's tiles in the launch (or phase)
    int32_t tt0;     // its first token tile among the call's token tiles (persistent form)
};

struct MoeArgs {
    Seg seg[2 * kMaxWave];
    int32_t nseg;
    int32_t n_l1, n_l2;   // tiles of each kind in the launch
    int32_t k, hidden, inter;
    int32_t out_local;    // 1: Linear-2 writes receive row i (y_local); 0: its Combine slot
    int32_t n_xcd;        // XCDs of the device
    const uint16_t *x;
    const int32_t *row_slot;
    const float *topk_w;
    const uint16_t *w1;
    const uint16_t *w2;
    uint16_t *act;
    uint16_t *out;
};

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi)
{
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, RNE
    return __builtin_bit_cast(unsigned, h);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// MFMA operand reads from the LDS as explicit instructions with
// compile-time offsets, each waited for exactly (lgkm_wait) before the MFMAs
// that consume it: the compiler does not see them, so it inserts no waits of
// its own -- none on the global->LDS copies into the other stage, which it
// could not tell apart from these reads.  The wait is tied to the fragment
// registers, so nothing may copy or reuse them before it.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read(unsigned addr)
{
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int N, int NB>
__device__ __forceinline__ void lgkm_wait(u32x4 (&fa)[4], u32x4 (&fb)[2])
{
    if constexpr (NB > 1)
        asm volatile("s_waitcnt lgkmcnt(%6)"
                     : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1])
                     : "i"(N));
    else
        asm volatile("s_waitcnt lgkmcnt(%5)"
                     : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0])
                     : "i"(N));
}

// One output tile: 256 features x 256 token rows, K in steps of 64.
// Operand tiles in the LDS: [row][128 B] (the step's 64 k values), the eight
// 16-byte chunks of a row at positions chunk ^ ((row / 2) % 8), so that a
// fragment read (16 rows per quarter-wave, one chunk each) spreads over all
// banks.  Weight stage w sits at w * TILE (w = 0, 1, 2), token stage x at
// (3 + x) * TILE.  The tiles are filled by 1 KiB global->LDS copies (lane L
// of copy c lands at byte 1024 c + 16 L: row 8 c + L / 8, position L % 8,
// fetching chunk (L % 8) ^ (4 (c % 2) + L / 16)): as step s starts, the
// token tile of step s+1 and then the weight tile of step s+2.  Wave (wf, wt)
// computes features 128 wf .. +127 (four 32-row blocks) of the token blocks
// wt and wt + 4 (rows 32 wt .. +31 and 128 + 32 wt .. +31), so that the
// rows of a partial tile (an expert's last) spread over all waves.  A token
// block that lies wholly past the expert's rows is skipped: no fragment
// reads, no MFMAs (and no copies of its rows).
template <int KIND, bool COH>
__device__ __forceinline__ void tile(const MoeArgs &a, const Seg &sg, int m, int n, lds_u8 *lds)
{
    // COH: act rows (Linear-2's token operand) are read at device scope
    // (sc1), past any copy of them in this XCD's L2: in the persistent form
    // they were written by other workgroups of the same launch.
    constexpr int XAUX = KIND == 1 && COH ? 16 : 0;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wf = wave & 1, wt = wave >> 1;
    const int l32 = lane & 31, g = lane >> 5;
    const int K = KIND == 0 ? a.hidden : a.inter;
    const int nk = K / BK;  // K is a multiple of 128: nk is even
    const char *wbase = (const char *)(KIND == 0 ? a.w1 + (int64_t)sg.expert * 2 * a.inter * a.hidden
                                                 : a.w2 + (int64_t)sg.expert * a.hidden * a.inter);
    const char *bbase = (const char *)(KIND == 0 ? a.x : a.act);
    // rows of this tile inside the expert; this wave's token blocks among them
    const int vrows = min(BM, sg.rows - m * BM);
    const int nb = (32 * wt < vrows) + (128 + 32 * wt < vrows);
    const bool xcopy = 32 * wave < vrows;  // this wave copies token rows 32 wave .. +31

    // This wave's copies: numbers NCPW wave .. of each operand tile.
    static_assert(NCPW % 2 == 0, "copy parity is the copy index's parity");
    unsigned aoff[NCPW], boff[NCPW];
#pragma unroll
    for (int i = 0; i < NCPW; ++i) {
        const int c = NCPW * wave + i;
        const int r = 8 * c + (lane >> 3);
        const unsigned chunk16 = (unsigned)((lane & 7) ^ (4 * (i & 1) + (lane >> 4))) * 16;
        // weight row of tile row r: Linear-1 rows 128 h .. 128 h + 63 are gate
        // rows 128 n + 64 h .., rows 128 h + 64 .. the matching up rows, so a
        // wave's feature blocks 0, 1 (gate) and 2, 3 (up) hold the same
        // intermediate columns; Linear-2 takes hidden rows 256 n + r
        const int h = r >> 7, q = r & 127;
        const int wrow = KIND == 0 ? (q < 64 ? L1_COLS * n + 64 * h + q : a.inter + L1_COLS * n + 64 * h + q - 64)
                                   : L2_COLS * n + r;
        aoff[i] = (unsigned)wrow * (unsigned)K * 2 + chunk16;
        // token row: rows past the expert's end repeat its last row (not stored)
        const int rl = m * BM + r < sg.rows ? m * BM + r : sg.rows - 1;
        const int ri = sg.row0 + rl;
        const unsigned brow = KIND == 0 ? (unsigned)(a.row_slot[ri] / a.k) : (unsigned)ri;
        boff[i] = brow * (unsigned)K * 2 + chunk16;
    }
    // weight tile of step s into weight stage w; token tile into token stage x
    // Buffer loads into the LDS: the operand's base in a descriptor, the
    // lane's 32-bit offset, and the step's k offset as the scalar offset, so
    // a copy costs no vector instruction.  The descriptor's range is the
    // whole 32-bit offset space (no clipping): the host keeps every offset
    // of an operand below 2^32.
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void *)wbase, (short)0, -1, kBufferFlags);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc((void *)bbase, (short)0, -1, kBufferFlags);
    auto copy_w = [&](int s, int w) {
        lds_u8 *dst = lds + w * TILE + NCPW * wave * 1024;
#pragma unroll
        for (int i = 0; i < NCPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void *)(dst + i * 1024), 16, aoff[i], s * BK * 2, 0, 0);
    };
    auto copy_x = [&](int s, int x) {
        if (!xcopy) return;
        lds_u8 *dst = lds + (NSTAGE_W + x) * TILE + NCPW * wave * 1024;
#pragma unroll
        for (int i = 0; i < NCPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void *)(dst + i * 1024), 16, boff[i], s * BK * 2, 0, XAUX);
    };

    // Per-lane LDS addresses of the fragment reads, one per k-substep KK
    // (0..3); stage and block are instruction offsets.  Fragment element
    // layout: lane l gives row (block + l % 32), k values 16 KK + 8 (l / 32)
    // .. +7, i.e. chunk 2 KK + l / 32, at position chunk ^ ((l % 32 / 2) % 8).
    const unsigned lbase = (unsigned)(uintptr_t)lds;
    const unsigned sw = (unsigned)((l32 >> 1) & 7);
    const unsigned ra = lbase + (unsigned)(128 * wf + l32) * 128;
    const unsigned rb = lbase + NSTAGE_W * TILE + (unsigned)(32 * wt + l32) * 128;
    // weight stage 2 through its own bases (offset past the 16-bit field)
    unsigned pa[4], pa2[4], pb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        pa[kk] = ra + (((unsigned)(2 * kk + g) ^ sw) * 16);
        pa2[kk] = pa[kk] + 2 * TILE;
        pb[kk] = rb + (((unsigned)(2 * kk + g) ^ sw) * 16);
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fb][tb][r] = 0.f;

    // Fragment registers: three sets.  A set is read into again only once
    // the MFMAs of another set were issued after its own, which have
    // therefore started and taken their operands.
    u32x4 fa[3][4], fbr[3][2];
    // the fragment reads of k-substep KK of weight stage WS and token stage
    // XS into set SET: four weight blocks and this wave's NB token blocks
    auto reads = [&](auto nbc, auto wsc, auto xsc, auto kkc, auto setc) {
        constexpr int NB = decltype(nbc)::value, WS = decltype(wsc)::value, XS = decltype(xsc)::value;
        constexpr int KK = decltype(kkc)::value, SET = decltype(setc)::value;
        constexpr int OA = (WS & 1) * TILE, OB = XS * TILE;
        const unsigned p = WS == 2 ? pa2[KK] : pa[KK];
        u32x4 (&da)[4] = fa[SET];
        u32x4 (&db)[2] = fbr[SET];
        da[0] = lds_read<OA + 0 * 4096>(p);
        da[1] = lds_read<OA + 1 * 4096>(p);
        da[2] = lds_read<OA + 2 * 4096>(p);
        da[3] = lds_read<OA + 3 * 4096>(p);
        db[0] = lds_read<OB>(pb[KK]);
        if constexpr (NB > 1) db[1] = lds_read<OB + 128 * 128>(pb[KK]);
    };
    auto mfmas = [&](auto nbc, u32x4 (&da)[4], u32x4 (&db)[2]) {
        constexpr int NB = decltype(nbc)::value;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb)
                acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, da[fb]), __builtin_bit_cast(bf16x8, db[tb]), acc[fb][tb], 0, 0, 0);
    };
    // One k-step on weight stage s % 3 and token stage s % 2.  Its copies
    // (weights issued as step s-2 started, tokens as step s-1 started,
    // before the weights of step s+1) have landed once at most the weight
    // copies of step s+1 remain in flight; after the barrier every wave's
    // have, and every wave is done with step s-1, whose stages take the
    // token tile of step s+1 and the weight tile of step s+2.  Each
    // substep's reads are issued before the previous substep's MFMAs; all
    // are waited for within the step.  PH = s % 3 also picks the fragment
    // register sets (substep 4 s + j uses set (PH + j) % 3).  NB: this
    // wave's token blocks inside the expert (a wave with none still copies
    // and meets every barrier).
    auto step = [&](auto nbc, int s, auto xsc, auto phc) {
        constexpr int NB = decltype(nbc)::value, NR = 4 + NB;  // reads per substep
        constexpr int XS = decltype(xsc)::value, PH = decltype(phc)::value;
        using WS = std::integral_constant<int, PH>;
        constexpr int A = PH % 3, B = (PH + 1) % 3, C = (PH + 2) % 3;  // sets of substeps 0 (and 3), 1, 2
        using K0 = std::integral_constant<int, 0>;
        using K1 = std::integral_constant<int, 1>;
        using K2 = std::integral_constant<int, 2>;
        using K3 = std::integral_constant<int, 3>;
        using SA = std::integral_constant<int, A>;
        using SB = std::integral_constant<int, B>;
        using SC = std::integral_constant<int, C>;
        if (s + 1 < nk)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(NCPW) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (s + 1 < nk) copy_x(s + 1, XS ^ 1);
        if (s + 2 < nk) copy_w(s + 2, (PH + 2) % 3);
        if constexpr (NB > 0) {
            reads(nbc, WS(), xsc, K0(), SA());
            reads(nbc, WS(), xsc, K1(), SB());
            lgkm_wait<NR, NB>(fa[A], fbr[A]);
            mfmas(nbc, fa[A], fbr[A]);
            __builtin_amdgcn_sched_barrier(0);
            reads(nbc, WS(), xsc, K2(), SC());
            lgkm_wait<NR, NB>(fa[B], fbr[B]);
            mfmas(nbc, fa[B], fbr[B]);
            __builtin_amdgcn_sched_barrier(0);
            reads(nbc, WS(), xsc, K3(), SA());
            lgkm_wait<NR, NB>(fa[C], fbr[C]);
            mfmas(nbc, fa[C], fbr[C]);
            __builtin_amdgcn_sched_barrier(0);
            lgkm_wait<0, NB>(fa[A], fbr[A]);
            mfmas(nbc, fa[A], fbr[A]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: the weight and token tiles of step 0, the weight tile of
    // step 1; then the steps, six at a time (stages and register sets fixed
    // at compile time), and the last 0, 2 or 4 (nk is even)
    copy_w(0, 0);
    copy_x(0, 0);
    copy_w(1, 1);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    auto loop = [&](auto nbc) {
        int s = 0;
        for (; s + 6 <= nk; s += 6) {
            step(nbc, s, S0(), P0());
            step(nbc, s + 1, S1(), P1());
            step(nbc, s + 2, S0(), P2());
            step(nbc, s + 3, S1(), P0());
            step(nbc, s + 4, S0(), P1());
            step(nbc, s + 5, S1(), P2());
        }
        if (s < nk) {
            step(nbc, s, S0(), P0());
            step(nbc, s + 1, S1(), P1());
        }
        if (s + 2 < nk) {
            step(nbc, s + 2, S0(), P2());
            step(nbc, s + 3, S1(), P0());
        }
    };
    if (nb == 2)
        loop(std::integral_constant<int, 2>());
    else if (nb == 1)
        loop(std::integral_constant<int, 1>());
    else
        loop(std::integral_constant<int, 0>());
    // every wave is done with the operand tiles (the Linear-2 epilogue reuses the LDS)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // Accumulator register r of block (fb, tb) is feature 8(r/4) + 4g + r%4 of
    // the block, token row l32 of the block.
    if constexpr (KIND == 0) {
        // SiLU(gate) * up -> act[row][128 n + 64 wf + ...], bf16
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int rl = m * BM + 32 * (wt + 4 * tb) + l32;
            if (rl >= sg.rows) continue;
            uint16_t *dst = a.act + (int64_t)(sg.row0 + rl) * a.inter + L1_COLS * n + 64 * wf + 4 * g;
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = silu(acc[fb][tb][4 * q4 + e]) * acc[fb + 2][tb][4 * q4 + e];
                    u32x2 w;
                    w[0] = pack_bf16(v[0], v[1]);
                    w[1] = pack_bf16(v[2], v[3]);
                    *(u32x2 *)(dst + 32 * fb + 8 * q4) = w;
                }
        }
    } else {
        // weighted rows, staged as [token row][256 features] (chunk c of row
        // r at position c ^ (r % 32)), then stored as whole 512-byte rows
        float wrow[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int rl = m * BM + 32 * (wt + 4 * tb) + l32;
            wrow[tb] = rl < sg.rows ? a.topk_w[a.row_slot[sg.row0 + rl]] : 0.f;
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int tr = 32 * (wt + 4 * tb) + l32;
#pragma unroll
            for (int fb = 0; fb < 4; ++fb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int c = 16 * wf + 4 * fb + q4;
                    u32x2 w;
                    w[0] = pack_bf16(acc[fb][tb][4 * q4] * wrow[tb], acc[fb][tb][4 * q4 + 1] * wrow[tb]);
                    w[1] = pack_bf16(acc[fb][tb][4 * q4 + 2] * wrow[tb], acc[fb][tb][4 * q4 + 3] * wrow[tb]);
                    *(lds_u32x2 *)(lds + tr * 512 + ((c ^ (tr & 31)) << 4) + 8 * g) = w;
                }
        }
        __syncthreads();
        const int chunk = lane & 31;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int tr = 32 * wave + 2 * j + (lane >> 5);
            const u32x4 v = *(const lds_u32x4 *)(lds + tr * 512 + ((chunk ^ (tr & 31)) << 4));
            const int rl = m * BM + tr;
            if (rl < sg.rows) {
                const int ri = sg.row0 + rl;
                const int64_t orow = a.out_local ? (int64_t)ri : (int64_t)a.row_slot[ri];
                *(u32x4 *)(a.out + orow * a.hidden + L2_COLS * n + chunk * 8) = v;
            }
        }
    }
}

// Workgroup i is dispatched to XCD i % nx; give each XCD a contiguous run
// of the launch's tile sequence, so that the token tiles sharing a weight
// slice (neighbours in the sequence) run on one XCD and share its L2.  A
// bijection on [0, n).
__device__ __forceinline__ int64_t xcd_block(int64_t bid, int64_t n, int64_t nx)
{
    const int64_t xcd = bid % nx, k = bid / nx;
    const int64_t q = n / nx, r = n % nx;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// Position b of the tile sequence of a launch with n_l2 Linear-2 and n_l1
// Linear-1 tiles: the kinds are dealt in proportion to their counts
// (position b is a Linear-2 tile when floor((b+1) n_l2 / N) > floor(b n_l2 /
// N)), so in a mixed launch every stretch of the sequence holds both kinds;
// then the segment and its (token tile, feature tile), feature tiles
// outermost so that neighbours share the weight slice.
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void moe_tiles(MoeArgs a)
{
    __shared__ __attribute__((aligned(1024))) unsigned char lds_all[LDS_BYTES];  // 160 KiB: one workgroup per CU
    static_assert(LDS_BYTES >= BM * 512, "the Linear-2 epilogue stages 256 rows of 512 bytes");
    lds_u8 *const lds = (lds_u8 *)lds_all;
    const int64_t N = (int64_t)a.n_l1 + a.n_l2;
    const int64_t b = xcd_block(blockIdx.x, N, a.n_xcd);
    const int64_t c2 = b * a.n_l2 / N, c2n = (b + 1) * a.n_l2 / N;
    const int kind = c2n > c2 ? 1 : 0;
    const int idx = kind ? (int)c2 : (int)(b - c2);
    int si = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const Seg &s = a.seg[i];
        if (s.kind == kind && idx >= s.tile0 && idx < s.tile0 + s.mtiles * s.ntiles) si = i;
    }
    const Seg sg = a.seg[si];
    const int t = idx - sg.tile0;
    const int nn = t / sg.mtiles, mm = t - nn * sg.mtiles;
    if (kind == 0)
        tile<0, false>(a, sg, mm, nn, lds);
    else
        tile<1, false>(a, sg, mm, nn, lds);
}

// ---- persistent form: one launch runs the whole schedule.  The schedule is
// a sequence of phases (Expert-Wave: Linear-1 of wave 0, Linear-2 of wave 0,
// Linear-1 of wave 1, ...; interleaved: Linear-1 of wave 0, then Linear-2 of
// wave w-1 dealt between Linear-1 of wave w, ..., then the last Linear-2),
// each dealt like one launch above.  Workgroups take queue positions in
// order from one device counter, so long and short tiles pack over the CUs
// as they free up instead of ending at each launch's tail.  (One queue per
// XCD, each taking its XCD's run of every phase as the launch form maps
// blocks, kept token tiles that share a weight slice in one L2 but ran
// slower: a phase then ends at different times on different XCDs, and the
// Linear-2 tiles of the next wait for the slowest.)  A Linear-2 tile
// waits until all Linear-1 tiles of its token tile have stored their act
// rows: each Linear-1 tile counts itself (release add) once every wave's
// stores are complete; the Linear-2 tile's thread 0 polls the count at
// device scope, bounded, then acquires, and the tile reads act at device
// scope (sc1, past any line of it in this XCD's L2).  The
// Linear-1 tiles a Linear-2 tile waits for sit earlier in the queue, were
// taken by running workgroups, and never wait themselves, so the waits end.

struct Phase {
    int32_t start;               // first queue position of the phase
    int32_t seg_begin, seg_end;  // its segments in PersistArgs::m.seg
    int32_t n_l1, n_l2;          // tiles of each kind in the phase
};

constexpr int kMaxPhase = 2 * kMaxWave + 1;
constexpr unsigned kSpinLimit = 1u << 20;  // polls of a ready count before giving up

struct PersistArgs {
    MoeArgs m;          // operands and the segments of every phase
    Phase ph[kMaxPhase];
    int32_t nph;
    int32_t n_tiles;    // queue positions
    uint32_t l1_cols;   // Linear-1 tiles per token tile (inter / 128): the count a Linear-2 tile waits for
    unsigned *queue;    // this launch's position counter (zero at the start)
    unsigned *timeouts; // bounded waits that gave up (stays zero)
    unsigned *ready;    // per token tile: Linear-1 tiles done
};

static_assert(sizeof(PersistArgs) <= 4096, "kernel arguments");

__global__ __launch_bounds__(256) void clear_words(unsigned *p, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void moe_persist(PersistArgs a)
{
    __shared__ __attribute__((aligned(1024))) unsigned char lds_all[LDS_BYTES];
    lds_u8 *const lds = (lds_u8 *)lds_all;
    typedef __attribute__((address_space(3))) int lds_i32;
    lds_i32 *const pos_slot = (lds_i32 *)lds_all;
    for (;;) {
        __syncthreads();  // every wave is done with the previous tile's LDS
        if (threadIdx.x == 0) *pos_slot = (int)atomicAdd(a.queue, 1u);
        __syncthreads();
        const int t = __builtin_amdgcn_readfirstlane(*pos_slot);  // uniform: the decode below stays scalar
        __syncthreads();  // read by every wave before the tile's copies land
        if (t >= a.n_tiles) return;
        int k = 0;
        while (k + 1 < a.nph && a.ph[k + 1].start <= t) ++k;
        const Phase ph = a.ph[k];
        const int64_t N = (int64_t)ph.n_l1 + ph.n_l2, b = t - ph.start;
        const int64_t c2 = b * ph.n_l2 / N, c2n = (b + 1) * ph.n_l2 / N;
        const int kind = c2n > c2 ? 1 : 0;
        const int idx = kind ? (int)c2 : (int)(b - c2);
        int si = ph.seg_begin;
        for (int i = ph.seg_begin; i < ph.seg_end; ++i) {
            const Seg &s = a.m.seg[i];
            if (s.kind == kind && idx >= s.tile0 && idx < s.tile0 + s.mtiles * s.ntiles) si = i;
        }
        const Seg sg = a.m.seg[si];
        const int tt = idx - sg.tile0;
        const int nn = tt / sg.mtiles, mm = tt - nn * sg.mtiles;
        const int rci = sg.tt0 + mm;  // this token tile's ready count
        if (kind == 0) {
            tile<0, true>(a.m, sg, mm, nn, lds);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's act stores are complete
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(a.ready + rci, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            unsigned *const rc = a.ready + rci;
            if (threadIdx.x == 0) {
                for (unsigned it = 0; __hip_atomic_load(rc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.l1_cols;
                     ++it) {
                    if (it >= kSpinLimit) {
                        atomicAdd(a.timeouts, 1u);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                // pairs with the Linear-1 tiles' release adds
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();  // the act reads follow thread 0's acquire
            tile<1, true>(a.m, sg, mm, nn, lds);
        }
    }
}

// Serial Combine: one 16-byte chunk per thread, row i of y_local to slot
// row_slot[i] of the Combine buffer.
__global__ __launch_bounds__(256) void scatter_rows(const uint16_t *src, const int32_t *row_slot, int64_t n_chunks,
                                                    int32_t chunks_per_row, uint16_t *dst)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n_chunks) return;
    const int64_t row = c / chunks_per_row;
    const int64_t w = c - row * chunks_per_row;
    *(u32x4 *)(dst + ((int64_t)row_slot[row] * chunks_per_row + w) * 8) = *(const u32x4 *)(src + c * 8);
}

// Append expert e's tiles of `kind` to a launch (or a phase).
void add_seg(MoeArgs &a, const Problem &p, int e, int kind, int32_t tt0 = 0)
{
    const int64_t rows = p.offsets[e + 1] - p.offsets[e];
    if (rows == 0) return;
    Seg &s = a.seg[a.nseg++];
    s.tt0 = tt0;
    s.kind = kind;
    s.expert = e;
    s.row0 = (int32_t)p.offsets[e];
    s.rows = (int32_t)rows;
    s.mtiles = (int32_t)((rows + BM - 1) / BM);
    s.ntiles = (int32_t)(kind == 0 ? p.inter / L1_COLS : p.hidden / L2_COLS);
    int32_t &count = kind == 0 ? a.n_l1 : a.n_l2;
    s.tile0 = count;
    count += s.mtiles * s.ntiles;
}

}  // namespace

hipError_t launch_moe(const Problem &p, int schedule, int per_wave, bool local, hipStream_t stream)
{
    MoeArgs base = {};
    base.k = (int32_t)p.k;
    base.hidden = (int32_t)p.hidden;
    base.inter = (int32_t)p.inter;
    base.out_local = local ? 1 : 0;
    base.x = p.x;
    base.row_slot = p.row_slot;
    base.topk_w = p.topk_w;
    base.w1 = p.w1;
    base.w2 = p.w2;
    base.act = p.act;
    base.out = p.out;
    base.n_xcd = ua::device_xcd_count();
    const int n_waves = (int)((p.E_l + per_wave - 1) / per_wave);
    // kinds: bit 0 = Linear-1 of wave w1, bit 1 = Linear-2 of wave w2
    auto run = [&](int w1, int w2) -> hipError_t {
        MoeArgs a = base;
        if (w2 >= 0)
            for (int e = w2 * per_wave; e < (w2 + 1) * per_wave && e < p.E_l; ++e) add_seg(a, p, e, 1);
        if (w1 >= 0)
            for (int e = w1 * per_wave; e < (w1 + 1) * per_wave && e < p.E_l; ++e) add_seg(a, p, e, 0);
        const int64_t blocks = (int64_t)a.n_l1 + a.n_l2;
        if (blocks == 0) return hipSuccess;
        void *args[] = {&a};
        return hipLaunchKernel((const void *)moe_tiles, dim3((unsigned)blocks), dim3(NT), args, 0, stream);
    };
    hipError_t e = hipSuccess;
    if (schedule == kInterleaved && !local) {
        e = run(0, -1);
        for (int w = 1; w < n_waves && e == hipSuccess; ++w) e = run(w, w - 1);
        if (e == hipSuccess) e = run(-1, n_waves - 1);
    } else {
        for (int w = 0; w < n_waves && e == hipSuccess; ++w) {
            e = run(w, -1);
            if (e == hipSuccess) e = run(-1, w);
        }
    }
    return e;
}

int64_t token_tiles(const int64_t *offsets, int64_t E_l)
{
    int64_t n = 0;
    for (int64_t e = 0; e < E_l; ++e) n += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    return n;
}

hipError_t launch_moe_persist(const Problem &p, int schedule, int per_wave, bool local, unsigned *ws,
                              hipStream_t stream)
{
    // workspace: [0, kWsHeader) queue counters (one per launch) and the
    // timeout count, then one ready count per token tile; cleared first
    const int64_t n_tt = token_tiles(p.offsets, p.E_l);
    const int n_words = (int)(kWsHeader + n_tt);
    {
        unsigned *q = ws;
        int n = n_words;
        void *args[] = {(void *)&q, &n};
        const hipError_t e = hipLaunchKernel((const void *)clear_words, dim3((unsigned)((n + 255) / 256)), dim3(256),
                                             args, 0, stream);
        if (e != hipSuccess) return e;
    }
    PersistArgs a = {};
    a.m.k = (int32_t)p.k;
    a.m.hidden = (int32_t)p.hidden;
    a.m.inter = (int32_t)p.inter;
    a.m.out_local = local ? 1 : 0;
    a.m.n_xcd = ua::device_xcd_count();
    a.m.x = p.x;
    a.m.row_slot = p.row_slot;
    a.m.topk_w = p.topk_w;
    a.m.w1 = p.w1;
    a.m.w2 = p.w2;
    a.m.act = p.act;
    a.m.out = p.out;
    a.l1_cols = (uint32_t)(p.inter / L1_COLS);
    a.timeouts = ws + kWsTimeouts;
    a.ready = ws + kWsHeader;
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    std::vector<int32_t> tt0(p.E_l + 1, 0);
    for (int64_t x = 0; x < p.E_l; ++x) tt0[x + 1] = tt0[x] + (int32_t)((p.offsets[x + 1] - p.offsets[x] + BM - 1) / BM);
    const bool inter = schedule == kInterleaved && !local;
    // launches of whole waves, at most kMaxWave experts each (one segment per
    // expert and kind)
    const int waves_per_launch = kMaxWave / per_wave;
    const int n_waves = (int)((p.E_l + per_wave - 1) / per_wave);
    int q = 0;
    for (int w0 = 0; w0 < n_waves; w0 += waves_per_launch, ++q) {
        const int w1 = std::min(n_waves, w0 + waves_per_launch);
        a.m.nseg = 0;
        a.nph = 0;
        int32_t pos = 0;
        // one phase: Linear-2 of wave l2w (or -1), Linear-1 of wave l1w (or -1)
        auto phase = [&](int l1w, int l2w) {
            Phase &ph = a.ph[a.nph];
            ph.start = pos;
            ph.seg_begin = a.m.nseg;
            a.m.n_l1 = a.m.n_l2 = 0;
            if (l2w >= 0)
                for (int x = l2w * per_wave; x < (l2w + 1) * per_wave && x < p.E_l; ++x) add_seg(a.m, p, x, 1, tt0[x]);
            if (l1w >= 0)
                for (int x = l1w * per_wave; x < (l1w + 1) * per_wave && x < p.E_l; ++x) add_seg(a.m, p, x, 0, tt0[x]);
            ph.seg_end = a.m.nseg;
            ph.n_l1 = a.m.n_l1;
            ph.n_l2 = a.m.n_l2;
            if (ph.n_l1 + ph.n_l2 == 0) return;
            pos += ph.n_l1 + ph.n_l2;
            ++a.nph;
        };
        if (inter) {
            phase(w0, -1);
            for (int w = w0 + 1; w < w1; ++w) phase(w, w - 1);
            phase(-1, w1 - 1);
        } else {
            for (int w = w0; w < w1; ++w) {
                phase(w, -1);
                phase(-1, w);
            }
        }
        if (pos == 0) continue;
        a.n_tiles = pos;
        a.queue = ws + q;
        const unsigned grid = (unsigned)std::min<int64_t>(pos, n_cu > 0 ? n_cu : 1);
        void *args[] = {&a};
        e = hipLaunchKernel((const void *)moe_persist, dim3(grid), dim3(NT), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_scatter(const uint16_t *y_local, const int32_t *row_slot, int64_t N, int64_t hidden,
                          uint16_t *combine, hipStream_t stream)
{
    int64_t n = N * (hidden / 8);
    int32_t cpr = (int32_t)(hidden / 8);
    const uint16_t *src = y_local;
    const int32_t *rs = row_slot;
    uint16_t *dst = combine;
    void *args[] = {(void *)&src, (void *)&rs, &n, &cpr, (void *)&dst};
    return hipLaunchKernel((const void *)scatter_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), args, 0, stream);
}

}  // namespace moe
