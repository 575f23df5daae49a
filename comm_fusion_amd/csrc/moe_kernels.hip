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
//    per eight MFMAs), over k-steps of 32;
//  * outputs are computed transposed, C^T = W X^T: the weight rows are the A
//    operand and the token rows the B operand, so every lane holds one token
//    row and 16 of its features per block (runs of 4 consecutive features);
//  * operand tiles go global -> LDS directly (no VGPR staging) through a
//    ring of four stages, each copy issued three k-steps before its use; one
//    barrier per step; the operand reads are explicit LDS instructions
//    prefetched a k-substep ahead;
//  * Linear-1 tiles take 128 gate rows and the 128 matching up rows of W1,
//    arranged so that each wave's feature blocks hold gate and up of the
//    same intermediate columns: SiLU(gate) * up is formed in registers;
//  * token rows are gathered through row_slot (slot / k is the token), so the
//    dispatch exchange's receive side is read in place;
//  * the Linear-2 epilogue multiplies each row by its routing weight, rounds
//    to bf16, stages the tile in the LDS and stores whole 512-byte row
//    segments (16 bytes per lane) into each row's Combine slot.
#include "moe_internal.h"
#include "ua_internal.h"

#include <type_traits>
#include <utility>

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
constexpr int BK = 32;                  // k per step
constexpr int NSTAGE = 4;               // LDS ring: copies run three steps ahead
constexpr int NW = 8;                   // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int TILE = 256 * BK * 2;      // bytes of one operand tile (16 KiB)
constexpr int STAGE = 2 * TILE;         // W tile + token tile (32 KiB)
constexpr int NCPW = TILE / 1024 / NW;  // 1 KiB copies per wave per operand tile
constexpr int L1_COLS = 128;            // intermediate columns per Linear-1 tile
constexpr int L2_COLS = 256;            // hidden columns per Linear-2 tile

typedef const __attribute__((address_space(1))) void gbl_void;
typedef __attribute__((address_space(3))) void lds_void;

// One expert's tiles of one kind in a launch.
struct Seg {
    int32_t kind;    // 0: Linear-1 (+ activation), 1: Linear-2 (+ Combine)
    int32_t expert;  // local expert
    int32_t row0;    // its first receive row
    int32_t rows;    // its receive rows
    int32_t mtiles;  // token tiles, ceil(rows / BM)
    int32_t ntiles;  // feature tiles
    int32_t tile0;   // first tile of the segment among its kind's tiles in the launch
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
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4 (&fa)[4], u32x4 (&fb)[2])
{
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1])
                 : "i"(N));
}

// One output tile: 256 features x 256 token rows, K in steps of 32.
// Operand tiles in the LDS: [row][64 B] (the step's 32 k values), the four
// 16-byte chunks of a row at positions chunk ^ ((row / 4) % 4), so a
// fragment read (32 rows, one chunk each per half-wave) spreads over all
// banks.  They are filled by 1 KiB global->LDS copies (lane L of copy c
// lands at byte 1024 c + 16 L: row 16 c + L / 4, fetching chunk
// (L % 4) ^ ((L / 16) % 4)) into a ring of four stages: the copies of step
// s+3 are issued as step s starts, so each has three steps to land.  Wave
// (wf, wt) computes features 128 wf .. +127 (four 32-row blocks) of token
// rows 64 wt .. +63 (two).
template <int KIND>
__device__ __forceinline__ void tile(const MoeArgs &a, const Seg &sg, int m, int n, lds_u8 *lds)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wf = wave & 1, wt = wave >> 1;
    const int l32 = lane & 31, g = lane >> 5;
    const int K = KIND == 0 ? a.hidden : a.inter;
    const int nk = K / BK;
    const char *wbase = (const char *)(KIND == 0 ? a.w1 + (int64_t)sg.expert * 2 * a.inter * a.hidden
                                                 : a.w2 + (int64_t)sg.expert * a.hidden * a.inter);
    const char *bbase = (const char *)(KIND == 0 ? a.x : a.act);

    // This wave's copies: numbers NCPW wave .. of each operand tile.
    const unsigned chunk16 = (unsigned)((lane & 3) ^ ((lane >> 4) & 3)) * 16;
    unsigned aoff[NCPW], boff[NCPW];
#pragma unroll
    for (int i = 0; i < NCPW; ++i) {
        const int c = NCPW * wave + i;
        const int r = 16 * c + (lane >> 2);
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
    auto copy = [&](int s, int st) {
        const unsigned ko = (unsigned)s * BK * 2;
        lds_u8 *dst = lds + st * STAGE + NCPW * wave * 1024;
#pragma unroll
        for (int i = 0; i < NCPW; ++i) {
            __builtin_amdgcn_global_load_lds((gbl_void *)(wbase + aoff[i] + ko), (lds_void *)(dst + i * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void *)(bbase + boff[i] + ko), (lds_void *)(dst + TILE + i * 1024),
                                             16, 0, 0);
        }
    };

    // Per-lane LDS addresses of the fragment reads; stage and block are
    // instruction offsets (stages 2 and 3 through their own base registers:
    // the offset field holds 16 bits).  Fragment element layout: lane l gives
    // row (block + l % 32), k values 8 (l / 32) .. +7 of the 16-wide
    // k-substep (substep 0: chunks 0, 1; substep 1: chunks 2, 3).
    const unsigned lbase = (unsigned)(uintptr_t)lds;
    const unsigned sw0 = (unsigned)(((0 + g) ^ ((l32 >> 2) & 3)) * 16);
    const unsigned sw1 = (unsigned)(((2 + g) ^ ((l32 >> 2) & 3)) * 16);
    const unsigned ra = lbase + (unsigned)(128 * wf + l32) * 64;
    const unsigned rb = lbase + TILE + (unsigned)(64 * wt + l32) * 64;
    // [stage / 2][substep]
    const unsigned abase[2][2] = {{ra + sw0, ra + sw1}, {ra + 2 * STAGE + sw0, ra + 2 * STAGE + sw1}};
    const unsigned bbase2[2][2] = {{rb + sw0, rb + sw1}, {rb + 2 * STAGE + sw0, rb + 2 * STAGE + sw1}};

    f32x16 acc[4][2];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fb][tb][r] = 0.f;

    // fragment registers: the first k-substep's in two sets (a step's own,
    // and the next step's, read ahead), the second substep's in one
    u32x4 fa[3][4], fbr[3][2];
    // the six fragment reads of k-substep KK (0, 1) of the stage ST
    auto reads = [&](auto stc, auto kkc, u32x4 (&da)[4], u32x4 (&db)[2]) {
        constexpr int ST = decltype(stc)::value, KK = decltype(kkc)::value;
        constexpr int OFF = (ST & 1) * STAGE;
        const unsigned pa = abase[ST >> 1][KK], pb = bbase2[ST >> 1][KK];
        da[0] = lds_read<OFF + 0 * 2048>(pa);
        da[1] = lds_read<OFF + 1 * 2048>(pa);
        da[2] = lds_read<OFF + 2 * 2048>(pa);
        da[3] = lds_read<OFF + 3 * 2048>(pa);
        db[0] = lds_read<OFF + 0 * 2048>(pb);
        db[1] = lds_read<OFF + 1 * 2048>(pb);
    };
    auto mfmas = [&](u32x4 (&da)[4], u32x4 (&db)[2]) {
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, da[fb]), __builtin_bit_cast(bf16x8, db[tb]), acc[fb][tb], 0, 0, 0);
    };
    // One k-step on stage ST = s % 4.  The copies of steps s and s+1 have
    // landed once at most those of s+2 (2 NCPW, issued one step earlier)
    // remain in flight; after the barrier every wave's have, and every wave
    // is done with step s-1, whose stage takes the copies of step s+3.  The
    // first k-substep's reads of step s were issued at the end of step s-1
    // (into set PS = s % 2; those of step 0 by the prologue); the end of
    // step s issues those of step s+1 into the other set, so the MFMAs of a
    // step start without waiting for the LDS.  The last step issues them too
    // (from a stage that is not used any more): no branch, so the compiler
    // has no reason to move fragment registers while reads are in flight.
    auto step = [&](int s, auto stc) {
        constexpr int ST = decltype(stc)::value, PS = ST & 1, PN = PS ^ 1;
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using SN = std::integral_constant<int, (ST + 1) & 3>;
        if (s + 2 < nk)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(2 * NCPW) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (s + 3 < nk) copy(s + 3, (ST + 3) & 3);
        reads(stc, I1(), fa[2], fbr[2]);
        lgkm_wait<6>(fa[PS], fbr[PS]);
        mfmas(fa[PS], fbr[PS]);
        __builtin_amdgcn_sched_barrier(0);
        reads(SN(), I0(), fa[PN], fbr[PN]);
        lgkm_wait<6>(fa[2], fbr[2]);
        mfmas(fa[2], fbr[2]);
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: the copies of steps 0, 1, 2, and once step 0's have landed
    // everywhere, its first k-substep's reads
    for (int p = 0; p < 3 && p < nk; ++p) copy(p, p);
    if (nk > 2)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(4 * NCPW) : "memory");
    else if (nk > 1)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(2 * NCPW) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    reads(std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), fa[0], fbr[0]);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    // K is a multiple of 128 (hidden % 256, inter % 128), so nk % 4 == 0
    for (int s = 0; s < nk; s += 4) {
        step(s, S0());
        step(s + 1, S1());
        step(s + 2, S2());
        step(s + 3, S3());
    }
    // every wave is done with the operand tiles (the Linear-2 epilogue reuses
    // the LDS); the last step's read-ahead lands in one of the two sets, so
    // both stay reserved until the wait.  The copy offsets stay reserved up
    // to here too: otherwise their registers, free after the last copies,
    // may take fragments read ahead in the last steps.
    static_assert(NCPW == 2, "copy offsets tied below");
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier"
                 : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[0][2]), "+v"(fa[0][3]), "+v"(fbr[0][0]), "+v"(fbr[0][1]),
                   "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fa[1][2]), "+v"(fa[1][3]), "+v"(fbr[1][0]), "+v"(fbr[1][1]),
                   "+v"(aoff[0]), "+v"(aoff[1]), "+v"(boff[0]), "+v"(boff[1])
                 :
                 : "memory");

    // Accumulator register r of block (fb, tb) is feature 8(r/4) + 4g + r%4 of
    // the block, token row l32 of the block.
    if constexpr (KIND == 0) {
        // SiLU(gate) * up -> act[row][128 n + 64 wf + ...], bf16
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int rl = m * BM + 64 * wt + 32 * tb + l32;
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
            const int rl = m * BM + 64 * wt + 32 * tb + l32;
            wrow[tb] = rl < sg.rows ? a.topk_w[a.row_slot[sg.row0 + rl]] : 0.f;
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int tr = 64 * wt + 32 * tb + l32;
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
    __shared__ __attribute__((aligned(1024))) unsigned char lds_all[NSTAGE * STAGE];  // 128 KiB: one workgroup per CU
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
        tile<0>(a, sg, mm, nn, lds);
    else
        tile<1>(a, sg, mm, nn, lds);
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

// Append expert e's tiles of `kind` to a launch.
void add_seg(MoeArgs &a, const Problem &p, int e, int kind)
{
    const int64_t rows = p.offsets[e + 1] - p.offsets[e];
    if (rows == 0) return;
    Seg &s = a.seg[a.nseg++];
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
