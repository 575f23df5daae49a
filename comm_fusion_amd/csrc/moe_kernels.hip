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
//  * one kernel for both layers: a workgroup of 4 wave64s computes a tile of
//    128 output features x 128 token rows, each wave 64 x 64 as 2 x 2 blocks
//    of v_mfma_f32_32x32x16_bf16, over k-steps of 64;
//  * outputs are computed transposed, C^T = W X^T: the weight rows are the A
//    operand and the token rows the B operand, so every lane holds one token
//    row and 16 of its features per block (runs of 4 consecutive features);
//  * operand tiles go global -> VGPR -> LDS, double-buffered: the loads for
//    step s+1 are in flight while step s computes; one barrier per step.  In
//    the LDS a tile row (64 k values, 128 B) keeps its eight 16-byte chunks at
//    positions chunk ^ ((row / 2) % 8), so both the row-wise stores and the
//    fragment reads (32 rows, one chunk each) spread over all banks;
//  * Linear-1 tiles take 64 gate rows and the 64 matching up rows of W1, so a
//    wave's two feature blocks hold gate and up of the same intermediate
//    columns and SiLU(gate) * up is formed in registers (bf16 out);
//  * token rows are gathered through row_slot (slot / k is the token), so the
//    dispatch exchange's receive side is read in place;
//  * the Linear-2 epilogue multiplies each row by its routing weight, rounds
//    to bf16, stages the tile in the LDS and stores whole 256-byte row
//    segments (16 bytes per lane) into each row's Combine slot.
#include "moe_internal.h"
#include "ua_internal.h"

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

constexpr int BM = 128;                 // token rows per tile
constexpr int BK = 64;                  // k per step
constexpr int NT = 256;                 // threads per workgroup (4 waves)
constexpr int TILE = 128 * BK * 2;      // bytes of one operand tile (16 KiB)
constexpr int STAGE = 2 * TILE;         // W tile + token tile
constexpr int L1_COLS = 64;             // intermediate columns per Linear-1 tile
constexpr int L2_COLS = 128;            // hidden columns per Linear-2 tile

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

// Position of 16-byte chunk c of tile row r in the LDS (see the file comment).
__device__ __forceinline__ int lds_pos(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int KIND>
__device__ __forceinline__ void tile(const MoeArgs &a, const Seg &sg, int m, int n, lds_u8 *lds)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wf = wave & 1, wt = wave >> 1;  // feature half, token half of the tile
    const int l32 = lane & 31, g = lane >> 5;
    const int K = KIND == 0 ? a.hidden : a.inter;
    const int nk = K / BK;
    const char *wbase = (const char *)(KIND == 0 ? a.w1 + (int64_t)sg.expert * 2 * a.inter * a.hidden
                                                 : a.w2 + (int64_t)sg.expert * a.hidden * a.inter);
    const char *bbase = (const char *)(KIND == 0 ? a.x : a.act);

    // This thread's share of each operand tile: rows rr + 32 i (i < 4),
    // 16-byte chunk kc of the step's 64 k values.
    const int rr = tid >> 3, kc = tid & 7;
    unsigned aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rr + 32 * i;
        // weight row of tile row r: Linear-1 takes gate rows 64n .. 64n+63 and
        // up rows inter + 64n .. ; Linear-2 takes hidden rows 128n .. 128n+127
        const int wrow = KIND == 0 ? (r < 64 ? L1_COLS * n + r : a.inter + L1_COLS * n + r - 64) : L2_COLS * n + r;
        aoff[i] = ((unsigned)wrow * (unsigned)K + kc * 8) * 2;
        // token row: rows past the expert's end repeat its last row (not stored)
        const int rl = m * BM + r < sg.rows ? m * BM + r : sg.rows - 1;
        const int ri = sg.row0 + rl;
        const unsigned brow = KIND == 0 ? (unsigned)(a.row_slot[ri] / a.k) : (unsigned)ri;
        boff[i] = (brow * (unsigned)K + kc * 8) * 2;
    }
    const int spos = lds_pos(rr, kc);  // the same for rr + 32 i (the swizzle has period 16)

    u32x4 ra[4], rb[4];
    auto load = [&](int s) {
        const unsigned ko = (unsigned)s * BK * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *(const u32x4 *)(wbase + aoff[i] + ko);
            rb[i] = *(const u32x4 *)(bbase + boff[i] + ko);
        }
    };
    auto store = [&](int st) {
        lds_u8 *s = lds + st * STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(lds_u32x4 *)(s + spos + i * 32 * 128) = ra[i];
            *(lds_u32x4 *)(s + TILE + spos + i * 32 * 128) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fb][tb][r] = 0.f;
    // tile rows of the wave's feature blocks: Linear-1 pairs the gate block
    // (rows 32 wf ..) with the up block of the same columns (rows 64 + 32 wf ..)
    const int frow0 = KIND == 0 ? 32 * wf : 64 * wf;
    const int fstep = KIND == 0 ? 64 : 32;
    const int trow0 = 64 * wt;

    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        if (s + 1 < nk) load(s + 1);
        const lds_u8 *st = lds + (s & 1) * STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + g;
            u32x4 af[2], bf[2];
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) af[fb] = *(const lds_u32x4 *)(st + lds_pos(frow0 + fstep * fb + l32, c));
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) bf[tb] = *(const lds_u32x4 *)(st + TILE + lds_pos(trow0 + 32 * tb + l32, c));
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, af[fb]), __builtin_bit_cast(bf16x8, bf[tb]), acc[fb][tb], 0, 0, 0);
        }
        if (s + 1 < nk) store((s + 1) & 1);
        __syncthreads();
    }

    // Accumulator register r of block (fb, tb) is feature 8(r/4) + 4g + r%4 of
    // the block, token row l32 of the block.
    if constexpr (KIND == 0) {
        // SiLU(gate) * up -> act[row][64n + 32 wf + ...], bf16
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int rl = m * BM + trow0 + 32 * tb + l32;
            if (rl >= sg.rows) continue;
            uint16_t *dst = a.act + (int64_t)(sg.row0 + rl) * a.inter + L1_COLS * n + 32 * wf + 4 * g;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = silu(acc[0][tb][4 * q4 + e]) * acc[1][tb][4 * q4 + e];
                u32x2 w;
                w[0] = pack_bf16(v[0], v[1]);
                w[1] = pack_bf16(v[2], v[3]);
                *(u32x2 *)(dst + 8 * q4) = w;
            }
        }
    } else {
        // weighted rows, staged as [token row][128 features] (chunk c of row
        // r at position c ^ (r % 16)), then stored as whole 256-byte segments
        float wrow[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int rl = m * BM + trow0 + 32 * tb + l32;
            wrow[tb] = rl < sg.rows ? a.topk_w[a.row_slot[sg.row0 + rl]] : 0.f;
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int tr = trow0 + 32 * tb + l32;
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int c = 8 * wf + 4 * fb + q4;
                    u32x2 w;
                    w[0] = pack_bf16(acc[fb][tb][4 * q4] * wrow[tb], acc[fb][tb][4 * q4 + 1] * wrow[tb]);
                    w[1] = pack_bf16(acc[fb][tb][4 * q4 + 2] * wrow[tb], acc[fb][tb][4 * q4 + 3] * wrow[tb]);
                    *(lds_u32x2 *)(lds + tr * 256 + ((c ^ (tr & 15)) << 4) + 8 * g) = w;
                }
        }
        __syncthreads();
        const int chunk = lane & 15;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tr = 32 * wave + 4 * j + (lane >> 4);
            const u32x4 v = *(const lds_u32x4 *)(lds + tr * 256 + ((chunk ^ (tr & 15)) << 4));
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
    __shared__ __attribute__((aligned(1024))) unsigned char lds_all[2 * STAGE];
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
