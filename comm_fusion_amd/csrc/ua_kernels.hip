// ua_kernels.hip -- gfx950 (MI355X) kernels for one Ulysses rank's attention
// with the post-attention All-to-All fused into the output epilogue (and, on
// request, the pre-attention one fused into its loads), plus the stand-alone
// permute and gather used by the serial baselines.
//
// Method (X-Stage paper, arXiv 2607.23264): Fig. 5 of the pith.science review
// page (Ulysses attention; steps d-e are attention plus the post-attention
// All-to-All), Fig. 6 (FlashAttention's Q-loop: each output tile is owned by
// the worker that runs the loop over all KV tiles for it) and Fig. 7 (the
// output-tile owner issues the exchange stores itself, then moves on).
//
// Design for CDNA4, not a translation of the pages' FlashAttention-3/4:
//  * a workgroup of NW wave64s (8, or 4 for small problems) owns 32*RB*NW/KS
//    query rows of one (batch, local head); each wave owns RB blocks of 32
//    rows (RB = 2 for d = 64, where the registers allow it: each K or V
//    fragment read from LDS then feeds two MFMAs).  With KS = 2 (launches
//    with fewer than 128 units of 256 rows) two key groups of waves share the rows, each
//    taking half the K/V tiles, and merge their partial results through LDS
//    at the end.  The waves of a key group share each K/V tile, so a tile
//    crosses L2 -> LDS once per 32*RB*NW/KS rows;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K streams from LDS as the A operand and the
//    wave's Q rows stay in VGPRs as the B operand.  The accumulator layout
//    then gives every lane ONE query row (lane % 32) and 16 keys per block,
//    so a row max needs one v_permlane32_swap and the row sum none until the
//    end;
//  * P^T is fed from those registers (rounded to bf16) as the B operand of
//    O^T += V^T P^T; V^T comes from the key-major V tile through the gfx950
//    transposing LDS read ds_read_b64_tr_b16;
//  * K and V tiles (64 keys; 32 with RB = 2 or KS = 2) go global -> LDS
//    with global_load_lds_dwordx4 (no VGPR staging), through rings of three
//    buffers, each copy issued two iterations before its tile is used;
//    the operand reads of an iteration's first MFMAs are issued before its
//    barrier, at the end of the previous iteration;
//  * software pipeline: in steady state, iteration t interleaves the
//    softmax of S_t with the MFMAs of O += V_{t-1} P_{t-1} and of S_{t+1},
//    one MFMA plus a slice of softmax VALU work per issue slot, so every
//    wave keeps its matrix pipe fed while it does its exponentials (at
//    d = 64, where every slot carries VALU work, each slice issues at raised
//    wave priority);
//  * online softmax in fp32, log2 domain, with a lazily raised running max:
//    the tiles between a work item's first and last take P against the max
//    as it stands (no tile max in the loop) and go to an exact path only
//    when a lane's sum of the tile's P passes 2^15;
//  * epilogue: each wave normalises its rows, stages them through the LDS
//    (free after the loop) and stores whole rows, 16 bytes per lane, straight
//    into the destination slots computed from (rank, P) -- the fused
//    All-to-All.  The local (serial) output is the same epilogue with one
//    region;
//  * launches whose query tiles leave CUs idle (the calls with a workspace)
//    split each tile's keys over several workgroups, in equal runs or
//    stream-K (equal runs of (query tile, key tile) iterations across tile
//    boundaries); the parts write their partial softmax state to the
//    workspace at device scope and the last to arrive merges them in key
//    order and stores the tile;
//  * workgroup ids are remapped so that consecutive work units of one head
//    run on the same XCD and share its L2 while they stream the same K/V;
//  * Q, K, V rows are read with a row stride of in_heads*d: the local layout
//    [B][S][Hl][d], or this rank's heads of the sequence-partitioned input
//    [B][P][S/P][H][d] of the pre-attention All-to-All (Fig. 5, steps a-c),
//    read in place.
//
// The LDS operand reads are inline assembly with explicit lgkmcnt waits, so
// the compiler believes their results exist as soon as they issue.  Nothing
// may copy, spill or overwrite such a register before its wait: the wait is
// tied to the very ring slot the read wrote, the ring is drained by a tied
// wait before the final iteration, and the kernels must not spill (checked
// on the assembly by the CPU tests).

#include "ua_internal.h"

#include <math.h>
#include <cstdlib>

#include <atomic>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>

namespace ua {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

constexpr int kPF = 2;  // operand prefetch distance, in LDS fragments (each feeds RB MFMAs)

struct AttnArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    Placement out;
    int64_t S;
    int32_t Hl;
    int32_t in_heads;  // heads per sequence row of Q, K, V (Hl, or H for the pre-exchange layout)
    int32_t in_head0;  // this rank's first head among them (0, or rank*Hl)
    int32_t n_qtiles;
    int32_t n_units;
    int32_t n_xcd;     // XCDs of the device (workgroups are dealt round robin over them)
    float scale_log2;  // softmax scale * log2(e)
    uint64_t *trace;   // measurement build only: 4 timestamps per work unit
    // write check (optional, any build): +1 per 16-byte chunk of the
    // destination the epilogue stores, indexed from out.base
    unsigned *wcount;
    // key split across workgroups (XS builds only): n_split workgroups per
    // query tile, each on a run of about 1/n_split of the keys; their partial
    // results meet in ws_part, and ws_cnt counts arrivals per query tile
    int32_t n_split;   // parts per query tile (stream-K: the most any query tile has)
    float *ws_part;
    unsigned *ws_cnt;
    // stream-K (XS builds): iterations per workgroup (0: split as above) and
    // the query tiles of the launch, B*Hl*n_qtiles
    int32_t sk_iters;
    int32_t n_units_q;
};

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi)
{
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, RNE
    return __builtin_bit_cast(unsigned, h);
}

// Device-scope relaxed atomic store and load of a float: coherent across the
// XCDs' L2 caches (sc1), used for the partial results of a key split.
__device__ __forceinline__ void store_dev(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lanes l and l+32 hold the same query row (for different keys / columns).
// v_permlane32_swap of a register with itself hands both lanes the pair
// (value of lane l, value of lane l+32); these combine the pair the same way
// in both lanes, so the two copies stay bit-identical.
__device__ __forceinline__ f32x2 row_pair(float x)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return f32x2{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}
__device__ __forceinline__ float row_max(float x)
{
    const f32x2 p = row_pair(x);
    return fmaxf(p[0], p[1]);
}
__device__ __forceinline__ float row_sum(float x)
{
    const f32x2 p = row_pair(x);
    return p[0] + p[1];
}

// MFMA operand reads from LDS, as explicit instructions with compile-time
// offsets (every LDS read of the attention kernel).  The compiler does not
// track them, so it inserts no waits for them -- in particular none on the
// asynchronous global->LDS copies into other buffers, which it cannot tell
// apart from these reads -- and each read is waited for exactly, with
// lgkm_wait, right before the MFMA that consumes it.  The kernel's scalar
// loads all complete before its first LDS read, so the LDS counter counts
// exactly these reads (the steady loop keeps a few in flight across
// iterations).
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(unsigned addr)
{
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr16(unsigned addr)
{
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
// Wait until at most N LDS reads are outstanding; tied to the fragment so the
// compiler cannot move the fragment's consumer above the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4 &f)
{
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f) : "i"(N));
}
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F &&f)
{
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(std::make_integer_sequence<int, N>(), f);
}

// Logical work unit of this workgroup.  Workgroups are dispatched round
// robin over the device's nx XCDs (workgroup i to XCD i % nx); give each XCD
// a contiguous run of units (same head, neighbouring Q tiles) so they share
// K/V in that XCD's L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_unit(int bid, int n, int nx)
{
    const int xcd = bid % nx, k = bid / nx;
    const int q = n / nx, r = n % nx;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// Template parameters: D head dim; NW waves per workgroup; RB 32-row query
// blocks per wave; KB keys per K/V tile; KS key groups per workgroup.
// NW = 8: two waves per SIMD, one workgroup per CU.  NW = 4 only runs for
// small shapes (fewer than 128 units of 256 rows) whose 32-key tile count
// cannot be split evenly between two key groups, so it is built for one wave
// per SIMD (and gets that SIMD's whole register file).  RB = 2 (d = 64 only, where the registers allow it): each
// K or V fragment read from LDS feeds two MFMAs, one per row block, which
// halves the LDS operand bytes per flop.
// XS: key split across workgroups, for launches with fewer query tiles than
// CUs.  Each query tile is shared by a.n_split workgroups, each taking a
// run of the K/V tiles (the runs differ by at most one unit of KS tiles);
// every one writes its partial O, m and l to
// a.ws_part, and the last to arrive (an atomic count per query tile) merges
// all of them in split order -- the same arithmetic whichever workgroup
// arrives last -- and stores the rows like the unsplit kernel.
// TRACE: measurement build with the same arithmetic and output, which also
// records per workgroup (in a.trace[4*u ..], u its work unit, or its run of
// a key-split launch): the 100 MHz constant clock at the start, when every
// wave last had its normalised rows ready (a workgroup barrier; the end,
// if it stored no rows), at the end once every wave's stores have completed
// (vmcnt(0) and a barrier), and the shader-clock cycles from start to end.
template <int D, int NW, int RB, int KB, int KS, bool XS, bool TRACE>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(NW / 4, NW / 4)))
void attn_fwd(AttnArgs a)
{
    uint64_t tr_t0 = 0, tr_c0 = 0, tr_rows = 0;
    if constexpr (TRACE) {
        tr_t0 = __builtin_amdgcn_s_memrealtime();
        tr_c0 = __builtin_amdgcn_s_memtime();
    }
    constexpr int KNB = KB / 32;             // 32-key blocks per K/V tile
    constexpr int TILE = KB * D * 2;         // bytes of one K (or V) tile
    constexpr int NCP = TILE / 1024;         // 1 KiB global->LDS copies per tile
    constexpr int NWG = NW / KS;             // waves per key group
    // With at least as many copies as waves in a key group, every wave copies
    // NLD chunks of K and of V; with fewer, the group's waves [0, NCP) copy K
    // and [NCP, 2 NCP) copy V.
    constexpr bool SPLIT = NCP < NWG;
    constexpr int NLD = SPLIT ? 1 : NCP / NWG;
    constexpr int CPG = KB / 16;             // 1 KiB copies per 32-column group
    constexpr int KK = D / 16;               // MFMA k-steps over d for S^T
    constexpr int DB = D / 32;               // 32-row blocks of O^T over d
    constexpr int GB = KB * 64;              // bytes of one 32-column group of a tile
    constexpr int RW = 32 * RB;              // query rows per wave
    constexpr int BR = RW * NWG;             // query rows per work unit
    static_assert(SPLIT ? 2 * NCP <= NWG : NCP % NWG == 0, "tile split");
    static_assert(NW % KS == 0 && (KS == 1 || (KS == 2 && RB == 1)), "key groups");
    static_assert(KB % 32 == 0 && GB == CPG * 1024, "tile geometry");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // KS key groups of NWG waves each: the groups work on the same query
    // rows, each on its own share of the K/V tiles, and are combined at the
    // end.  wq is the wave's index within its group.
    const int grp = KS == 1 ? 0 : wave / NWG;
    const int wq = wave - grp * NWG;

    // Per key group, three K and three V tile buffers (a ring: tile j lives
    // in buffer j % 3).  Every LDS read in the main loop is an explicit
    // instruction (lds_b128, lds_tr16) with exact waits, so the compiler
    // needs no alias information about these buffers.
    // The same LDS later stages the normalised output rows of the NWG storing
    // waves (RW rows of D bf16 each) for the row-coalesced epilogue stores.
    constexpr int RING_BYTES = 2 * KS * 3 * TILE;
    constexpr int STAGE_BYTES = NWG * RW * D * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char lds_all[RING_BYTES > STAGE_BYTES ? RING_BYTES : STAGE_BYTES];
    lds_u8 *const ks = (lds_u8 *)lds_all + grp * 3 * TILE;
    lds_u8 *const vs = (lds_u8 *)lds_all + (KS + grp) * 3 * TILE;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // One work item: query tile qt of (batch, local head) bh over ntl key
    // tiles per key group, key group g starting at key tile kt0 + g*ntl; in
    // XS builds it is part `part` of the `nparts` parts of the query tile's
    // keys (parts in key order), whose partial results meet in the
    // workspace.  `unit` names the item in the measurement build's trace.
    auto run = [&](const int unit, const int qt, const int bh, const int kt0, const int ntl, const int part,
                   const int nparts) {
    // The per-lane indices (and every address derived from them) are formed
    // anew for each work item from an opaque copy of the lane id: in the
    // stream-K loop the compiler would otherwise hoist them out of the loop
    // and keep them live through the whole item, and the kernel has no
    // registers to spare.
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int il = lane & 31;  // query row of this lane within each row block
    const int g = lane >> 5;   // half-wave
    const int i16 = lane & 15;
    const int half = (lane >> 4) & 1;
    const int h = bh % a.Hl;
    const int64_t b = bh / a.Hl;
    const int64_t S = a.S;
    // Q, K, V rows: [B][S][in_heads][D], this unit's head at in_head0 + h.
    // With in_heads = H this is the sequence-partitioned input of the
    // pre-attention exchange, [B][P][S/P][H][D] (source rank p's rows
    // [p*S/P, (p+1)*S/P) back to back), read in place.
    const int rs = a.in_heads * D;  // elements between sequence rows
    const int64_t head = (b * S * a.in_heads + a.in_head0 + h) * D;
    // Keys of this wave's group: Skv keys starting at key kvbase (the KS
    // groups of a work item run the same number of tiles, so the same
    // iterations and barriers).
    const int ntiles = ntl;
    const int64_t kvbase = (int64_t)(kt0 + grp * ntl) * KB;
    const int64_t Skv = S - kvbase < (int64_t)ntiles * KB ? S - kvbase : (int64_t)ntiles * KB;
    const uint16_t *qh = a.q + head;
    const uint16_t *kh = a.k + head + kvbase * rs;
    const uint16_t *vh = a.v + head + kvbase * rs;

    // LDS tile layouts (filled by whole-wave 1 KiB global->LDS copies, lane
    // L of a copy landing at byte 16*L, so a layout is just a per-lane choice
    // of the global chunk to fetch):
    //   K tile: [group of 32 columns][key row][64 B], the four 16 B chunks of
    //     a row segment stored in the order chunk ^ ((row / 4) % 4), so the
    //     S^T operand read (16 rows, one chunk per quarter-wave) hits 16
    //     distinct 16 B bank slots;
    //   V tile: [group of 32 columns][key row][64 B]; a transposing read
    //     (8 rows x 64 B of one group per wave) is 512 contiguous bytes.
    // Each copy fetches 16 row segments of 64 contiguous bytes: 1 KiB copy
    // number c covers group c / CPG, rows 16*(c % CPG) .. +15, and lane L
    // takes row 16*(c % CPG) + L/4, 16 B chunk L % 4 of the segment.  The
    // row's swizzle (row / 4) % 4 is then (L / 16) % 4 for every copy, so
    // only these per-lane parts live in VGPRs.
    const int lrow = lane >> 2;
    const unsigned k_chunk = (unsigned)((lane & 3) ^ ((lane >> 4) & 3)) * 16;  // bytes
    const unsigned v_chunk = (unsigned)(lane & 3) * 16;
    // First copy of this wave in a tile (wave-uniform), and whether it copies.
    const int kcp0 = SPLIT ? wq : wq * NLD;
    const int vcp0 = SPLIT ? wq - NCP : wq * NLD;
    const bool kcopies = !SPLIT || wq < NCP;
    const bool vcopies = !SPLIT || (wq >= NCP && wq < 2 * NCP);
    // Source address = wave-uniform base (scalar registers) + a non-negative
    // 32-bit per-lane byte offset.  Rows past S (last, partial tile) are
    // clamped to row S-1: finite data that the softmax masks out.
    // (S < 2^31 rows, so tile arithmetic fits 32-bit scalar registers.)
    const int S32 = (int)Skv;
    // per-lane byte offsets of a full tile (the same for every tile)
    unsigned koff[NLD], voff[NLD];
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const int kc = kcopies ? kcp0 + n : 0, vc = vcopies ? vcp0 + n : 0;
        koff[n] = (unsigned)((16 * (kc % CPG) + lrow) * rs + (kc / CPG) * 32) * 2 + k_chunk;
        voff[n] = (unsigned)((16 * (vc % CPG) + lrow) * rs + (vc / CPG) * 32) * 2 + v_chunk;
    }
    auto tile_copy = [&](const uint16_t *src, const unsigned *off, unsigned chunk, int cp0, int t, lds_u8 *dst) {
        const int kv0 = t * KB;
        const char *base = (const char *)(src + (int64_t)kv0 * rs);
        if (kv0 + KB <= S32) {
#pragma unroll
            for (int n = 0; n < NLD; ++n)
                __builtin_amdgcn_global_load_lds((gbl_void *)(base + off[n]),
                                                 (lds_void *)(dst + (cp0 + n) * 1024), 16, 0, 0);
        } else {
            asm volatile("");  // a real branch: full tiles keep their precomputed offsets
            const int last = S32 - 1 - kv0;  // last row inside S
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                const int cp = cp0 + n;
                const int row = 16 * (cp % CPG) + lrow;
                const int r = row < last ? row : last;
                const unsigned o = (unsigned)(r * rs + (cp / CPG) * 32) * 2 + chunk;
                __builtin_amdgcn_global_load_lds((gbl_void *)(base + o), (lds_void *)(dst + cp * 1024), 16, 0, 0);
            }
        }
    };
    auto copy_k = [&](int t, int buf) {
        if (kcopies) tile_copy(kh, koff, k_chunk, kcp0, t, (lds_u8 *)ks + buf * TILE);
    };
    auto copy_v = [&](int t, int buf) {
        if (vcopies) tile_copy(vh, voff, v_chunk, vcp0, t, (lds_u8 *)vs + buf * TILE);
    };
    // All of this wave's copies have landed; after the barrier every wave's
    // have, and every wave has finished the previous iteration.  A plain
    // s_barrier: reads still in flight (operand prefetch) target other buffers.
    auto sync_tiles = [&]() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };

    // This lane's query row in each row block; rows past S (ragged last Q
    // tile) compute on row S-1 and are not stored.
    u32x4 qf[RB][KK];  // B operand of S^T = K Q^T: lane holds Q[s][16kk + 8g .. +7]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int64_t s_q = (int64_t)qt * BR + wq * RW + rb * 32 + il;
        const int64_t s_ld = s_q < S ? s_q : S - 1;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[rb][kk] = *(const u32x4 *)(qh + s_ld * rs + 16 * kk + 8 * g);
    }

    // Per-lane LDS byte addresses of the operand reads; buffers and blocks
    // are instruction offsets.
    //   K (A operand of S^T = K Q^T): row il of a 32-row block, 16 B chunk
    //   (2*(kk%2) + g) ^ ((il/4)%4) of the 64 B group row.  Accumulator
    //   element r of block jb is key jb*32 + 8(r/4) + 4g + r%4, query il.
    //   V^T (A operand of O^T += V^T P^T), two transposing reads of 4 keys
    //   each: in a 16-lane group, source lane i16 points at V row
    //   k0 + i16/4, columns dd0 + 4(i16%4) .. +3 (dd0 = db*32 + 16*half),
    //   and result lane i16 gets column dd0 + i16.  P^T (B operand): chunk
    //   cc holds registers 8(cc%2)..+7 of score block cc/2, i.e. element e
    //   is key 16cc + 8(e/4) + 4g + e%4.
    const unsigned kb0 = (unsigned)(uintptr_t)(lds_u8 *)ks + il * 64 + (((0 + g) ^ ((il >> 2) & 3)) * 16);
    const unsigned kb1 = (unsigned)(uintptr_t)(lds_u8 *)ks + il * 64 + (((2 + g) ^ ((il >> 2) & 3)) * 16);
    const unsigned vb = (unsigned)(uintptr_t)(lds_u8 *)vs + (4 * g + (i16 >> 2)) * 64 + (16 * half + 4 * (i16 & 3)) * 2;
    f32x16 oacc[RB][DB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[rb][db][r] = 0.f;
    // S^T of the K tile in buffer kbuf (outside the steady loop).
    auto qk = [&](int kbuf, f32x16 (&s)[RB][KNB]) {
        const unsigned ko = kbuf * TILE;
        static_for<KNB>([&](auto jc) {
            constexpr int jb = decltype(jc)::value;
            u32x4 kf[KK];
            static_for<KK>([&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                kf[kk] = lds_b128<(kk >> 1) * GB + jb * 32 * 64>(((kk & 1) ? kb1 : kb0) + ko);
            });
            const f32x16 zero = {};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[rb][jb] = zero;
            static_for<KK>([&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                lgkm_wait<KK - 1 - kk>(kf[kk]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    s[rb][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, kf[kk]), __builtin_bit_cast(bf16x8, qf[rb][kk]), s[rb][jb], 0, 0, 0);
            });
        });
    };
    // Score block jb of S^T for K tile t, read straight from global memory
    // (the tile's LDS buffer is reused by then): the same fragments and the
    // same MFMA order as qk, so the same values.  Full tiles only.
    auto qk_global = [&](int t, int jb, f32x16 (&s)[RB]) {
        const uint16_t *kr = kh + (int64_t)(t * KB + jb * 32 + il) * rs + 8 * g;
        const f32x16 zero = {};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb] = zero;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const u32x4 kf = *(const u32x4 *)(kr + 16 * kk);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf),
                                                                __builtin_bit_cast(bf16x8, qf[rb][kk]), s[rb], 0, 0, 0);
        }
    };
    // O^T += V^T P^T for the V tile in buffer vbuf (outside the steady loop).
    auto pv = [&](int vbuf, const u32x4 (&pb)[RB][2 * KNB]) {
        const unsigned vo = vbuf * TILE;
        static_for<2 * KNB>([&](auto ccc) {
            constexpr int cc = decltype(ccc)::value;
            u32x4 af[DB];
            static_for<DB>([&](auto dbc) {
                constexpr int db = decltype(dbc)::value;
                constexpr int off = db * GB + 16 * cc * 64;
                const u32x2 a1 = lds_tr16<off>(vb + vo);
                const u32x2 a2 = lds_tr16<off + 8 * 64>(vb + vo);
                af[db] = u32x4{a1[0], a1[1], a2[0], a2[1]};
            });
            static_for<DB>([&](auto dbc) {
                constexpr int db = decltype(dbc)::value;
                lgkm_wait<2 * (DB - 1 - db)>(af[db]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, af[db]), __builtin_bit_cast(bf16x8, pb[rb][cc]), oacc[rb][db], 0, 0, 0);
            });
        });
    };

    // ---- online softmax in the log2 domain, per row block.  m_run is a
    // stabiliser, not the exact running max: O / l comes out the same for
    // any choice of it, and fp32 has room to spare, so it is raised only
    // when P would grow large.  The first and the last tile of a work item
    // take their tile max first and raise m_run when it exceeds m_run by
    // more than 8 (a factor 256).  The tiles between take P against m_run
    // as it stands and go to an exact path only when a lane's sum of the
    // tile's P passes 2^15 (or is +inf), where m_run is raised to the tile
    // max; so P stays below 2^15 and O rarely needs rescaling.  l_run is
    // this lane's part of the row sum, taken over the same bf16-rounded P
    // that feeds the PV product.
    const float c = a.scale_log2;
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
    }
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // Raise decision for row block rb and a tile whose scaled max is mt.
    // Returns this lane's decision; O must be multiplied by alpha once the
    // previous tile's PV product has been added.
    auto raise_max = [&](int rb, float mt, float &alpha) -> bool {
        const bool raise = mt > m_run[rb] + 8.0f;  // same in both lanes of a row
        const float m_new = raise ? mt : m_run[rb];
        alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);  // exactly 1 when kept, 0 at the start
        m_run[rb] = m_new;
        l_run[rb] *= alpha;
        return raise;
    };
    // Tile max and raise for every row block; true (for the whole wave) when
    // some row raised its max.
    auto softmax_max = [&](f32x16 (&s)[RB][KNB], int valid, float (&alpha)[RB]) -> bool {
        bool raised = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (valid < KB) {
#pragma unroll
                for (int jb = 0; jb < KNB; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (jb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= valid) s[rb][jb][r] = -INFINITY;
            }
            // two independent chains keep the max reduction short
            float m0 = fmaxf(s[rb][0][0], s[rb][0][1]), m1 = fmaxf(s[rb][0][2], s[rb][0][3]);
#pragma unroll
            for (int jb = 0; jb < KNB; ++jb)
#pragma unroll
                for (int r = (jb == 0 ? 4 : 0); r < 16; r += 2) {
                    m0 = fmaxf(m0, s[rb][jb][r]);
                    m1 = fmaxf(m1, s[rb][jb][r + 1]);
                }
            raised |= raise_max(rb, row_max(fmaxf(m0, m1)) * c, alpha[rb]);
        }
        return __builtin_amdgcn_ballot_w64(raised) != 0;
    };
    // P for two neighbouring keys of chunk cc of row block rb, rounded to
    // bf16 and packed as the B operand of the PV product; the row sum takes
    // the rounded values.
    // (sb: score block cc/2 of row block rb)
    auto exp_pair_b = [&](const f32x16 &sb, u32x4 (&pb)[RB][2 * KNB], int rb, int cc, int e2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sb[8 * (cc & 1) + 2 * e2], c, -m_run[rb]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sb[8 * (cc & 1) + 2 * e2 + 1], c, -m_run[rb]));
        f32x2 f = {p0, p1};
        const bf16x2 hb = __builtin_convertvector(f, bf16x2);
        pb[rb][cc][e2] = __builtin_bit_cast(unsigned, hb);
        l_run[rb] = __builtin_amdgcn_fdot2_f32_bf16(hb, ones, l_run[rb], false);
        // Pin both results here in program order: otherwise the compiler
        // sinks the whole exp work towards its first use (the next
        // iteration's PV MFMAs) and runs it as one block without MFMA overlap.
        asm volatile("" : "+v"(pb[rb][cc][e2]), "+v"(l_run[rb]));
    };
    auto exp_pair = [&](const f32x16 (&s)[RB][KNB], u32x4 (&pb)[RB][2 * KNB], int rb, int cc, int e2) {
        exp_pair_b(s[rb][cc >> 1], pb, rb, cc, e2);
    };
    auto softmax_exp = [&](const f32x16 (&s)[RB][KNB], u32x4 (&pb)[RB][2 * KNB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cc = 0; cc < 2 * KNB; ++cc)
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) exp_pair(s, pb, rb, cc, e2);
    };
    auto rescale_o = [&](const float (&alpha)[RB]) {
        asm volatile("");  // keeps this off the common path (no if-conversion)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha[rb];
    };

    // ---- software pipeline over KV tiles.  Iteration t: softmax of S_t
    // interleaves with the MFMAs of PV_{t-1} and of S_{t+1}.  Tile copies
    // run ahead through three-buffer rings (iteration t copies K_{t+3} and
    // V_{t+1}), so the operand reads of the next iteration's first MFMAs can
    // be issued before its barrier.
    const int valid_last = (int)(Skv - (int64_t)(ntiles - 1) * KB);
    f32x16 s_cur[RB][KNB], s_nxt[RB][KNB];         // S_t, S_{t+1}
    u32x4 p_cur[RB][2 * KNB], p_prv[RB][2 * KNB];  // packed P_t, P_{t-1}
    auto rotate = [&]() {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int jb = 0; jb < KNB; ++jb) s_cur[rb][jb] = s_nxt[rb][jb];
#pragma unroll
            for (int cc = 0; cc < 2 * KNB; ++cc) p_prv[rb][cc] = p_cur[rb][cc];
        }
    };

    // Steady iteration with an explicit issue order.  The MFMAs come in
    // groups of RB that share one LDS operand fragment (one MFMA per row
    // block).  Slot m issues MFMA m; the first slot of fragment f's group
    // also issues the LDS reads for fragment f + kPF (of the next iteration
    // near the end) and waits for fragment f; every slot carries a fixed
    // slice of the softmax VALU work, and scheduling fences keep the
    // compiler from gathering it into one block.
    //   Fragment order: PV_{t-1} (chunk cc, block db), then S_{t+1} (block
    //   jb, k-step kk).  VALU work: the exp pairs of S_t, taken against the
    //   running max as it stands (no tile max in the loop), from the first
    //   slot on.  The tile's lane sums are checked at the start of the next
    //   iteration, after the barrier and before PV uses that P; the exact
    //   path (rare) forms the tile's S again from K in global memory, takes
    //   its max, raises m_run to it and forms P again.
    constexpr int NPV = 2 * KNB * DB;  // PV fragments
    constexpr int NS = KNB * KK;       // S fragments
    constexpr int NF = NPV + NS;       // fragments per iteration
    constexpr int NM = NF * RB;        // MFMAs (slots) per iteration
    constexpr int NEX = 8 * KNB * RB;  // exp pairs
    constexpr int EPS = (NEX + NM - 1) / NM;  // exp pairs per slot
    static_assert(kPF <= NPV, "the prefetch crossing into the next iteration reads V fragments");
    constexpr int NRD_PV = 2, NRD_S = 1;  // LDS reads per fragment
    // reads issued after fragment f's and before its first MFMA (fragments
    // f+1 .. f+kPF, those past NF belonging to the next iteration)
    auto after = [](int f) constexpr {
        int n = 0;
        for (int j = f + 1; j <= f + kPF; ++j) n += (j % NF) < NPV ? NRD_PV : NRD_S;
        return n;
    };
    // fragment f of an iteration whose V_{t-1} / K_{t+1} sit in buffers VBUF / KBUF
    auto load_frag = [&](auto fc, auto vbufc, auto kbufc, u32x4 &dst) {
        constexpr int f = decltype(fc)::value;
        constexpr int VO = decltype(vbufc)::value * TILE, KO = decltype(kbufc)::value * TILE;
        if constexpr (f < NPV) {
            constexpr int cc = f / DB, db = f % DB;
            constexpr int off = VO + db * GB + 16 * cc * 64;
            const u32x2 a1 = lds_tr16<off>(vb);
            const u32x2 a2 = lds_tr16<off + 8 * 64>(vb);
            dst = u32x4{a1[0], a1[1], a2[0], a2[1]};
        } else {
            constexpr int q = f - NPV, jb = q / KK, kk = q % KK;
            constexpr int off = KO + (kk >> 1) * GB + jb * 32 * 64;
            dst = lds_b128<off>((kk & 1) ? kb1 : kb0);
        }
    };
    // Operand fragments in flight, carried across iterations: fragment f of
    // every iteration sits in fr[f % FR], so the ring size must divide NF.
    constexpr int FR = 4;
    static_assert(FR > kPF && NF % FR == 0 && FR == 4, "fragment ring");
    u32x4 fr[FR] = {};
    // Row sums before the last tile's P was added (for its sum check).
    float l_chk[RB];
    // Sum check of tile u, whose P sits in p_prv: a lane sum of its P above
    // 2^15 (also +inf) sends it to the exact path, which restores the row
    // sums, forms S_u again from K_u in global memory, takes its max, raises
    // m_run to it when it exceeds m_run by more than 8 (always, as a sum
    // above 2^15 of at most 32 values needs one above 2^10; rescaling O, which
    // holds PV up to u-1) and forms P_u again.  u < ntiles - 1 (full tiles).
    auto check_prev = [&](int u) {
        bool big = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) big |= l_run[rb] - l_chk[rb] > 32768.0f;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(big) == 0, 1)) return;
        float mt[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mt[rb] = -INFINITY;
#pragma unroll
        for (int jb = 0; jb < KNB; ++jb) {
            f32x16 s_re[RB];
            qk_global(u, jb, s_re);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt[rb] = fmaxf(mt[rb], s_re[rb][r]);
        }
        float alpha[RB];
        bool raised = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            l_run[rb] = l_chk[rb];
            raised |= raise_max(rb, row_max(mt[rb]) * c, alpha[rb]);
        }
        // P in the order of softmax_exp (row block, chunk, pair)
        static_assert(RB == 1 || KNB == 1, "one score block at a time keeps that order");
#pragma unroll
        for (int jb = 0; jb < KNB; ++jb) {
            f32x16 s_re[RB];
            qk_global(u, jb, s_re);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int cc = 2 * jb; cc < 2 * jb + 2; ++cc)
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) exp_pair_b(s_re[rb], p_prv, rb, cc, e2);
        }
        if (__builtin_amdgcn_ballot_w64(raised) != 0) rescale_o(alpha);
    };
    auto steady = [&](int t, auto par) {
        constexpr int P = decltype(par)::value;  // t % 3
        using VB = std::integral_constant<int, (P + 2) % 3>;   // V_{t-1}
        using KB_ = std::integral_constant<int, (P + 1) % 3>;  // K_{t+1}
        using VBn = std::integral_constant<int, P>;            // V_t: next iteration
        using KBn = std::integral_constant<int, (P + 2) % 3>;  // K_{t+2}: next iteration
        // K_{t+2} and V_t (copied during iteration t-1) have landed and
        // every wave is done with iteration t-1: K_t's and V_{t-2}'s buffers
        // are free for K_{t+3} and V_{t+1}.
        sync_tiles();
        check_prev(t - 1);
        if (t + 3 < ntiles) copy_k(t + 3, P);
        copy_v(t + 1, (P + 1) % 3);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_chk[rb] = l_run[rb];
        static_for<NM>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int f = m / RB, r = m % RB;  // fragment, row block
            if constexpr (r == 0) {
                if constexpr (f + kPF < NF)
                    load_frag(std::integral_constant<int, f + kPF>(), VB(), KB_(), fr[(f + kPF) % FR]);
                else
                    load_frag(std::integral_constant<int, f + kPF - NF>(), VBn(), KBn(), fr[(f + kPF - NF) % FR]);
                lgkm_wait<after(f)>(fr[f % FR]);
            }
            u32x4 &fg = fr[f % FR];
            if constexpr (f < NPV) {
                constexpr int cc = f / DB, db = f % DB;
                oacc[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, fg), __builtin_bit_cast(bf16x8, p_prv[r][cc]), oacc[r][db], 0, 0, 0);
            } else {
                constexpr int q = f - NPV, jb = q / KK, kk = q % KK;
                if constexpr (kk == 0) {
                    const f32x16 zero = {};
                    s_nxt[r][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, fg), __builtin_bit_cast(bf16x8, qf[r][kk]), zero, 0, 0, 0);
                } else {
                    s_nxt[r][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, fg), __builtin_bit_cast(bf16x8, qf[r][kk]), s_nxt[r][jb], 0, 0, 0);
                }
            }
            // At d = 64 the wave issues its softmax slice at raised priority
            // (back to normal after it): where both waves of a SIMD could
            // issue, the one with VALU work goes first while the other's
            // MFMA runs.  Measured +2% at d = 64 and neutral at d = 128,
            // where a slot carries half as much VALU work per MFMA.
            if constexpr (D == 64) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(1);
            }
            // softmax slice of slot m: exp pairs m*EPS .. m*EPS+EPS-1
            static_for<NEX>([&](auto ec) {
                constexpr int e = decltype(ec)::value;
                if constexpr (e / EPS == m) {
                    constexpr int erb = e / (8 * KNB), w = e % (8 * KNB);
                    exp_pair(s_cur, p_cur, erb, w >> 2, w & 3);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
        });
        rotate();
    };
    // Full wait (also drains operand reads still in flight) and barrier.
    auto sync_all = [&]() {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // prologue: K_0, K_1, K_2 and V_0, then S_0
    copy_k(0, 0);
    if (ntiles > 1) copy_k(1, 1);
    if (ntiles > 2) copy_k(2, 2);
    copy_v(0, 0);
    sync_all();
    qk(0, s_cur);

    // iteration 0: softmax S_0 -> P_0 with S_1
    float alpha0[RB];
    softmax_max(s_cur, ntiles == 1 ? valid_last : KB, alpha0);
    if (ntiles == 1) {
        softmax_exp(s_cur, p_cur);
        pv(0, p_cur);
    } else {
        qk(1, s_nxt);
        softmax_exp(s_cur, p_cur);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_chk[rb] = l_run[rb];
        rotate();
        // every wave is done with K_0: its buffer takes K_3; V_1 goes to buffer 1
        sync_all();
        if (ntiles > 3) copy_k(3, 0);
        copy_v(1, 1);
        // operands of the first steady iteration (V_0 and K_2, landed)
        if (ntiles > 2)
            static_for<kPF>([&](auto fc) {
                load_frag(fc, std::integral_constant<int, 0>(), std::integral_constant<int, 2>(),
                          fr[decltype(fc)::value % FR]);
            });
        // steady iterations t = 1 .. ntiles-2, unrolled by three so that
        // every buffer is fixed at compile time.
        using I2 = std::integral_constant<int, 2>;
        int t = 1;
        for (; t + 3 < ntiles; t += 3) {
            steady(t, I1());
            steady(t + 1, I2());
            steady(t + 2, I0());
        }
        if (t + 1 < ntiles) {
            steady(t, I1());
            ++t;
        }
        if (t + 1 < ntiles) {
            steady(t, I2());
            ++t;
        }
        // last iteration t = ntiles-1: softmax of the last, possibly partial
        // tile with PV_{t-1}; then PV of the last tile.  No copies left.
        // The last steady iteration prefetched fragments for an iteration
        // that does not come: their reads are still in flight, so their
        // registers stay reserved (tied to this wait) until they land.
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fr[0]), "+v"(fr[1]), "+v"(fr[2]), "+v"(fr[3])::"memory");
        sync_all();
        check_prev(t - 1);
        float alpha[RB];
        const bool any = softmax_max(s_cur, valid_last, alpha);
        pv((t + 2) % 3, p_prv);
        softmax_exp(s_cur, p_cur);
        if (any) rescale_o(alpha);
        pv(t % 3, p_cur);
    }

    // ---- key groups: group 1 hands its partial O, m and l to the group-0 wave
    // with the same rows (same lane layout) through LDS, free after the loop;
    // that wave merges them, O = O0 a0 + O1 a1 and l = l0 a0 + l1 a1 with
    // a_i = 2^(m_i - max(m0, m1)), and alone stores the rows.
    if constexpr (KS == 2) {
        constexpr int NX = RB * DB * 16 + 2 * RB;  // floats per lane
        static_assert(NWG * NX * 64 * 4 <= 2 * KS * 3 * TILE, "combine area");
        typedef __attribute__((address_space(3))) float lds_f32;
        lds_f32 *const xb = (lds_f32 *)lds_all + wq * NX * 64 + lane;
        sync_all();
        if (grp == 1) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) xb[((rb * DB + db) * 16 + r) * 64] = oacc[rb][db][r];
                xb[(RB * DB * 16 + rb) * 64] = m_run[rb];
                xb[(RB * DB * 16 + RB + rb) * 64] = l_run[rb];
            }
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float m1 = xb[(RB * DB * 16 + rb) * 64];
                const float l1 = xb[(RB * DB * 16 + RB + rb) * 64];
                const float m = fmaxf(m_run[rb], m1);
                const float a0 = __builtin_amdgcn_exp2f(m_run[rb] - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        oacc[rb][db][r] = oacc[rb][db][r] * a0 + xb[((rb * DB + db) * 16 + r) * 64] * a1;
                l_run[rb] = l_run[rb] * a0 + l1 * a1;
                m_run[rb] = m;
            }
        }
    }

    // ---- key split across workgroups: publish this workgroup's partial
    // (group 0's waves hold it, same layout as the key-group hand-off), count
    // the arrival, and let only the last arrival go on.  It merges the
    // partials of splits 0 .. n_split-1 in that order, resets the count for
    // the next call, and stores the rows.
    // Ordering: the waves' partial stores, each wave's wait for their
    // completion, a workgroup barrier, then thread 0's device-scope release
    // add; in the merging workgroup, thread 0's device-scope acquire, a
    // workgroup barrier, then the loads (the usual last-block pattern).  The partials are device-scope atomic stores and
    // loads (sc1: written through and read past the XCD's L2), so the
    // release's L2 write-back has little to flush.  Only thread 0 fences: the
    // same fences in every wave (an L2 write-back each, and an invalidate of
    // the L2 the other workgroups stream their K/V tiles through) slowed the
    // split launch by up to 40%.
    if constexpr (XS) {
        constexpr int NX = RB * DB * 16 + 2 * RB;  // floats per lane
        constexpr int MO = RB * DB * 16;          // m_run at MO + rb, l_run at MO + RB + rb
        const int64_t tile = (int64_t)bh * a.n_qtiles + qt;
        const int64_t sstride = (int64_t)NWG * NX * 64;  // floats per split
        float *const part0 = a.ws_part + tile * a.n_split * sstride + wq * NX * 64 + lane;
        if (grp == 0) {
            float *const mine = part0 + part * sstride;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) store_dev(&mine[((rb * DB + db) * 16 + r) * 64], oacc[rb][db][r]);
                store_dev(&mine[(MO + rb) * 64], m_run[rb]);
                store_dev(&mine[(MO + RB + rb) * 64], l_run[rb]);
            }
        }
        // Each wave waits until its own partial stores have completed at
        // device scope (an sc1 store counts as done once written through its
        // XCD's L2) before the barrier; the barrier then orders every wave's
        // completed stores before thread 0's release add.  The release's own
        // wait covers only the stores of thread 0's wave.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // (also: every wave's LDS reads are done)
        typedef __attribute__((address_space(3))) int lds_i32;
        lds_i32 *const flag = (lds_i32 *)lds_all;
        if (threadIdx.x == 0) {
            const unsigned seen = __hip_atomic_fetch_add(a.ws_cnt + tile, 1u, __ATOMIC_RELEASE,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            const int last = seen == (unsigned)(nparts - 1);
            if (last) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every part's release is seen
                atomicExch(a.ws_cnt + tile, 0u);
            }
            *flag = last;
        }
        __syncthreads();  // the other waves' loads follow thread 0's acquire
        if (!*flag) return;
        // Merge in split order with a running max: part 0 is taken as is, and
        // part i rescales the sum so far by 2^(M - M') and adds its own by
        // 2^(m_i - M').  The order is fixed, so the result does not depend on
        // which workgroup merges; that workgroup takes its own part from
        // registers (the same values it stored) and loads each other part's
        // O, m and l in one batch, one memory round trip per part.
        if (grp == 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                f32x16 own[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db) own[db] = oacc[rb][db];
                float M = 0.f, L = 0.f;
                for (int i = 0; i < nparts; ++i) {
                    f32x16 oi[DB];
                    float mi, li;
                    if (i == part) {
#pragma unroll
                        for (int db = 0; db < DB; ++db) oi[db] = own[db];
                        mi = m_run[rb];
                        li = l_run[rb];
                    } else {
                        const float *const pi = part0 + i * sstride;
#pragma unroll
                        for (int db = 0; db < DB; ++db)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oi[db][r] = load_dev(&pi[((rb * DB + db) * 16 + r) * 64]);
                        mi = load_dev(&pi[(MO + rb) * 64]);
                        li = load_dev(&pi[(MO + RB + rb) * 64]);
                    }
                    if (i == 0) {
#pragma unroll
                        for (int db = 0; db < DB; ++db) oacc[rb][db] = oi[db];
                        M = mi;
                        L = li;
                    } else {
                        const float Mn = fmaxf(M, mi);
                        const float aa = __builtin_amdgcn_exp2f(M - Mn), ai = __builtin_amdgcn_exp2f(mi - Mn);
#pragma unroll
                        for (int db = 0; db < DB; ++db)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                oacc[rb][db][r] = __builtin_fmaf(oi[db][r], ai, oacc[rb][db][r] * aa);
                        L = __builtin_fmaf(li, ai, L * aa);
                        M = Mn;
                    }
                }
                l_run[rb] = L;
            }
        }
    }

    // ---- epilogue: normalise, round to bf16 and store every row straight
    // into its destination slot (region p, row i, head g0 + h).  Each storing
    // wave first stages its rows in the LDS (the K/V rings are free by now),
    // then reads them back so that every store instruction writes whole
    // rows: 16 lanes x 16 B per 256-byte row at d = 128 (4 rows per
    // instruction), 8 lanes per 128-byte row at d = 64 (8 rows).  In the
    // staging buffer the 16-byte chunk c of row r sits at position
    // c ^ ((r / R256) % CPR), R256 rows per 256 bytes, so both the 8-byte
    // writes (32 rows, one column chunk) and the row reads are spread over
    // all LDS banks.
    float inv[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) inv[rb] = 1.0f / row_sum(l_run[rb]);
    constexpr int ROWB = D * 2;      // bytes per output row
    constexpr int CPR = ROWB / 16;   // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;    // rows per store instruction
    constexpr int R256 = 256 / ROWB; // rows per 256 bytes of LDS
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    lds_u8 *const stg = (lds_u8 *)lds_all + wq * RW * ROWB;
    __syncthreads();  // every wave is done with the K/V rings and the key-group hand-off
    if (grp == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int row = rb * 32 + il;
            const int sw = (row / R256) % CPR;
            // O^T element r of block db is column db*32 + 8(r/4) + 4g + r%4:
            // registers 4q4 .. 4q4+3 fill bytes 8g .. 8g+7 of chunk 4db + q4
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    u32x2 w;
                    w[0] = pack_bf16(oacc[rb][db][4 * q4] * inv[rb], oacc[rb][db][4 * q4 + 1] * inv[rb]);
                    w[1] = pack_bf16(oacc[rb][db][4 * q4 + 2] * inv[rb], oacc[rb][db][4 * q4 + 3] * inv[rb]);
                    *(lds_u32x2 *)(stg + row * ROWB + (((4 * db + q4) ^ sw) * 16) + 8 * g) = w;
                }
        }
    }
    __syncthreads();  // the staged rows are visible to every lane of their wave
    uint64_t tr_sb = 0;
    if constexpr (TRACE) tr_sb = __builtin_amdgcn_s_memrealtime();
    const Placement &o = a.out;
    if (grp == 0) {
        const int chunk = lane % CPR;
        const uint32_t rr = (uint32_t)o.region_rows;
#pragma unroll
        for (int j = 0; j < RW / RPI; ++j) {
            const int row = j * RPI + lane / CPR;
            const u32x4 val = *(const lds_u32x4 *)(stg + row * ROWB + ((chunk ^ ((row / R256) % CPR)) * 16));
            const int64_t sq = (int64_t)qt * BR + wq * RW + row;
            if (sq < S) {
                // S < 2^31 rows: the region arithmetic fits 32 bits
                const uint32_t p = (uint32_t)sq / rr;
                const uint32_t i = (uint32_t)sq - p * rr;
                uint16_t *dst = o.base + (((b * o.regions + p) * o.region_rows + i) * o.heads + o.head0 + h) * D;
                *(u32x4 *)(dst + chunk * 8) = val;
                if (a.wcount) atomicAdd(a.wcount + (dst + chunk * 8 - o.base) / 8, 1u);
            }
        }
    }
    if constexpr (TRACE) tr_rows = tr_sb;
    };

    // The work of this workgroup, one call site so the body is inlined once.
    //  * Plain builds: unit u = (b*Hl + h)*n_qtiles + qt, all keys.
    //  * XS builds, key split: unit u = ((b*Hl + h)*n_split + split)*n_qtiles
    //    + qt; split s of n takes units [s*U/n, (s+1)*U/n) of the U =
    //    tiles/KS units of KS tiles each (parts of at least 8 units), and its
    //    key groups halve that run.  The units that run side by side on one
    //    XCD read the same keys.
    //  * XS builds, stream-K (one key group, one row block per wave: the
    //    two-row-block kernel has no registers to spare for the loop):
    //    workgroup w takes iterations
    //    [w L, (w+1) L) of the sequence of (query tile, key tile) pairs, query
    //    tiles (bh * n_qtiles + qt) outermost, so every workgroup does the
    //    same work, in one round; a query tile's keys are cut at the
    //    workgroup boundaries into parts, numbered in key order.  Workgroups
    //    with neighbouring runs (the same head) run on one XCD.
    const int nt_all = (int)((a.S + KB - 1) / KB);  // key tiles of a query tile
    const int wid = xcd_unit(blockIdx.x, a.n_units, a.n_xcd);
    const bool sk = XS && KS == 1 && RB == 1 && a.sk_iters > 0;
    const int64_t L = a.sk_iters, T = nt_all;
    int64_t it = sk ? (int64_t)wid * L : 0;
    const int64_t end = sk ? ((int64_t)wid + 1) * L < (int64_t)a.n_units_q * T ? ((int64_t)wid + 1) * L
                                                                                : (int64_t)a.n_units_q * T
                           : 0;
    // The host launches ceil(total / L) workgroups, so every run is
    // non-empty; a workgroup past the end would otherwise take a query tile
    // beyond the last (and a negative tile count) in the loop below.
    if (sk && it >= end) return;
    do {
        int qt, bh, kt0, ntl, part, nparts;
        if (sk) {
            const int64_t tile = it / T;
            kt0 = (int)(it - tile * T);
            ntl = (int)(T - kt0 < end - it ? T - kt0 : end - it);
            const int first = (int)(tile * T / L), last = (int)(((tile + 1) * T - 1) / L);
            part = wid - first;
            nparts = last - first + 1;
            qt = (int)(tile % a.n_qtiles);
            bh = (int)(tile / a.n_qtiles);
            __syncthreads();  // the LDS of the previous item is free
            it += ntl;
        } else if (XS) {
            const int split = wid / a.n_qtiles % a.n_split;
            const int U = nt_all / KS;
            const int u0 = (int)((int64_t)split * U / a.n_split), u1 = (int)((int64_t)(split + 1) * U / a.n_split);
            qt = wid % a.n_qtiles;
            bh = wid / a.n_qtiles / a.n_split;
            kt0 = u0 * KS;
            ntl = u1 - u0;
            part = split;
            nparts = a.n_split;
        } else {
            qt = wid % a.n_qtiles;
            bh = wid / a.n_qtiles;
            kt0 = 0;
            ntl = nt_all / KS;
            part = 0;
            nparts = 1;
        }
        run(wid, qt, bh, kt0, ntl, part, nparts);
    } while (sk && it < end);
    if constexpr (TRACE) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const uint64_t tr_se = __builtin_amdgcn_s_memrealtime();
        const uint64_t tr_c1 = __builtin_amdgcn_s_memtime();
        if (threadIdx.x == 0) {
            uint64_t *t = a.trace + 4 * (int64_t)wid;
            t[0] = tr_t0;
            t[1] = tr_rows ? tr_rows : tr_se;
            t[2] = tr_se;
            t[3] = tr_c1 - tr_c0;
        }
    }
}

// Epilogue stores alone: the attention kernel's grid, work-unit order and
// store pattern (whole rows, 16 bytes per lane, RPI rows per instruction,
// each storing wave its RB*32 rows, only key group 0 storing), placed by the
// same Placement arithmetic, with a closed-form value instead of attention
// output: element (s, head g, column c) gets bf16 bits (7s + 13g + 3c) &
// 0x3FFF (finite, positive).  Measures what the destination layout sustains.
template <int D, int NW, int RB, int KS>
__global__ __launch_bounds__(64 * NW) void epilogue_only(Placement o, int64_t S, int32_t Hl, int32_t n_qtiles,
                                                         int32_t n_units, int32_t n_xcd)
{
    constexpr int CPR = D * 2 / 16, RPI = 64 / CPR, RW = 32 * RB, BR = RW * NW / KS;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int unit = xcd_unit(blockIdx.x, n_units, n_xcd);
    const int qt = unit % n_qtiles;
    const int bh = unit / n_qtiles;
    const int h = bh % Hl;
    const int64_t b = bh / Hl;
    if (wave >= NW / KS) return;
    const int chunk = lane % CPR;
    const uint32_t rr = (uint32_t)o.region_rows;
    const int64_t gh = o.head0 + h;
#pragma unroll
    for (int j = 0; j < RW / RPI; ++j) {
        const int64_t s_q = (int64_t)qt * BR + wave * RW + j * RPI + lane / CPR;
        if (s_q >= S) continue;
        const uint32_t p = (uint32_t)s_q / rr;
        const uint32_t i = (uint32_t)s_q - p * rr;
        uint16_t *dst = o.base + (((b * o.regions + p) * o.region_rows + i) * o.heads + gh) * D;
        const unsigned base = (unsigned)(7 * s_q + 13 * gh);
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned c = chunk * 8 + 2 * e;
            w[e] = ((base + 3 * c) & 0x3FFFu) | (((base + 3 * (c + 1)) & 0x3FFFu) << 16);
        }
        *(u32x4 *)(dst + chunk * 8) = w;
    }
}

// Serial All-to-All: each thread copies one 16-byte chunk.  For a fixed
// (b, s) the Hl*d local elements are contiguous in O_local and also
// contiguous in the destination row (heads g0 .. g0+Hl-1 are adjacent).
__global__ __launch_bounds__(256) void permute_rows(const uint16_t *src, uint32_t n_chunks,
                                                    uint32_t chunks_per_slab, uint32_t S,
                                                    Placement out, int d)
{
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;
    if (c >= n_chunks) return;
    const uint32_t slab = c / chunks_per_slab;       // = b*S + s
    const uint32_t within = c - slab * chunks_per_slab;
    const uint32_t b = slab / S, s = slab - b * S;
    const uint32_t p = s / (uint32_t)out.region_rows;
    const uint32_t i = s - p * (uint32_t)out.region_rows;
    uint16_t *dst = out.base + ((((int64_t)b * out.regions + p) * out.region_rows + i) * out.heads +
                                out.head0) * d + (int64_t)within * 8;
    *(u32x4 *)dst = *(const u32x4 *)(src + (int64_t)c * 8);
}

// Serial pre-attention All-to-All: each thread copies one 16-byte chunk of
// X_local [B][S][Hl][d] from its slot of the sequence-partitioned input
// (described by a Placement like the exchange's destination: row s of local
// head h sits in region p = s / region_rows, row i, head head0 + h).  For a
// fixed (b, s) the Hl*d elements are contiguous on both sides.
__global__ __launch_bounds__(256) void gather_rows(Placement in, uint32_t n_chunks,
                                                   uint32_t chunks_per_slab, uint32_t S,
                                                   uint16_t *dst, int d)
{
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;
    if (c >= n_chunks) return;
    const uint32_t slab = c / chunks_per_slab;       // = b*S + s
    const uint32_t within = c - slab * chunks_per_slab;
    const uint32_t b = slab / S, s = slab - b * S;
    const uint32_t p = s / (uint32_t)in.region_rows;
    const uint32_t i = s - p * (uint32_t)in.region_rows;
    const uint16_t *src = in.base + ((((int64_t)b * in.regions + p) * in.region_rows + i) * in.heads +
                                     in.head0) * d + (int64_t)within * 8;
    *(u32x4 *)(dst + (int64_t)c * 8) = *(const u32x4 *)src;
}

// Zero n 16-byte chunks (the arrival counts of the fixed device scratch,
// cleared before each call that uses it; a kernel rather than a memset, so
// that the call can be captured into a HIP graph).
__global__ __launch_bounds__(256) void zero_chunks(u32x4 *p, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = u32x4{0u, 0u, 0u, 0u};
}

// Fixed device scratch of the call that allocates nothing
// (attn_ulysses_fused_noalloc): the key-split workspace (arrival counts, then
// partial results) in a file-scope device array.  Every GPU the library runs
// on holds one copy, at its own address, until the process ends.  Host code
// must never pass this name to a kernel or a copy: it reaches the memory only
// through the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Compute units and XCDs of the current device, queried once per device.
// Without a device (the size queries run on hosts without a GPU) the full
// MI355X is assumed: 256 CUs in 8 XCDs.  A failed query leaves no error
// behind for the caller's next hipGetLastError.
struct DeviceInfo {
    int cus, xcds;
};
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_cus[kMaxDevices];
std::atomic<int> g_dev_xcds[kMaxDevices];

DeviceInfo device_info()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return {256, 8};
    }
    int cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    int xcds = g_dev_xcds[dev].load(std::memory_order_relaxed);
    if (cus > 0 && xcds > 0) return {cus, xcds};
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds <= 0) {
        (void)hipGetLastError();
        xcds = 1;
    }
    g_dev_cus[dev].store(cus, std::memory_order_relaxed);
    g_dev_xcds[dev].store(xcds, std::memory_order_relaxed);
    return {cus, xcds};
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Launch shape of the attention kernel for a problem: waves per workgroup,
// 32-row blocks per wave, keys per K/V tile, key groups.  With at least
// cus/2 units of 256 rows (half a workgroup per CU; 128 on the MI355X's 256
// CUs): 8 waves on 64-key tiles (one K/V tile per 256 query rows); for
// d = 64, 8 waves of two row blocks each on 32-key tiles (512 rows per unit;
// each LDS operand fragment feeds two MFMAs, ~4% faster per row) when that
// also gives at least cus/2 units and its estimated time -- rounds of units
// over the CUs times the rows a unit processes -- is at most 25/24 of the
// other's.  Below cus/2 units: 128-row units, as two key groups of 4 waves
// on 32-key tiles when the 32-key tile count is even, else as 4 waves on
// 64-key tiles.
struct LaunchShape {
    int nw, rb, kb, ks;
    int rows() const { return 32 * rb * nw / ks; }
};

// UA_TILE (environment, read once per process; for tuning): forces the
// launch shape, as query rows x keys per tile: "256x64" (8 waves), "512x32"
// (8 waves of two row blocks, d = 64 only), "128x64" (4 waves) or "128x32"
// (two key groups of 4 waves, an even number of 32-key tiles only).  Any
// other value, or a shape it does not fit, leaves the choice below.
enum class TileOverride { none, r256k64, r512k32, r128k64, r128k32 };
TileOverride tile_override_setting()
{
    static const TileOverride v = [] {
        const char *e = std::getenv("UA_TILE");
        if (!e) return TileOverride::none;
        const std::string t(e);
        if (t == "256x64") return TileOverride::r256k64;
        if (t == "512x32") return TileOverride::r512k32;
        if (t == "128x64") return TileOverride::r128k64;
        if (t == "128x32") return TileOverride::r128k32;
        return TileOverride::none;
    }();
    return v;
}
bool tile_override(int64_t S, int d, LaunchShape *ls)
{
    switch (tile_override_setting()) {
    case TileOverride::r256k64: *ls = {8, 1, 64, 1}; return true;
    case TileOverride::r512k32:
        if (d != 64) return false;
        *ls = {8, 2, 32, 1};
        return true;
    case TileOverride::r128k64: *ls = {4, 1, 64, 1}; return true;
    case TileOverride::r128k32: {
        const int64_t nt = (S + 31) / 32;
        if (nt < 2 || nt % 2 != 0) return false;
        *ls = {8, 1, 32, 2};
        return true;
    }
    default: return false;
    }
}

LaunchShape launch_shape(int64_t B, int64_t S, int64_t Hl, int d, int64_t cus)
{
    LaunchShape forced;
    if (tile_override(S, d, &forced)) return forced;
    const auto units = [&](int64_t rows) { return B * Hl * ((S + rows - 1) / rows); };
    // rounds of units over the CUs times the rows a unit processes
    const auto cost = [&](int64_t rows) { return (units(rows) + cus - 1) / cus * (S < rows ? S : rows); };
    if (units(256) < cus / 2) {
        // 128-row units: two key groups of 4 waves on 32-key tiles (two waves
        // per SIMD) when the tile count is even, else 4 waves (one per SIMD)
        const int64_t nt = (S + 31) / 32;
        if (nt >= 2 && nt % 2 == 0) return {8, 1, 32, 2};
        return {4, 1, 64, 1};
    }
    // per-row time of the two-row-block shape: 24/25 of the one-row-block one
    if (d == 64 && units(512) >= cus / 2 && cost(512) * 24 <= cost(256) * 25) return {8, 2, 32, 1};
    return {8, 1, 64, 1};
}

// Key split across workgroups for launches with fewer than 1024 query tiles
// (four rounds over the CUs), where too few tiles or a last round that fills
// the CUs poorly leave CUs idle: the launch shape and the number n of
// workgroups per query tile, for a device of `cus` compute units.  The
// candidates are the plain call's shape and, where that shape uses 128-row
// units (fewer than cus/2 units of 256 rows), the 256-row shape on 64-key
// tiles; only 8-wave shapes split.  Each candidate with n in 1 .. 4 costs
// (rounds of n * units over the CUs) * (keys one wave processes + 512
// + 128 (n - 1)): 512 keys' worth of time stand for a workgroup's fixed cost
// (prologue, partial write, count) and 128 for each part the merging
// workgroup loads (one memory round trip), both fitted to measured 2- to
// 16-way splits of dit_image and dit_long.  Parts hold at least 8 units of
// KS tiles.  The cheapest wins, ties going to the smaller n and then to the
// plain call's shape; n = 1 means the plain launch (the other shape only
// competes with a split).
constexpr int kSplitMaxN = 4;
constexpr int64_t kSplitMaxTiles = 1024;
constexpr int64_t kCountBytes = kSplitMaxTiles * 4;
constexpr int64_t kMinSplitUnits = 8;
constexpr int64_t kSplitFixedKeys = 512;
constexpr int64_t kSplitPartKeys = 128;

struct SplitPlan {
    LaunchShape ls;
    int n;         // parts per query tile (stream-K: the most any query tile has)
    int sk_iters;  // stream-K: (query tile, key tile) iterations per workgroup; 0: no
};

// Stream-K candidate for a shape with one key group and one row block per
// wave: `cus` workgroups, each on L
// = ceil(total / cus) consecutive iterations of the (query tile, key tile)
// sequence.  Returns L (0 when the runs would be under 16 key tiles) and the
// most parts any query tile is cut into.
int64_t stream_k(int64_t qtiles, int64_t T, int64_t cus, int *max_parts)
{
    const int64_t total = qtiles * T;
    const int64_t L = (total + cus - 1) / cus;
    if (L < 16) return 0;
    int mp = 1;
    for (int64_t t = 0; t < qtiles; ++t) {
        const int64_t first = t * T / L, last = ((t + 1) * T - 1) / L;
        mp = (int)(last - first + 1) > mp ? (int)(last - first + 1) : mp;
    }
    *max_parts = mp;
    return L;
}

SplitPlan split_plan(int64_t B, int64_t S, int64_t Hl, int d, int64_t cus)
{
    const LaunchShape plain = launch_shape(B, S, Hl, d, cus);
    const auto units = [&](const LaunchShape &ls) { return B * Hl * ((S + ls.rows() - 1) / ls.rows()); };
    SplitPlan best = {plain, 1, 0};
    if (units(plain) >= kSplitMaxTiles) return best;
    const int64_t U0 = (S + plain.kb - 1) / plain.kb / plain.ks;
    int64_t best_cost = (units(plain) + cus - 1) / cus * (U0 * plain.kb + kSplitFixedKeys);
    LaunchShape cands[2] = {plain, {8, 1, 64, 1}};
    LaunchShape forced;
    const int ncand = plain.rows() == 128 && !tile_override(S, d, &forced) ? 2 : 1;
    for (int n = 1; n <= kSplitMaxN; ++n)
        for (int c = 0; c < ncand; ++c) {
            const LaunchShape &ls = cands[c];
            if (ls.nw != 8 || (n == 1 && c > 0)) continue;
            const int64_t U = (S + ls.kb - 1) / ls.kb / ls.ks;  // units of ks tiles
            if (n > 1 && U / n < kMinSplitUnits) continue;
            const int64_t cost = (units(ls) * n + cus - 1) / cus *
                                 ((U + n - 1) / n * ls.kb + kSplitFixedKeys + kSplitPartKeys * (n - 1));
            if (cost < best_cost) {
                best = {ls, n, 0};
                best_cost = cost;
            }
        }
    // stream-K: one round of equal runs; each workgroup pays up to two work
    // items' fixed cost and the merging one a round trip per other part.  It
    // has to beat the best plan above by 3% (a full last round gains nothing)
    for (int c = 0; c < ncand; ++c) {
        const LaunchShape &ls = cands[c];
        if (ls.nw != 8 || ls.ks != 1 || ls.rb != 1) continue;
        int mp = 1;
        const int64_t L = stream_k(units(ls), (S + ls.kb - 1) / ls.kb, cus, &mp);
        if (L == 0 || mp < 2) continue;
        const int64_t cost = L * ls.kb + 2 * kSplitFixedKeys + kSplitPartKeys * (mp - 1);
        if (cost * 100 < best_cost * 97) {
            best = {ls, mp, (int)L};
            best_cost = cost * 100 / 97;
        }
    }
    if (best.n == 1) best.ls = plain;
    // every split plan has fewer than kSplitMaxTiles query tiles (the other
    // candidate has fewer tiles than the plain shape), so its counts fit
    // kCountBytes
    return best;
}

template <bool TRACE>
const void *attention_kernel(int d, const LaunchShape &ls)
{
    if (d == 128) {
        if (ls.ks == 2) return (const void *)attn_fwd<128, 8, 1, 32, 2, false, TRACE>;
        return ls.nw == 8 ? (const void *)attn_fwd<128, 8, 1, 64, 1, false, TRACE>
                          : (const void *)attn_fwd<128, 4, 1, 64, 1, false, TRACE>;
    }
    if (ls.ks == 2) return (const void *)attn_fwd<64, 8, 1, 32, 2, false, TRACE>;
    if (ls.rb == 2) return (const void *)attn_fwd<64, 8, 2, 32, 1, false, TRACE>;
    return ls.nw == 8 ? (const void *)attn_fwd<64, 8, 1, 64, 1, false, TRACE>
                      : (const void *)attn_fwd<64, 4, 1, 64, 1, false, TRACE>;
}

// The key-split builds (8-wave shapes only).
template <bool TRACE>
const void *attention_kernel_xs(int d, const LaunchShape &ls)
{
    if (d == 128)
        return ls.ks == 2 ? (const void *)attn_fwd<128, 8, 1, 32, 2, true, TRACE>
                          : (const void *)attn_fwd<128, 8, 1, 64, 1, true, TRACE>;
    if (ls.ks == 2) return (const void *)attn_fwd<64, 8, 1, 32, 2, true, TRACE>;
    if (ls.rb == 2) return (const void *)attn_fwd<64, 8, 2, 32, 1, true, TRACE>;
    return (const void *)attn_fwd<64, 8, 1, 64, 1, true, TRACE>;
}

// Workspace of a key-split launch: one uint32 arrival count per query tile
// in a region of fixed size (a split only runs for fewer than
// kSplitMaxTiles query tiles), then per query tile and split the partial
// results of the NW/KS storing waves, lane-interleaved: (RB*(d/32)*16 +
// 2*RB) floats per lane.  The fixed count region keeps every shape's counts
// clear of every other shape's partials, so one workspace (counts zero)
// serves any shape it fits.
int64_t part_floats_per_split(const LaunchShape &ls, int d)
{
    return (int64_t)(ls.nw / ls.ks) * (ls.rb * (d / 32) * 16 + 2 * ls.rb) * 64;
}

}  // namespace

int device_xcd_count() { return device_info().xcds; }

int64_t attention_units(int64_t B, int64_t S, int64_t Hl, int d)
{
    const LaunchShape ls = launch_shape(B, S, Hl, d, device_info().cus);
    return B * Hl * ((S + ls.rows() - 1) / ls.rows());
}

int64_t attention_units_ws(int64_t B, int64_t S, int64_t Hl, int d)
{
    const SplitPlan sp = split_plan(B, S, Hl, d, device_info().cus);
    const int64_t units = B * Hl * ((S + sp.ls.rows() - 1) / sp.ls.rows());
    if (sp.n <= 1) return attention_units(B, S, Hl, d);
    if (sp.sk_iters > 0) return (units * ((S + sp.ls.kb - 1) / sp.ls.kb) + sp.sk_iters - 1) / sp.sk_iters;
    return units * sp.n;
}

int key_split(int64_t B, int64_t S, int64_t Hl, int d) { return split_plan(B, S, Hl, d, device_info().cus).n; }

int64_t stream_k_iters(int64_t B, int64_t S, int64_t Hl, int d)
{
    return split_plan(B, S, Hl, d, device_info().cus).sk_iters;
}

int64_t workspace_count_bytes(int64_t B, int64_t S, int64_t Hl, int d)
{
    const SplitPlan sp = split_plan(B, S, Hl, d, device_info().cus);
    return sp.n == 1 ? 0 : kCountBytes;
}

int64_t workspace_bytes(int64_t B, int64_t S, int64_t Hl, int d)
{
    const SplitPlan sp = split_plan(B, S, Hl, d, device_info().cus);
    if (sp.n == 1) return 0;
    const int64_t tiles = B * Hl * ((S + sp.ls.rows() - 1) / sp.ls.rows());
    return kCountBytes + tiles * sp.n * part_floats_per_split(sp.ls, d) * 4;  // n parts' slots per query tile
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int64_t in_heads, int64_t in_head0, int64_t B, int64_t S, int64_t Hl,
                            int d, float scale, const Placement &out, hipStream_t stream,
                            uint64_t *trace, void *workspace, unsigned *wcount)
{
    const DeviceInfo dv = device_info();
    const SplitPlan sp = workspace ? split_plan(B, S, Hl, d, dv.cus)
                                   : SplitPlan{launch_shape(B, S, Hl, d, dv.cus), 1, 0};
    const LaunchShape ls = sp.ls;
    const int n_split = sp.n;
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.S = S;
    a.Hl = (int32_t)Hl;
    a.in_heads = (int32_t)in_heads;
    a.in_head0 = (int32_t)in_head0;
    a.n_qtiles = (int32_t)((S + ls.rows() - 1) / ls.rows());
    a.n_units = (int32_t)(B * Hl * a.n_qtiles);
    a.n_xcd = dv.xcds;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.trace = trace;
    a.wcount = wcount;
    a.n_split = n_split;
    a.ws_cnt = nullptr;
    a.ws_part = nullptr;
    const void *fn;
    a.sk_iters = sp.sk_iters;
    a.n_units_q = a.n_units;
    if (n_split > 1) {
        a.ws_cnt = (unsigned *)workspace;
        a.ws_part = (float *)((char *)workspace + kCountBytes);
        // stream-K: one workgroup per run of sk_iters iterations (at most one
        // per CU; the last run may be shorter); else n_split per query tile
        const int64_t total = (int64_t)a.n_units * ((S + ls.kb - 1) / ls.kb);
        a.n_units = sp.sk_iters > 0 ? (int32_t)((total + sp.sk_iters - 1) / sp.sk_iters) : a.n_units * n_split;
        fn = trace ? attention_kernel_xs<true>(d, ls) : attention_kernel_xs<false>(d, ls);
    } else {
        fn = trace ? attention_kernel<true>(d, ls) : attention_kernel<false>(d, ls);
    }
    void *args[] = {&a};
    return hipLaunchKernel(fn, dim3(a.n_units), dim3(64 * ls.nw), args, 0, stream);
}

hipError_t launch_attention_scratch(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t B,
                                    int64_t S, int64_t Hl, int d, float scale, const Placement &out,
                                    hipStream_t stream)
{
    if (workspace_bytes(B, S, Hl, d) == 0)  // no split: the plain launch, no scratch
        return launch_attention(q, k, v, Hl, 0, B, S, Hl, d, scale, out, stream);
    void *ws = nullptr;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    // the counts must start at zero whatever an earlier call left behind
    u32x4 *cnt = (u32x4 *)ws;
    int n = (int)(kCountBytes / 16);
    void *zargs[] = {(void *)&cnt, &n};
    e = hipLaunchKernel((const void *)zero_chunks, dim3((n + 255) / 256), dim3(256), zargs, 0, stream);
    if (e != hipSuccess) return e;
    return launch_attention(q, k, v, Hl, 0, B, S, Hl, d, scale, out, stream, nullptr, ws);
}

hipError_t launch_epilogue_only(int64_t B, int64_t S, int64_t Hl, int d, const Placement &out,
                                hipStream_t stream)
{
    const DeviceInfo dv = device_info();
    const LaunchShape ls = launch_shape(B, S, Hl, d, dv.cus);
    Placement o = out;
    int64_t S64 = S;
    int32_t Hl32 = (int32_t)Hl;
    int32_t n_qtiles = (int32_t)((S + ls.rows() - 1) / ls.rows());
    int32_t n_units = (int32_t)(B * Hl * n_qtiles);
    int32_t n_xcd = dv.xcds;
    void *args[] = {&o, &S64, &Hl32, &n_qtiles, &n_units, &n_xcd};
    const void *fn;
    if (ls.ks == 2)
        fn = d == 128 ? (const void *)epilogue_only<128, 8, 1, 2> : (const void *)epilogue_only<64, 8, 1, 2>;
    else if (d == 128)
        fn = ls.nw == 8 ? (const void *)epilogue_only<128, 8, 1, 1> : (const void *)epilogue_only<128, 4, 1, 1>;
    else if (ls.rb == 2)
        fn = (const void *)epilogue_only<64, 8, 2, 1>;
    else
        fn = ls.nw == 8 ? (const void *)epilogue_only<64, 8, 1, 1> : (const void *)epilogue_only<64, 4, 1, 1>;
    return hipLaunchKernel(fn, dim3(n_units), dim3(64 * ls.nw), args, 0, stream);
}

hipError_t launch_permute(const uint16_t *o_local, int64_t B, int64_t S, int64_t Hl, int d,
                          const Placement &out, hipStream_t stream)
{
    uint32_t cps = (uint32_t)(Hl * d / 8);
    uint32_t n = (uint32_t)(B * S * cps);
    uint32_t S32 = (uint32_t)S;
    int d32 = d;
    Placement o = out;
    const uint16_t *src = o_local;
    void *args[] = {(void *)&src, &n, &cps, &S32, &o, &d32};
    return hipLaunchKernel((const void *)permute_rows, dim3((n + 255) / 256), dim3(256), args, 0,
                           stream);
}

hipError_t launch_gather(const Placement &in, int64_t B, int64_t S, int64_t Hl, int d,
                         uint16_t *x_local, hipStream_t stream)
{
    uint32_t cps = (uint32_t)(Hl * d / 8);
    uint32_t n = (uint32_t)(B * S * cps);
    uint32_t S32 = (uint32_t)S;
    int d32 = d;
    Placement i = in;
    uint16_t *dst = x_local;
    void *args[] = {&i, &n, &cps, &S32, (void *)&dst, &d32};
    return hipLaunchKernel((const void *)gather_rows, dim3((n + 255) / 256), dim3(256), args, 0,
                           stream);
}

}  // namespace ua
