// ua_kernels.hip -- gfx950 (MI355X) kernels for one Ulysses rank's attention
// with the post-attention All-to-All fused into the output epilogue, and the
// stand-alone permute used by the serial baseline.
//
// Method (X-Stage paper, arXiv 2607.23264): Fig. 5 of the pith.science review
// page (Ulysses attention; steps d-e are attention plus the post-attention
// All-to-All), Fig. 6 (FlashAttention's Q-loop: each output tile is owned by
// the worker that runs the loop over all KV tiles for it) and Fig. 7 (the
// output-tile owner issues the exchange stores itself, then moves on).
//
// Design for CDNA4, not a translation of the pages' FlashAttention-3/4:
//  * one workgroup = 4 wave64s = one work unit of 128 query rows of one
//    (batch, local head); each wave owns 32 query rows;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K streams from LDS as the A operand and the
//    wave's Q rows stay in VGPRs as the B operand.  The accumulator layout
//    then gives every lane ONE query row (lane % 32) and 16 keys, so the
//    row max needs one cross-half swap (v_permlane32_swap) per KV tile and
//    the row sum none until the end;
//  * P^T is fed from those same registers (rounded to bf16) as the B operand
//    of O^T += V^T P^T; V^T comes from the row-major V tile through the
//    gfx950 transposing LDS read ds_read_b64_tr_b16;
//  * K and V tiles (64 keys) go global -> LDS with global_load_lds_dwordx4
//    (no VGPR staging), double buffered; both tiles are XOR-swizzled in
//    16-byte chunks so the MFMA operand reads are free of bank conflicts;
//  * online softmax in fp32 with exp2 (log2 e folded into the scale);
//  * epilogue: each lane normalises its row and stores it straight to the
//    destination slot computed from (rank, P) -- the fused All-to-All.  The
//    local (serial) output is the same epilogue with one region.
//  * workgroup ids are remapped so that consecutive work units of one head
//    run on the same XCD and share its L2 while they stream the same K/V.

#include "ua_internal.h"

#include <math.h>

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

constexpr int kWaves = 4;             // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;      // query rows per work unit
constexpr int kBn = 64;               // keys per KV tile

struct AttnArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    Placement out;
    int64_t S;
    int32_t Hl;
    int32_t n_qtiles;
    int32_t n_units;
    float scale_log2;  // softmax scale * log2(e)
};

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi)
{
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, RNE
    return __builtin_bit_cast(unsigned, h);
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

// Logical work unit of this workgroup.  Workgroup i is dispatched to XCD
// i % 8; give each XCD a contiguous run of units (same head, neighbouring Q
// tiles) so they share K/V in that XCD's L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_unit(int bid, int n)
{
    const int xcd = bid & 7, k = bid >> 3;
    const int q = n >> 3, r = n & 7;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void attn_fwd(AttnArgs a)
{
    constexpr int RB = D * 2;             // bytes per K/V row
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int RPL = 256 / RB;         // rows per 256-byte LDS bank line
    constexpr int TILE = kBn * RB;        // bytes of one K (or V) tile
    constexpr int NLD = TILE / (kWaves * 1024);  // 1 KiB global->LDS copies per wave
    constexpr int KK = D / 16;            // MFMA k-steps over d for S^T
    constexpr int DB = D / 32;            // 32-row blocks of O^T over d
    static_assert(NLD >= 1 && TILE % (kWaves * 1024) == 0, "tile split");

    // Two K and two V tiles as four distinct arrays: the compiler can then
    // tell the reads of one buffer from the asynchronous global->LDS writes
    // into the other, and needs no wait on those writes mid-iteration.
    __shared__ __attribute__((aligned(1024))) unsigned char k0s[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char k1s[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char v0s[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char v1s[TILE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int il = lane & 31;  // query row of this lane within the wave
    const int g = lane >> 5;   // half-wave

    const int unit = xcd_unit(blockIdx.x, a.n_units);
    const int qt = unit % a.n_qtiles;
    const int bh = unit / a.n_qtiles;
    const int h = bh % a.Hl;
    const int64_t b = bh / a.Hl;
    const int64_t S = a.S;
    const int rs = a.Hl * D;  // elements between sequence rows
    const int64_t head = (b * S * a.Hl + h) * D;
    const uint16_t *qh = a.q + head;
    const uint16_t *kh = a.k + head;
    const uint16_t *vh = a.v + head;

    // Swizzles (16-byte chunk index XOR), see the operand reads below.
    auto kswz = [](int row) { return (row / RPL) % CPR; };
    auto vswz = [](int row) { return 4 * ((row / RPL) % (CPR / 4)); };

    // Global->LDS copy of one KV tile: each wave moves NLD contiguous 1 KiB
    // pieces of each tile; lane L of a piece lands at byte 16*L of it, so the
    // lane fetches the global chunk that belongs there.  Per-lane element
    // offsets within a full tile are fixed; only the tile base moves.
    int koff[NLD], voff[NLD], lrow[NLD];
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const int lin = (wave * NLD + n) * 1024 + lane * 16;
        const int row = lin / RB;
        const int pos = (lin % RB) >> 4;
        lrow[n] = row;
        koff[n] = row * rs + (pos ^ kswz(row)) * 8;
        voff[n] = row * rs + (pos ^ vswz(row)) * 8;
    }
    auto issue = [&](int64_t kv0, lds_u8 *kd, lds_u8 *vd) {
        const uint16_t *kb = kh + kv0 * rs;
        const uint16_t *vb = vh + kv0 * rs;
        if (kv0 + kBn <= S) {
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                const int off = (wave * NLD + n) * 1024;
                __builtin_amdgcn_global_load_lds((gbl_void *)(kb + koff[n]), (lds_void *)(kd + off), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((gbl_void *)(vb + voff[n]), (lds_void *)(vd + off), 16, 0, 0);
            }
        } else {
            // Last, partial tile: keys past S read row S-1 (finite data,
            // masked out of the softmax).
            const int last = (int)(S - 1 - kv0);
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                const int off = (wave * NLD + n) * 1024;
                const int shift = (lrow[n] > last ? last - lrow[n] : 0) * rs;
                __builtin_amdgcn_global_load_lds((gbl_void *)(kb + koff[n] + shift), (lds_void *)(kd + off), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((gbl_void *)(vb + voff[n] + shift), (lds_void *)(vd + off), 16, 0, 0);
            }
        }
    };

    // This lane's query row; rows past S (ragged last tile) compute on row
    // S-1 and are not stored.
    const int64_t s_q = (int64_t)qt * kBr + wave * 32 + il;
    const int64_t s_ld = s_q < S ? s_q : S - 1;

    // B operand of S^T = K Q^T: lane holds Q[s][16kk + 8g .. +7].
    u32x4 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = *(const u32x4 *)(qh + s_ld * rs + 16 * kk + 8 * g);

    const int ntiles = (int)((S + kBn - 1) / kBn);
    const float c = a.scale_log2;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    // Running max of this row's scaled scores (log2 domain).  It is only a
    // stabiliser: it is raised when a tile's max exceeds it by more than 8
    // (a factor 256), so P stays below 2^8 and O rarely needs rescaling;
    // the final O / l is the same for any choice of it.
    float m_run = -INFINITY;
    float l_run = 0.f;  // this lane's part of the running row sum

    const int i16 = lane & 15;
    const int half = (lane >> 4) & 1;

    auto step = [&](int t, const lds_u8 *kt, const lds_u8 *vt, lds_u8 *kn, lds_u8 *vn) {
        // Tile t has landed for this wave; the barrier makes every wave's
        // part visible and ends all reads of the other buffer.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < ntiles) issue((int64_t)(t + 1) * kBn, kn, vn);

        // ---- S^T (64 keys x 32 queries) = K_t Q^T.  A operand: lane reads
        // K row jb*32 + il, d-chunk 2kk+g (16 B); the XOR swizzle spreads the
        // 16 rows a quarter-wave reads over all banks.
        f32x16 sacc[2];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[jb][r] = 0.f;
            const int row = jb * 32 + il;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int pos = (2 * kk + g) ^ kswz(row);
                const u32x4 kf = *(const lds_u32x4 *)(kt + row * RB + pos * 16);
                sacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[kk]), sacc[jb],
                    0, 0, 0);
            }
        }
        // Accumulator element r of block jb is key kv0 + jb*32 + 8(r/4) + 4g + r%4.
        const int64_t kv0 = (int64_t)t * kBn;
        if (kv0 + kBn > S) {
            const int lim = (int)(S - kv0);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (jb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= lim) sacc[jb][r] = -INFINITY;
        }

        // ---- online softmax (fp32, log2 domain).
        float mt = sacc[0][0];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[jb][r]);
        mt = row_max(mt) * c;
        const bool raise = mt > m_run + 8.0f;  // same in both lanes of a row
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float m_new = raise ? mt : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 if kept, 0 at start
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float mb = m_run;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[jb][r], c, -mb));
                sacc[jb][r] = p;
                l_run += p;
            }

        // ---- O^T (d x 32 queries) += V_t^T P^T, four 16-key chunks.
        // B operand (P^T): chunk cc takes registers 8(cc%2)..+7 of block cc/2,
        // i.e. element e is key 16cc + 8(e/4) + 4g + e%4.
        // A operand (V^T): lane needs V[those keys][db*32 + lane%32]; two
        // transposing reads, each giving 4 consecutive keys: in a 16-lane
        // group, source lane i16 points at V row (k0 + i16/4), columns
        // dd0 + 4(i16%4) .. +3, and result lane i16 gets column dd0 + i16.
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            u32x4 pb;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
                pb[e2] = pack_bf16(sacc[cc >> 1][8 * (cc & 1) + 2 * e2],
                                   sacc[cc >> 1][8 * (cc & 1) + 2 * e2 + 1]);
            const int row1 = 16 * cc + 4 * g + (i16 >> 2);
            const int row2 = row1 + 8;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dd = db * 32 + 16 * half + 4 * (i16 & 3);
                const int ch = dd >> 3, within = (dd & 7) * 2;
                const lds_u8 *p1 = vt + row1 * RB + ((ch ^ vswz(row1)) << 4) + within;
                const lds_u8 *p2 = vt + row2 * RB + ((ch ^ vswz(row2)) << 4) + within;
                const u32x2 a1 = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p1));
                const u32x2 a2 = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p2));
                const u32x4 af = {a1[0], a1[1], a2[0], a2[1]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, pb), oacc[db], 0, 0,
                    0);
            }
        }
    };

    lds_u8 *const K0 = (lds_u8 *)k0s;
    lds_u8 *const K1 = (lds_u8 *)k1s;
    lds_u8 *const V0 = (lds_u8 *)v0s;
    lds_u8 *const V1 = (lds_u8 *)v1s;
    issue(0, K0, V0);
    for (int t = 0; t < ntiles; t += 2) {
        step(t, K0, V0, K1, V1);
        if (t + 1 < ntiles) step(t + 1, K1, V1, K0, V0);
    }

    // ---- epilogue: normalise and store this lane's half of its row straight
    // into the destination slot (region p, row i, head g0 + h).
    const float lt = row_sum(l_run);
    const float inv = 1.0f / lt;
    if (s_q < S) {
        const Placement &o = a.out;
        const int64_t p = s_q / o.region_rows;
        const int64_t i = s_q - p * o.region_rows;
        uint16_t *dst = o.base + (((b * o.regions + p) * o.region_rows + i) * o.heads + o.head0 + h) * D;
        // O^T element r of block db is column db*32 + 8(r/4) + 4g + r%4.
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2 w;
                w[0] = pack_bf16(oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv);
                w[1] = pack_bf16(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
                *(u32x2 *)(dst + db * 32 + 8 * q4 + 4 * g) = w;
            }
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

}  // namespace

int64_t attention_units(int64_t B, int64_t S, int64_t Hl)
{
    return B * Hl * ((S + kBr - 1) / kBr);
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int64_t B, int64_t S, int64_t Hl, int d, float scale,
                            const Placement &out, hipStream_t stream)
{
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.S = S;
    a.Hl = (int32_t)Hl;
    a.n_qtiles = (int32_t)((S + kBr - 1) / kBr);
    a.n_units = (int32_t)attention_units(B, S, Hl);
    a.scale_log2 = scale * 1.4426950408889634f;
    void *args[] = {&a};
    const void *fn = d == 128 ? (const void *)attn_fwd<128> : (const void *)attn_fwd<64>;
    return hipLaunchKernel(fn, dim3(a.n_units), dim3(kThreads), args, 0, stream);
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

}  // namespace ua
