// moe_api.cpp -- C ABI of the MoE expert path with the fused Combine
// (declared in include/moe_combine.h; part of libulysses_attn.so).
//
// Host-side only: argument validation (no device access), the receive layout
// of a rank, and launches.  The library allocates nothing: the persistent
// form's counters live in the caller's workspace.

#include "moe_combine.h"

#include <stdint.h>

#include <vector>

#include "moe_internal.h"
#include "ulysses_attn.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by the MoE calls.
int check_moe_shape(const moe_shape *shp, int P)
{
    if (!shp) return UA_ERR_NULL;
    const int64_t T = shp->T, hid = shp->hidden, inter = shp->inter, E = shp->E, k = shp->k;
    if (P < 1 || T < 0 || hid < 256 || hid % 256 != 0 || inter < 128 || inter % 128 != 0 || E < 1 || E % P != 0 ||
        k < 1 || k > E)
        return UA_ERR_SHAPE;
    // 32-bit offsets inside the kernels: token rows of x, one expert's weights,
    // slots and receive rows
    const int64_t lim = (int64_t)1 << 32;
    if (T > lim / P || P * T * hid * 2 >= lim || 2 * inter * hid * 2 >= lim || P * T * k >= ((int64_t)1 << 31))
        return UA_ERR_UNSUPPORTED;
    return UA_OK;
}

// expert_offsets: 0 = off[0] <= ... <= off[E_l] = N <= P*T*k; N * max(inter,
// hidden) * 2 bytes addressable with 32-bit offsets.
int check_offsets(const int64_t *off, int64_t E_l, const moe_shape *shp, int P, int64_t *N)
{
    if (!off) return UA_ERR_NULL;
    if (off[0] != 0) return UA_ERR_SHAPE;
    for (int64_t e = 0; e < E_l; ++e)
        if (off[e + 1] < off[e]) return UA_ERR_SHAPE;
    *N = off[E_l];
    if (*N > P * shp->T * shp->k) return UA_ERR_SHAPE;
    const int64_t wide = shp->inter > shp->hidden ? shp->inter : shp->hidden;
    if (*N * wide * 2 >= ((int64_t)1 << 32)) return UA_ERR_UNSUPPORTED;
    return UA_OK;
}

// Words of the persistent form's workspace for these offsets, or -1 when
// the call needs more launches than the header holds queue counters for.
int64_t ws_words(const int64_t *offsets, int64_t E_l, int per_wave)
{
    const int64_t waves = (E_l + per_wave - 1) / per_wave, per_launch = moe::kMaxWave / per_wave;
    if ((waves + per_launch - 1) / per_launch > moe::kMaxLaunches) return -1;
    return moe::kWsHeader + moe::token_tiles(offsets, E_l);
}

// persistent: run the persistent form with `ws` (ws_bytes) as its counters
int experts_call(const void *x, const int32_t *row_slot, const float *topk_w, const int64_t *offsets,
                 const void *W1, const void *W2, int P, const moe_shape *shp, void *out, void *act,
                 int schedule, int per_wave, bool local, bool persistent, void *ws, size_t ws_bytes,
                 hipStream_t stream)
{
    int st = check_moe_shape(shp, P);
    if (st != UA_OK) return st;
    if (schedule != MOE_EXPERT_WAVE && schedule != MOE_INTERLEAVED) return UA_ERR_UNSUPPORTED;
    if (per_wave < 1 || per_wave > MOE_MAX_WAVE) return UA_ERR_UNSUPPORTED;
    const int64_t E_l = shp->E / P;
    int64_t N = 0;
    if ((st = check_offsets(offsets, E_l, shp, P, &N)) != UA_OK) return st;
    if (N == 0) return UA_OK;
    if (!x || !row_slot || !topk_w || !W1 || !W2 || !out || !act) return UA_ERR_NULL;
    if (!aligned16(x) || !aligned16(topk_w) || !aligned16(row_slot) || !aligned16(W1) || !aligned16(W2) ||
        !aligned16(out) || !aligned16(act))
        return UA_ERR_ALIGN;
    if (persistent) {
        const int64_t words = ws_words(offsets, E_l, per_wave);
        if (words < 0) return UA_ERR_UNSUPPORTED;
        if (!ws) return UA_ERR_NULL;
        if (!aligned16(ws)) return UA_ERR_ALIGN;
        if (ws_bytes < (size_t)words * 4) return UA_ERR_WORKSPACE;
    }
    moe::Problem p;
    p.x = (const uint16_t *)x;
    p.row_slot = row_slot;
    p.topk_w = topk_w;
    p.w1 = (const uint16_t *)W1;
    p.w2 = (const uint16_t *)W2;
    p.act = (uint16_t *)act;
    p.out = (uint16_t *)out;
    p.offsets = offsets;
    p.E_l = E_l;
    p.hidden = shp->hidden;
    p.inter = shp->inter;
    p.k = shp->k;
    const hipError_t e = persistent ? moe::launch_moe_persist(p, schedule, per_wave, local, (unsigned *)ws, stream)
                                    : moe::launch_moe(p, schedule, per_wave, local, stream);
    return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

}  // namespace

extern "C" {

int moe_recv_layout(const int32_t *topk_idx, int rank, int P, const moe_shape *shp, int64_t *expert_offsets,
                    int32_t *row_slot, int64_t capacity)
{
    int st = check_moe_shape(shp, P);
    if (st != UA_OK) return st;
    if (rank < 0 || rank >= P) return UA_ERR_RANK;
    if (!expert_offsets) return UA_ERR_NULL;
    const int64_t E_l = shp->E / P, slots = P * shp->T * shp->k;
    if (slots > 0 && (!topk_idx || !row_slot)) return UA_ERR_NULL;
    // counting sort of this rank's slots by local expert; slots stay in
    // increasing order within an expert
    std::vector<int64_t> count(E_l + 1, 0);
    for (int64_t s = 0; s < slots; ++s) {
        const int64_t g = topk_idx[s];
        if (g < 0 || g >= shp->E) return UA_ERR_SHAPE;
        if (g / E_l == rank) ++count[g - (int64_t)rank * E_l + 1];
    }
    for (int64_t e = 0; e < E_l; ++e) count[e + 1] += count[e];
    if (count[E_l] > capacity) return UA_ERR_SHAPE;
    for (int64_t e = 0; e <= E_l; ++e) expert_offsets[e] = count[e];
    for (int64_t s = 0; s < slots; ++s) {
        const int64_t g = topk_idx[s];
        if (g / E_l == rank) row_slot[count[g - (int64_t)rank * E_l]++] = (int32_t)s;
    }
    return UA_OK;
}

int moe_experts_combine(const void *x, const int32_t *row_slot, const float *topk_w,
                        const int64_t *expert_offsets, const void *W1, const void *W2, int P,
                        const moe_shape *shp, void *combine, void *act, int schedule, int experts_per_wave,
                        hipStream_t stream)
{
    return experts_call(x, row_slot, topk_w, expert_offsets, W1, W2, P, shp, combine, act, schedule,
                        experts_per_wave, false, false, nullptr, 0, stream);
}

int moe_experts_local(const void *x, const int32_t *row_slot, const float *topk_w, const int64_t *expert_offsets,
                      const void *W1, const void *W2, int P, const moe_shape *shp, void *y_local, void *act,
                      int experts_per_wave, hipStream_t stream)
{
    return experts_call(x, row_slot, topk_w, expert_offsets, W1, W2, P, shp, y_local, act, MOE_EXPERT_WAVE,
                        experts_per_wave, true, false, nullptr, 0, stream);
}

size_t moe_workspace_bytes(int P, const moe_shape *shp)
{
    if (check_moe_shape(shp, P) != UA_OK) return 0;
    // token tiles of any layout: at most N / 256 + E_l with N <= P*T*k
    const int64_t E_l = shp->E / P, n = moe::kWsHeader + (P * shp->T * shp->k) / 256 + E_l;
    return (size_t)(((n * 4 + 255) / 256) * 256);
}

int moe_experts_combine_ws(const void *x, const int32_t *row_slot, const float *topk_w,
                           const int64_t *expert_offsets, const void *W1, const void *W2, int P,
                           const moe_shape *shp, void *combine, void *act, int schedule, int experts_per_wave,
                           void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return experts_call(x, row_slot, topk_w, expert_offsets, W1, W2, P, shp, combine, act, schedule,
                        experts_per_wave, false, true, workspace, workspace_bytes, stream);
}

int moe_experts_local_ws(const void *x, const int32_t *row_slot, const float *topk_w,
                         const int64_t *expert_offsets, const void *W1, const void *W2, int P,
                         const moe_shape *shp, void *y_local, void *act, int experts_per_wave, void *workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    return experts_call(x, row_slot, topk_w, expert_offsets, W1, W2, P, shp, y_local, act, MOE_EXPERT_WAVE,
                        experts_per_wave, true, true, workspace, workspace_bytes, stream);
}

int moe_combine_scatter(const void *y_local, const int32_t *row_slot, int64_t N, int P, const moe_shape *shp,
                        void *combine, hipStream_t stream)
{
    int st = check_moe_shape(shp, P);
    if (st != UA_OK) return st;
    if (N < 0 || N > P * shp->T * shp->k) return UA_ERR_SHAPE;
    if (N == 0) return UA_OK;
    if (!y_local || !row_slot || !combine) return UA_ERR_NULL;
    if (!aligned16(y_local) || !aligned16(combine)) return UA_ERR_ALIGN;
    const hipError_t e = moe::launch_scatter((const uint16_t *)y_local, row_slot, N, shp->hidden,
                                             (uint16_t *)combine, stream);
    return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

}  // extern "C"
