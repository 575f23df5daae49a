/*
 * moe_combine.h -- C ABI of the MoE expert path with the Combine exchange
 * fused into its Linear-2 epilogue (part of libulysses_attn.so).
 *
 * The operation (X-Stage paper, arXiv 2607.23264; arXiv abstract page,
 * Abstract; pith.science review page, "If this is right" and Figs. 4, 8, 9):
 * an expert-parallel rank runs its local experts' Linear-1 and Linear-2 on
 * the tokens routed to it, and the owner of each Linear-2 output tile stores
 * it straight into the Combine buffer of the tokens' source ranks (the remote
 * stores of the pages' MegaMoE kernel).  The Expert-Wave schedule runs the
 * local experts in waves of G, each wave's Linear-1 tiles and then its
 * Linear-2 tiles; the interleaved schedule runs wave w's Linear-2 tiles
 * interleaved with wave w+1's Linear-1 tiles, so that computation sits
 * between the Combine stores.  On one GPU the P source ranks are P regions
 * of one buffer.
 *
 * An expert (the gated feed-forward block of DeepSeek-style models):
 *   h = x W1^T, W1 [2*inter][hidden] (rows 0..inter-1 gate, inter.. up);
 *   a = SiLU(gate) * up, rounded to bf16 (it crosses HBM between the layers);
 *   y = a W2^T, W2 [hidden][inter]; SiLU(z) = z / (1 + exp(-z)).
 * bf16 inputs and weights, fp32 accumulation, bf16 output (round to nearest
 * even).  Inputs are expected to be finite.
 *
 * Layouts (bf16 as raw 16-bit patterns; every pointer 16-byte aligned):
 *   x        [P][T][hidden]  the tokens of every source rank (the dispatch
 *            exchange's receive side, read in place through row_slot);
 *   topk_w   [P][T][k] float routing weights;
 *   combine  [P][T][k][hidden] region p = source rank p; slot (p, t, j)
 *            receives topk_w[p][t][j] * y of the expert token t of rank p
 *            chose j-th, if that expert is local (other slots untouched);
 *   W1 [E_l][2*inter][hidden], W2 [E_l][hidden][inter]: this rank's experts;
 *   rows: the N tokens routed to this rank's experts, grouped by local
 *            expert: rows expert_offsets[e] .. expert_offsets[e+1]-1 belong
 *            to local expert e, and row i serves slot row_slot[i] =
 *            (p*T + t)*k + j (token p*T + t, choice j);
 *   act      [N][inter] bf16 workspace (Linear-1 output, caller-owned).
 * Sizes: hidden % 256 == 0, inter % 128 == 0, P*T*hidden*2 < 2^32 bytes,
 * 2*inter*hidden*2 < 2^32 bytes (one expert's W1).
 *
 * Ownership: the caller allocates and frees every buffer; the library
 * allocates nothing.  Calls are asynchronous on `stream` (a hipStream_t of
 * the device holding the buffers; NULL = its default stream).
 * Errors: status codes of ulysses_attn.h (UA_OK, UA_ERR_NULL,
 * UA_ERR_SHAPE, UA_ERR_ALIGN, UA_ERR_UNSUPPORTED, UA_ERR_HIP,
 * UA_ERR_WORKSPACE); arguments are
 * validated on the host before any device access.  row_slot entries are
 * not read on the host: each must be < P*T*k and name a slot whose expert is
 * the row's (moe_recv_layout produces exactly such rows).
 */
#ifndef MOE_COMBINE_H
#define MOE_COMBINE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t T;      /* tokens per rank                  (>= 0)              */
    int64_t hidden; /* model width                      (>= 256, % 256 == 0) */
    int64_t inter;  /* expert intermediate size         (>= 128, % 128 == 0) */
    int64_t E;      /* experts over all ranks           (>= 1, E % P == 0)   */
    int64_t k;      /* experts per token                (1 .. E)            */
} moe_shape;

enum { MOE_EXPERT_WAVE = 0, MOE_INTERLEAVED = 1 };

/* Most local experts per wave (the launches carry a wave's experts inline). */
#define MOE_MAX_WAVE 32

/*
 * This rank's receive layout (host only; the dispatch exchange's bookkeeping):
 * from topk_idx [P][T][k] (global expert ids; rank r holds experts
 * r*E/P .. r*E/P + E/P - 1) it writes expert_offsets [E/P + 1] and the slots
 * of the rows routed here, row_slot [N], grouped by local expert and, within
 * an expert, in increasing slot order.  N = expert_offsets[E/P] must not
 * exceed `capacity` (UA_ERR_SHAPE otherwise; P*T*k always suffices).  An
 * expert id outside [0, E) gives UA_ERR_SHAPE.
 */
int moe_recv_layout(const int32_t *topk_idx, int rank, int P, const moe_shape *shp,
                    int64_t *expert_offsets, int32_t *row_slot, int64_t capacity);

/*
 * The fused path: Linear-1 with the gated activation into `act`, then
 * Linear-2 with the Combine in its epilogue (each row's topk_w times its
 * expert output, rounded to bf16, stored into its slot of `combine`), under
 * `schedule` (MOE_EXPERT_WAVE or MOE_INTERLEAVED) with `experts_per_wave`
 * local experts per wave (1 .. MOE_MAX_WAVE).  Both schedules compute every
 * tile with the same arithmetic: their outputs are bit-identical.
 * expert_offsets is a HOST array [E/P + 1] (0 = offsets[0] <= ... <=
 * offsets[E/P] = N); row_slot, topk_w, x, W1, W2, combine and act are device
 * pointers.  N == 0 is a valid empty call.
 */
int moe_experts_combine(const void *x, const int32_t *row_slot, const float *topk_w,
                        const int64_t *expert_offsets, const void *W1, const void *W2, int P,
                        const moe_shape *shp, void *combine, void *act, int schedule,
                        int experts_per_wave, hipStream_t stream);

/*
 * Workspace of the persistent form (below) for any call with this shape:
 * bytes of device memory, a multiple of 256 (0 for an invalid shape).
 */
size_t moe_workspace_bytes(int P, const moe_shape *shp);

/*
 * The fused path in its persistent form (the pages' MegaMoE runs the
 * schedule inside one persistent kernel; arXiv abstract page, Abstract;
 * pith.science review page, Fig. 4): the same tiles, arithmetic and outputs
 * as moe_experts_combine (bit-identical), run by one launch per 32 local
 * experts whose workgroups take the schedule's tiles in order from a device
 * queue; a Linear-2 tile starts once every Linear-1 tile of its token rows
 * has stored its act rows.  `workspace` (device, 16-byte aligned, at least
 * moe_workspace_bytes(P, shp) bytes, else UA_ERR_WORKSPACE; NULL gives
 * UA_ERR_NULL) holds the queue and the per-token-tile counts; the call
 * clears it on `stream` first, so it needs no initialisation, and calls
 * that share one workspace must not overlap.  Word 32 of the workspace
 * (as uint32) counts bounded waits that gave up (zero after every correct
 * call).  More
 * than 32 launches (more than 1024 local experts at 32 per wave) give
 * UA_ERR_UNSUPPORTED.
 */
int moe_experts_combine_ws(const void *x, const int32_t *row_slot, const float *topk_w,
                           const int64_t *expert_offsets, const void *W1, const void *W2, int P,
                           const moe_shape *shp, void *combine, void *act, int schedule,
                           int experts_per_wave, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Serial baseline, expert half: the same computation with Linear-2 writing
 * row i's weighted output to y_local [N][hidden] (row i of the receive
 * layout) instead of its Combine slot (Expert-Wave order).
 */
int moe_experts_local(const void *x, const int32_t *row_slot, const float *topk_w,
                      const int64_t *expert_offsets, const void *W1, const void *W2, int P,
                      const moe_shape *shp, void *y_local, void *act, int experts_per_wave,
                      hipStream_t stream);

/* moe_experts_local in the persistent form (Expert-Wave order; workspace as
 * for moe_experts_combine_ws). */
int moe_experts_local_ws(const void *x, const int32_t *row_slot, const float *topk_w,
                         const int64_t *expert_offsets, const void *W1, const void *W2, int P,
                         const moe_shape *shp, void *y_local, void *act, int experts_per_wave,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Serial baseline, exchange half: copies row i of y_local [N][hidden]
 * bit-for-bit into slot row_slot[i] of `combine` [P][T][k][hidden].
 * moe_experts_local followed by moe_combine_scatter writes exactly the bytes
 * moe_experts_combine writes.
 */
int moe_combine_scatter(const void *y_local, const int32_t *row_slot, int64_t N, int P,
                        const moe_shape *shp, void *combine, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_COMBINE_H */
