/*
 * ulysses_attn.h -- C ABI of the MI355X (gfx950) Ulysses-shard attention
 * library, libulysses_attn.so.
 *
 * The operation (X-Stage paper, arXiv 2607.23264):
 *   Fig. 5 of the pith.science review page, steps (a)-(c): after the
 *   pre-attention All-to-All, rank r of a P-rank Ulysses group holds the full
 *   sequence S for Hl = H/P heads.  Steps (d)-(e): attention runs on those
 *   heads and the post-attention All-to-All sends each output row back to the
 *   rank that owns its sequence chunk.  The abstract describes the fused form:
 *   the owner of an output tile stores it straight into the destination slot
 *   and resumes computing, with no wavefront or CU set aside for the exchange.
 *
 * Attention is non-causal softmax(Q K^T * scale) V per head, no mask, no
 * dropout, computed with bf16 inputs, fp32 accumulation and bf16 output
 * (round to nearest even).  Inputs are expected to be finite: an Inf or NaN
 * input gives unspecified values in the rows it reaches (never a fault).
 *
 * Layouts (bf16 = IEEE binary16-brain, passed as raw 16-bit patterns):
 *   Q, K, V, O_local : [B][S][Hl][d], contiguous, Hl = H / P.
 *   Xq, Xk, Xv, X (sequence-partitioned, before the pre-attention exchange):
 *       [B][P][S/P][H][d], contiguous: region p is source rank p's chunk of
 *       sequence rows [p*S/P, (p+1)*S/P) with all H heads; this rank's heads
 *       are g = rank*Hl .. rank*Hl+Hl-1.
 *   out (destination): [B][P][S/P][H][d], contiguous: P back-to-back regions,
 *       region p holding sequence rows [p*S/P, (p+1)*S/P) of all H heads.
 *       Row s of local head h_l lands in region p = s / (S/P), local row
 *       i = s mod (S/P), global head g = rank*Hl + h_l.
 *       (Because the regions are adjacent, this buffer is byte-identical to a
 *       [B][S][H][d] tensor: running every rank fills the full output.)
 *
 * Ownership: the caller allocates and frees every buffer (the *_ws calls'
 * workspace included); the library allocates nothing.  Between calls it
 * keeps only the device facts it queries once per device (compute units,
 * XCDs) and, for attn_ulysses_fused_noalloc, that call's fixed device
 * scratch (a static array, held until the process ends).  A call writes only
 * this rank's Hl head slots of `out` (every other slot keeps its bytes).
 * Output buffers must not overlap the inputs.
 *
 * The library must run on the process's one HIP runtime: a process that
 * also uses a copy of the runtime bundled elsewhere (a framework's own
 * libamdhip64) must load that copy before this library, so that it also
 * serves this library's dependency (the Python binding does so for torch).
 *
 * Pointers Q, K, V, out, O_local are DEVICE pointers on the current HIP
 * device, 16-byte aligned.  `stream` is a hipStream_t of that device
 * (NULL = its default stream).  Calls are asynchronous: they return after
 * the launch.  Launch shapes (and so ua_work_units, ua_key_split and the
 * workspace sizes) follow the current device's compute-unit and XCD counts,
 * queried once per device; on a host without a device they are computed for
 * the full MI355X (256 CUs in 8 XCDs).  For tuning, the environment variable
 * UA_TILE (read once per process) forces the launch shape, as query rows x
 * keys per tile: "256x64", "512x32" (d = 64 only), "128x64" or "128x32"
 * (an even number of 32-key tiles only); other values, or shapes it does
 * not fit, are ignored.  Results stay within the stated accuracy for any
 * shape, but their bits may differ between shapes.
 *
 * Errors: every call returns a status code and never prints or aborts.
 * Arguments are validated on the host before any device access, in this
 * order: shp NULL (UA_ERR_NULL); shape (UA_ERR_SHAPE); rank (UA_ERR_RANK);
 * head dim, scale and launch-size limits (UA_ERR_UNSUPPORTED); then an empty
 * call (B == 0 or S == 0) returns UA_OK without touching any pointer;
 * otherwise NULL buffers (UA_ERR_NULL) and alignment (UA_ERR_ALIGN).  A
 * launch failure reported by the runtime gives UA_ERR_HIP.  Size limits
 * (UA_ERR_UNSUPPORTED beyond them): B*S*Hl < 2^31 rows, B*S*Hl*d/8 < 2^32
 * 16-byte chunks, Hl*d <= 2^24 elements per sequence row (H*d <= 2^24 for
 * attn_ulysses_fused_io, which reads the sequence-partitioned rows in place).
 */
#ifndef ULYSSES_ATTN_H
#define ULYSSES_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t B; /* batch                                    (>= 0)          */
    int64_t S; /* full sequence length                     (>= 0, S % P == 0) */
    int64_t H; /* total heads of the Ulysses group         (>= 1, H % P == 0) */
    int64_t d; /* head dimension                           (64 or 128)     */
} ua_shape;

enum {
    UA_OK = 0,
    UA_ERR_NULL = -1,        /* a required pointer is NULL                    */
    UA_ERR_SHAPE = -2,       /* negative dims, H < 1, P < 1, S % P, H % P, overflow */
    UA_ERR_RANK = -3,        /* rank outside [0, P)                            */
    UA_ERR_ALIGN = -4,       /* a buffer pointer is not 16-byte aligned        */
    UA_ERR_UNSUPPORTED = -5, /* d not 64/128, scale not finite and > 0, too large */
    UA_ERR_HIP = -6,         /* the HIP runtime reported an error              */
    UA_ERR_WORKSPACE = -7,   /* workspace smaller than ua_workspace_bytes      */
    UA_ERR_SCRATCH = -8      /* split needs more than UA_SCRATCH_BYTES         */
};

/* Bytes of the fixed device scratch of attn_ulysses_fused_noalloc. */
#define UA_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * Fused path (abstract; Fig. 5 steps d-e; Fig. 7 piggybacked pipeline):
 * attention over this rank's Hl heads, each output tile stored by the
 * workgroup that computed it directly into its slot of `out`.
 *   scale: softmax scale (the usual choice is 1/sqrt(d)); finite and > 0.
 * B == 0 or S == 0 is a valid empty call (no launch, UA_OK).
 */
int attn_ulysses_fused(const void *Q, const void *K, const void *V, int rank, int P,
                       void *out, const ua_shape *shp, float scale, hipStream_t stream);

/*
 * Serial baseline, attention half ("FlashAttention alone" in the abstract):
 * the same attention kernel writing the head-partitioned O_local
 * [B][S][Hl][d].  rank and P are validated like the fused call and fix Hl.
 */
int attn_serial(const void *Q, const void *K, const void *V, int rank, int P,
                void *O_local, const ua_shape *shp, float scale, hipStream_t stream);

/*
 * Serial baseline, exchange half (the post-attention All-to-All of Fig. 5,
 * run after attention as a separate step): copies every row of O_local
 * [B][S][Hl][d] bit-for-bit into its slot of `out` [B][P][S/P][H][d].
 * attn_serial followed by a2a_permute writes exactly the bytes
 * attn_ulysses_fused writes.
 */
int a2a_permute(const void *O_local, int rank, int P, void *out,
                const ua_shape *shp, hipStream_t stream);

/*
 * The fused and serial calls with a workspace, for shapes whose query tiles
 * leave CUs idle: fewer tiles than the GPU has compute units (256 on an
 * MI355X; short sequences, few local heads), or a last round over the CUs
 * that few tiles fill.  The
 * computation is the same (Fig. 6 of the review page: each output tile has
 * one owner, which stores it into its destination slot, Fig. 7), except that
 * the keys of each query tile are split over ua_key_split workgroups: each
 * writes its partial softmax state (unnormalised O, running max, row sum;
 * fp32) to the workspace, and the last of them to finish merges the parts in
 * split order and stores the tile.  Outputs agree with the calls without a
 * workspace to rounding, not bit-for-bit; attn_serial_ws followed by
 * a2a_permute writes exactly the bytes attn_ulysses_fused_ws writes.
 *   workspace: device buffer of at least ua_workspace_bytes(shp, P) bytes,
 *     16-byte aligned, owned by the caller.  Its first
 *     ua_workspace_count_bytes(shp, P) bytes (4096 for every shape that
 *     splits) hold arrival counts that must be zero before the first call
 *     (allocate it zeroed); every call leaves them zero again.  The rest
 *     holds partial results.  So one workspace serves every shape whose
 *     ua_workspace_bytes does not exceed its size.  Calls that share a workspace must
 *     not run concurrently (use one stream, or one workspace per stream).
 *   When ua_workspace_bytes(shp, P) is 0 the shape needs no split: the
 *   workspace is not touched (it may be NULL) and the call is exactly the
 *   call without it.  Otherwise a NULL workspace gives UA_ERR_NULL, a
 *   misaligned one UA_ERR_ALIGN, and workspace_bytes below the requirement
 *   UA_ERR_WORKSPACE (checked after the other arguments).
 */
int attn_ulysses_fused_ws(const void *Q, const void *K, const void *V, int rank, int P,
                          void *out, const ua_shape *shp, float scale, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);
int attn_serial_ws(const void *Q, const void *K, const void *V, int rank, int P,
                   void *O_local, const ua_shape *shp, float scale, void *workspace,
                   size_t workspace_bytes, hipStream_t stream);
/* attn_ulysses_fused_io (below) with a workspace, as the two calls above:
 * bit-identical to a2a_gather of Xq, Xk, Xv followed by
 * attn_ulysses_fused_ws on the same workspace. */
int attn_ulysses_fused_io_ws(const void *Xq, const void *Xk, const void *Xv, int rank, int P,
                             void *out, const ua_shape *shp, float scale, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);
/*
 * attn_ulysses_fused_ws without a workspace argument and without allocating,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a fixed scratch array of UA_SCRATCH_BYTES (128 MiB) in device
 * memory that the library holds on every GPU it runs on until the process
 * ends; its address is looked up once per device, on the first call with
 * that device current.  Each call first clears the scratch's arrival counts
 * with a small kernel on `stream` (no memset), then runs exactly the launch
 * of attn_ulysses_fused_ws: the output is bit-identical to that call's.
 * Shapes that need no split run the plain launch and use no scratch.
 * A shape whose ua_workspace_bytes exceeds UA_SCRATCH_BYTES gives
 * UA_ERR_SCRATCH (checked after the other arguments, before any device
 * access).  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (different streams, or different host threads without
 * ordering) race and may produce wrong output; stream-ordered calls are safe.
 */
int attn_ulysses_fused_noalloc(const void *Q, const void *K, const void *V, int rank, int P,
                               void *out, const ua_shape *shp, float scale, hipStream_t stream);

/* Workspace bytes the *_ws calls need for this shape (0: no split, or an
 * invalid or empty shape). */
size_t ua_workspace_bytes(const ua_shape *shp, int P);
/* Leading bytes of that workspace holding the arrival counts: the part that
 * must be zero before a call (every call leaves it zero); 4096 for every
 * shape that splits, 0 when the shape needs no workspace. */
size_t ua_workspace_count_bytes(const ua_shape *shp, int P);
/* Workgroups sharing each query tile's keys in a *_ws call (1: no split; 0
 * for an invalid or empty shape).  For a stream-K split (below) the most
 * parts any query tile is cut into. */
int ua_key_split(const ua_shape *shp, int P);
/* The *_ws calls split a query tile's keys in one of two ways.  Either each
 * query tile's keys go to ua_key_split workgroups in equal runs, or, when
 * that leaves CUs idle in a last round, stream-K: one workgroup per CU, each
 * taking an equal run of ua_stream_k_iters consecutive (query tile, key tile)
 * iterations across query-tile boundaries, in one round; a query tile's keys
 * are then cut at the workgroup boundaries into at most ua_key_split parts.
 * Returns that run length for a stream-K split, else 0 (also for an invalid
 * or empty shape). */
int64_t ua_stream_k_iters(const ua_shape *shp, int P);

/*
 * Both exchanges fused.  Fig. 5 steps (a)-(c) of the review page: the
 * pre-attention All-to-All turns the sequence-partitioned projections into
 * head partitions; here, instead of a separate gather, the attention
 * kernel's Q load and K/V tile copies read this rank's heads straight from
 * the P source regions of Xq, Xk, Xv ([B][P][S/P][H][d]; the other heads'
 * bytes are never read).  The output side is attn_ulysses_fused's.  The
 * result is bit-identical to a2a_gather of Xq, Xk and Xv followed by
 * attn_ulysses_fused.  Validation as attn_ulysses_fused, plus H*d <= 2^24.
 */
int attn_ulysses_fused_io(const void *Xq, const void *Xk, const void *Xv, int rank, int P,
                          void *out, const ua_shape *shp, float scale, hipStream_t stream);
/*
 * Serial baseline of the pre-attention exchange (Fig. 5 steps a-c, run as a
 * separate step): copies this rank's Hl heads of every row of X
 * [B][P][S/P][H][d] bit-for-bit into X_local [B][S][Hl][d] (row s from
 * region s / (S/P), local row s mod (S/P)).  Validation as a2a_permute.
 */
int a2a_gather(const void *X, int rank, int P, void *X_local, const ua_shape *shp, hipStream_t stream);
/*
 * Measurement build of attn_ulysses_fused (the per-tile store spans the
 * pages time for the piggybacked epilogue; review page, Fig. 7): the same
 * arithmetic and bit-identical output, plus four uint64 per work unit in
 * trace[4*u + 0..3], u in [0, ua_work_units):
 *   [0] constant 100 MHz clock when the workgroup starts,
 *   [1] the same clock once every wave of it has its normalised rows
 *       (a workgroup barrier before the epilogue stores),
 *   [2] the same clock once every wave's epilogue stores have completed,
 *   [3] shader-clock cycles from [0] to [2] (so [3] / ([2]-[0]) * 100 MHz
 *       is the clock the workgroup ran at).
 * The two extra barriers make the measurement build slightly slower than the product
 * call.  trace: device buffer of ua_work_units(shp, P) * 4 uint64, 16-byte
 * aligned, owned by the caller; NULL gives UA_ERR_NULL (for a non-empty call).
 */
int attn_ulysses_fused_trace(const void *Q, const void *K, const void *V, int rank, int P,
                             void *out, const ua_shape *shp, float scale, hipStream_t stream,
                             uint64_t *trace);

/*
 * The measurement build of attn_ulysses_fused_ws: the same launch (the key
 * split or stream-K runs where the shape splits) and bit-identical output,
 * with one trace record per workgroup, trace[4*u + 0..3], u in
 * [0, ua_work_units_ws): [0] the 100 MHz clock at its start, [1] when its
 * waves last had normalised rows ready to store ([2] if it stored none: a
 * part of a split query tile that another workgroup merged), [2] once its
 * stores have completed, at its end, [3] shader-clock cycles from [0] to
 * [2].  So a split launch's clock is read on the launch itself.  Workspace
 * as attn_ulysses_fused_ws; trace as attn_ulysses_fused_trace.
 */
int attn_ulysses_fused_trace_ws(const void *Q, const void *K, const void *V, int rank, int P,
                                void *out, const ua_shape *shp, float scale, void *workspace,
                                size_t workspace_bytes, hipStream_t stream, uint64_t *trace);

/*
 * Write check of the fused path ("every destination element is written
 * exactly once"): attn_ulysses_fused_ws (the key split, stream-K, or the
 * plain call where the shape needs no workspace) that also adds 1 to
 * counts[c] for every 16-byte chunk c of `out` its epilogue stores (device
 * atomics; the stores themselves are the product call's, bit for bit).
 *   counts: device buffer of ua_dest_bytes(shp) / 16 uint32, 16-byte
 *     aligned, owned and zeroed by the caller; NULL gives UA_ERR_NULL.
 * After a call every chunk of this rank's head slots holds 1 and every other
 * chunk 0.  Other arguments and errors as attn_ulysses_fused_ws.
 */
int ua_fused_write_counts(const void *Q, const void *K, const void *V, int rank, int P,
                          void *out, const ua_shape *shp, float scale, void *workspace,
                          size_t workspace_bytes, hipStream_t stream, uint32_t *counts);

/*
 * Epilogue stores alone, for measuring what the destination layout sustains:
 * the fused call's grid, work-unit order and per-lane store pattern, writing
 * a closed-form value instead of attention output.  Element (s, global head
 * g, column c) of this rank's slots gets bf16 bits (7*s + 13*g + 3*c) & 0x3FFF;
 * every other slot keeps its bytes.  Validation as a2a_permute.
 */
int ua_epilogue_store_only(int rank, int P, void *out, const ua_shape *shp, hipStream_t stream);

/* Work units (workgroups) of the attention launch of the calls without a
 * workspace, and of attn_ulysses_fused_trace (its trace buffer holds 4 uint64
 * per unit); 0 for an invalid or empty shape.  A *_ws call that splits runs
 * ua_key_split workgroups per query tile of its own launch shape. */
int64_t ua_work_units(const ua_shape *shp, int P);

/* Workgroups of the launch of a *_ws call (the key split's or stream-K
 * runs when it splits, else ua_work_units), and so the records of
 * attn_ulysses_fused_trace_ws; 0 for an invalid or empty shape. */
int64_t ua_work_units_ws(const ua_shape *shp, int P);

/* Static English text for a status code; never NULL. */
const char *ua_status_string(int status);

/* Bytes of the destination buffer, B*S*H*d*2 (0 if shp is NULL or invalid). */
size_t ua_dest_bytes(const ua_shape *shp);

/* Bytes of one rank's Q, K, V or O_local, B*S*(H/P)*d*2 (0 if invalid). */
size_t ua_local_bytes(const ua_shape *shp, int P);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int ua_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_ATTN_H */
