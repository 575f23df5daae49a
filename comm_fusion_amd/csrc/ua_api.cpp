// ua_api.cpp -- C ABI of libulysses_attn.so (declared in include/ulysses_attn.h).
//
// Host-side only: argument validation (no device access, so it runs on a
// host without a GPU), placement set-up for the two epilogues, and launches.
// The library allocates nothing and keeps no state between calls (the *_ws
// calls use the workspace their caller passes in; attn_ulysses_fused_noalloc
// uses the library's fixed device scratch).

#include "ulysses_attn.h"

#include <math.h>
#include <stdint.h>

#include "ua_internal.h"

namespace {

constexpr int kVersion = 1 * 10000 + 2 * 100 + 0;

bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape-level checks shared by every entry point.  On success *elems holds
// B*S*H*d (the destination element count).
int check_shape(const ua_shape *shp, int rank, int P, int64_t *elems)
{
    if (!shp) return UA_ERR_NULL;
    const int64_t B = shp->B, S = shp->S, H = shp->H, d = shp->d;
    if (B < 0 || S < 0 || H < 1 || d < 1 || P < 1) return UA_ERR_SHAPE;
    if (H % P != 0 || S % P != 0) return UA_ERR_SHAPE;
    int64_t n = 0;
    if (!mul_ok(B, S, &n) || !mul_ok(n, H, &n) || !mul_ok(n, d, &n) || n > INT64_MAX / 2)
        return UA_ERR_SHAPE;
    if (rank < 0 || rank >= P) return UA_ERR_RANK;
    if (d != 64 && d != 128) return UA_ERR_UNSUPPORTED;
    *elems = n;
    return UA_OK;
}

// Size limits of the launch grids: work units and copied 16-byte chunks are
// counted in 32-bit integers.
int check_limits(const ua_shape *shp, int P)
{
    const int64_t Hl = shp->H / P;
    const int64_t rows = shp->B * shp->S * Hl;
    if (rows >= (int64_t)1 << 31) return UA_ERR_UNSUPPORTED;
    // row stride Hl*d: a 64-row K/V tile must span fewer than 2^31 bytes
    if (Hl * shp->d > (int64_t)1 << 24) return UA_ERR_UNSUPPORTED;
    if (rows * (shp->d / 8) > (int64_t)UINT32_MAX) return UA_ERR_UNSUPPORTED;
    if (ua::attention_units(shp->B, shp->S, Hl, (int)shp->d) > INT32_MAX) return UA_ERR_UNSUPPORTED;
    return UA_OK;
}

// The sequence-partitioned input [B][P][S/P][H][d] is read in place with a
// row stride of H*d elements: a 64-row K/V tile must span fewer than 2^31 bytes.
int check_limits_seq(const ua_shape *shp)
{
    if (shp->H * shp->d > (int64_t)1 << 24) return UA_ERR_UNSUPPORTED;
    return UA_OK;
}

bool empty(const ua_shape *shp) { return shp->B == 0 || shp->S == 0; }

ua::Placement dest_placement(void *out, const ua_shape *shp, int rank, int P)
{
    ua::Placement o;
    o.base = (uint16_t *)out;
    o.regions = P;
    o.region_rows = shp->S / P;
    o.heads = shp->H;
    o.head0 = (int64_t)rank * (shp->H / P);
    return o;
}

ua::Placement local_placement(void *o_local, const ua_shape *shp, int P)
{
    ua::Placement o;
    o.base = (uint16_t *)o_local;
    o.regions = 1;
    o.region_rows = shp->S;
    o.heads = shp->H / P;
    o.head0 = 0;
    return o;
}

// seq_input: Q, K, V are the sequence-partitioned [B][P][S/P][H][d] inputs
// of the pre-attention exchange (read in place), else [B][S][Hl][d].
// want_ws: a *_ws call, whose workspace (ws_bytes bytes) lets the launch
// split the keys of each query tile over several workgroups.
int attention_call(const void *Q, const void *K, const void *V, int rank, int P, void *out,
                   const ua_shape *shp, float scale, hipStream_t stream, bool fused, uint64_t *trace = nullptr,
                   bool want_trace = false, bool seq_input = false, bool want_ws = false,
                   void *ws = nullptr, size_t ws_bytes = 0, uint32_t *wcount = nullptr, bool want_count = false)
{
    int64_t elems = 0;
    int st = check_shape(shp, rank, P, &elems);
    if (st != UA_OK) return st;
    if (!isfinite(scale) || !(scale > 0.0f)) return UA_ERR_UNSUPPORTED;
    if ((st = check_limits(shp, P)) != UA_OK) return st;
    if (seq_input && (st = check_limits_seq(shp)) != UA_OK) return st;
    if (empty(shp)) return UA_OK;
    if (!Q || !K || !V || !out || (want_trace && !trace) || (want_count && !wcount)) return UA_ERR_NULL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || (want_trace && !aligned16(trace)) ||
        (want_count && !aligned16(wcount)))
        return UA_ERR_ALIGN;
    const int64_t Hl = shp->H / P;
    const int64_t need = want_ws ? ua::workspace_bytes(shp->B, shp->S, Hl, (int)shp->d) : 0;
    if (need > 0) {
        if (!ws) return UA_ERR_NULL;
        if (!aligned16(ws)) return UA_ERR_ALIGN;
        if (ws_bytes < (size_t)need) return UA_ERR_WORKSPACE;
    }
    const ua::Placement o = fused ? dest_placement(out, shp, rank, P) : local_placement(out, shp, P);
    const int64_t in_heads = seq_input ? shp->H : Hl;
    const int64_t in_head0 = seq_input ? (int64_t)rank * Hl : 0;
    const hipError_t e = ua::launch_attention((const uint16_t *)Q, (const uint16_t *)K,
                                              (const uint16_t *)V, in_heads, in_head0, shp->B, shp->S,
                                              Hl, (int)shp->d, scale, o, (hipStream_t)stream, trace,
                                              need > 0 ? ws : nullptr, (unsigned *)wcount);
    return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_ulysses_fused(const void *Q, const void *K, const void *V, int rank, int P, void *out,
                       const ua_shape *shp, float scale, hipStream_t stream)
{
    return attention_call(Q, K, V, rank, P, out, shp, scale, stream, true);
}

int attn_serial(const void *Q, const void *K, const void *V, int rank, int P, void *O_local,
                const ua_shape *shp, float scale, hipStream_t stream)
{
    return attention_call(Q, K, V, rank, P, O_local, shp, scale, stream, false);
}

int attn_ulysses_fused_ws(const void *Q, const void *K, const void *V, int rank, int P, void *out,
                          const ua_shape *shp, float scale, void *workspace, size_t workspace_bytes,
                          hipStream_t stream)
{
    return attention_call(Q, K, V, rank, P, out, shp, scale, stream, true, nullptr, false, false, true,
                          workspace, workspace_bytes);
}

int attn_serial_ws(const void *Q, const void *K, const void *V, int rank, int P, void *O_local,
                   const ua_shape *shp, float scale, void *workspace, size_t workspace_bytes,
                   hipStream_t stream)
{
    return attention_call(Q, K, V, rank, P, O_local, shp, scale, stream, false, nullptr, false, false, true,
                          workspace, workspace_bytes);
}

int attn_ulysses_fused_noalloc(const void *Q, const void *K, const void *V, int rank, int P, void *out,
                               const ua_shape *shp, float scale, hipStream_t stream)
{
    int64_t elems = 0;
    int st = check_shape(shp, rank, P, &elems);
    if (st != UA_OK) return st;
    if (!isfinite(scale) || !(scale > 0.0f)) return UA_ERR_UNSUPPORTED;
    if ((st = check_limits(shp, P)) != UA_OK) return st;
    if (empty(shp)) return UA_OK;
    if (!Q || !K || !V || !out) return UA_ERR_NULL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out)) return UA_ERR_ALIGN;
    const int64_t Hl = shp->H / P;
    if (ua::workspace_bytes(shp->B, shp->S, Hl, (int)shp->d) > ua::kScratchBytes) return UA_ERR_SCRATCH;
    const hipError_t e = ua::launch_attention_scratch((const uint16_t *)Q, (const uint16_t *)K,
                                                      (const uint16_t *)V, shp->B, shp->S, Hl, (int)shp->d,
                                                      scale, dest_placement(out, shp, rank, P), stream);
    return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

int attn_ulysses_fused_io_ws(const void *Xq, const void *Xk, const void *Xv, int rank, int P, void *out,
                             const ua_shape *shp, float scale, void *workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    return attention_call(Xq, Xk, Xv, rank, P, out, shp, scale, stream, true, nullptr, false, true, true,
                          workspace, workspace_bytes);
}

size_t ua_workspace_bytes(const ua_shape *shp, int P)
{
    int64_t elems = 0;
    if (check_shape(shp, 0, P, &elems) != UA_OK || check_limits(shp, P) != UA_OK) return 0;
    if (empty(shp)) return 0;
    return (size_t)ua::workspace_bytes(shp->B, shp->S, shp->H / P, (int)shp->d);
}

size_t ua_workspace_count_bytes(const ua_shape *shp, int P)
{
    int64_t elems = 0;
    if (check_shape(shp, 0, P, &elems) != UA_OK || check_limits(shp, P) != UA_OK) return 0;
    if (empty(shp)) return 0;
    return (size_t)ua::workspace_count_bytes(shp->B, shp->S, shp->H / P, (int)shp->d);
}

int64_t ua_stream_k_iters(const ua_shape *shp, int P)
{
    int64_t elems = 0;
    if (check_shape(shp, 0, P, &elems) != UA_OK || check_limits(shp, P) != UA_OK) return 0;
    if (empty(shp)) return 0;
    return ua::stream_k_iters(shp->B, shp->S, shp->H / P, (int)shp->d);
}

int ua_key_split(const ua_shape *shp, int P)
{
    int64_t elems = 0;
    if (check_shape(shp, 0, P, &elems) != UA_OK || check_limits(shp, P) != UA_OK) return 0;
    if (empty(shp)) return 0;
    return ua::key_split(shp->B, shp->S, shp->H / P, (int)shp->d);
}

int attn_ulysses_fused_io(const void *Xq, const void *Xk, const void *Xv, int rank, int P, void *out,
                          const ua_shape *shp, float scale, hipStream_t stream)
{
    return attention_call(Xq, Xk, Xv, rank, P, out, shp, scale, stream, true, nullptr, false, true);
}

int a2a_gather(const void *X, int rank, int P, void *X_local, const ua_shape *shp, hipStream_t stream)
{
    int64_t elems = 0;
    int st = check_shape(shp, rank, P, &elems);
    if (st != UA_OK) return st;
    if ((st = check_limits(shp, P)) != UA_OK) return st;
    if (empty(shp)) return UA_OK;
    if (!X || !X_local) return UA_ERR_NULL;
    if (!aligned16(X) || !aligned16(X_local)) return UA_ERR_ALIGN;
    // the source is described like the exchange's destination; only read
    const ua::Placement in = dest_placement(const_cast<void *>(X), shp, rank, P);
    const hipError_t e = ua::launch_gather(in, shp->B, shp->S, shp->H / P, (int)shp->d,
                                           (uint16_t *)X_local, (hipStream_t)stream);
    return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

int ua_fused_write_counts(const void *Q, const void *K, const void *V, int rank, int P, void *out,
                          const ua_shape *shp, float scale, void *workspace, size_t workspace_bytes,
                          hipStream_t stream, uint32_t *counts)
{
    return attention_call(Q, K, V, rank, P, out, shp, scale, stream, true, nullptr, false, false, true, workspace,
                          workspace_bytes, counts, true);
}

int attn_ulysses_fused_trace(const void *Q, const void *K, const void *V, int rank, int P, void *out,
                             const ua_shape *shp, float scale, hipStream_t stream, uint64_t *trace)
{
    return attention_call(Q, K, V, rank, P, out, shp, scale, stream, true, trace, true);
}

int attn_ulysses_fused_trace_ws(const void *Q, const void *K, const void *V, int rank, int P, void *out,
                                const ua_shape *shp, float scale, void *workspace, size_t workspace_bytes,
                                hipStream_t stream, uint64_t *trace)
{
    return attention_call(Q, K, V, rank, P, out, shp, scale, stream, true, trace, true, false, true, workspace,
                          workspace_bytes);
}

int ua_epilogue_store_only(int rank, int P, void *out, const ua_shape *shp, hipStream_t stream)
{
    int64_t elems = 0;
    int st = check_shape(shp, rank, P, &elems);
    if (st != UA_OK) return st;
    if ((st = check_limits(shp, P)) != UA_OK) return st;
    if (empty(shp)) return UA_OK;
    if (!out) return UA_ERR_NULL;
    if (!aligned16(out)) return UA_ERR_ALIGN;
    const hipError_t e = ua::launch_epilogue_only(shp->B, shp->S, shp->H / P, (int)shp->d,
                                                  dest_placement(out, shp, rank, P), (hipStream_t)stream);
    return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

int64_t ua_work_units(const ua_shape *shp, int P)
{
    int64_t elems = 0;
    if (check_shape(shp, 0, P, &elems) != UA_OK || check_limits(shp, P) != UA_OK) return 0;
    if (empty(shp)) return 0;
    return ua::attention_units(shp->B, shp->S, shp->H / P, (int)shp->d);
}

int64_t ua_work_units_ws(const ua_shape *shp, int P)
{
    int64_t elems = 0;
    if (check_shape(shp, 0, P, &elems) != UA_OK || check_limits(shp, P) != UA_OK) return 0;
    if (empty(shp)) return 0;
    return ua::attention_units_ws(shp->B, shp->S, shp->H / P, (int)shp->d);
}

int a2a_permute(const void *O_local, int rank, int P, void *out, const ua_shape *shp, hipStream_t stream)
{
    int64_t elems = 0;
    int st = check_shape(shp, rank, P, &elems);
    if (st != UA_OK) return st;
    if ((st = check_limits(shp, P)) != UA_OK) return st;
    if (empty(shp)) return UA_OK;
    if (!O_local || !out) return UA_ERR_NULL;
    if (!aligned16(O_local) || !aligned16(out)) return UA_ERR_ALIGN;
    const hipError_t e = ua::launch_permute((const uint16_t *)O_local, shp->B, shp->S, shp->H / P,
                                            (int)shp->d, dest_placement(out, shp, rank, P),
                                            (hipStream_t)stream);
    return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

const char *ua_status_string(int status)
{
    switch (status) {
    case UA_OK: return "ok";
    case UA_ERR_NULL: return "a required pointer is NULL";
    case UA_ERR_SHAPE: return "invalid shape (negative dims, H or P < 1, S or H not divisible by P, or size overflow)";
    case UA_ERR_RANK: return "rank outside [0, P)";
    case UA_ERR_ALIGN: return "a buffer pointer is not 16-byte aligned";
    case UA_ERR_UNSUPPORTED: return "unsupported (d not 64/128, scale not finite and > 0, or shape beyond launch limits)";
    case UA_ERR_HIP: return "the HIP runtime reported an error";
    case UA_ERR_WORKSPACE: return "workspace smaller than ua_workspace_bytes";
    case UA_ERR_SCRATCH: return "the shape's key split needs more than the library's fixed device scratch (UA_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

size_t ua_dest_bytes(const ua_shape *shp)
{
    if (!shp || shp->B < 0 || shp->S < 0 || shp->H < 1 || shp->d < 1) return 0;
    int64_t e = 0;
    if (!mul_ok(shp->B, shp->S, &e) || !mul_ok(e, shp->H, &e) || !mul_ok(e, shp->d, &e) ||
        e > INT64_MAX / 2)
        return 0;
    return (size_t)e * 2;
}

size_t ua_local_bytes(const ua_shape *shp, int P)
{
    if (!shp || P < 1 || shp->B < 0 || shp->S < 0 || shp->H < 1 || shp->d < 1 || shp->H % P != 0)
        return 0;
    int64_t e = 0;
    if (!mul_ok(shp->B, shp->S, &e) || !mul_ok(e, shp->H / P, &e) || !mul_ok(e, shp->d, &e) ||
        e > INT64_MAX / 2)
        return 0;
    return (size_t)e * 2;
}

int ua_version(void) { return kVersion; }

}  // extern "C"
