// ua_internal.h -- launch interface between the C-ABI layer (ua_api.cpp) and
// the gfx950 kernels (ua_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ua {

// Where attention output rows go.  One description serves both epilogues:
//   destination [B][P][S/P][H][d]: regions = P, region_rows = S/P,
//                                  heads = H, head0 = rank*Hl;
//   local       [B][S][Hl][d]:     regions = 1, region_rows = S,
//                                  heads = Hl, head0 = 0.
// Row s of local head h of batch b goes to region p = s / region_rows, row
// i = s - p*region_rows, head g = head0 + h, i.e. element offset
// (((b*regions + p)*region_rows + i)*heads + g)*d.
struct Placement {
    uint16_t *base;
    int64_t regions;
    int64_t region_rows;
    int64_t heads;
    int64_t head0;
};

// Attention over Hl local heads (bf16 bits).  Q, K, V are [B][S][in_heads][d]
// with this rank's heads at in_head0 .. in_head0+Hl-1: in_heads = Hl,
// in_head0 = 0 for the local layout [B][S][Hl][d]; in_heads = H,
// in_head0 = rank*Hl for the sequence-partitioned input [B][P][S/P][H][d].
// With a non-null trace, the measurement build runs and fills 4 uint64 per unit.
// With a non-null workspace (workspace_bytes of the shape, counts zero on
// entry and again on exit) and no trace, the launch splits each query tile's
// keys over key_split workgroups.  With a non-null wcount, the epilogue adds
// 1 to wcount[c] for every 16-byte chunk c (from out.base) it stores.
hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int64_t in_heads, int64_t in_head0, int64_t B, int64_t S, int64_t Hl,
                            int d, float scale, const Placement &out, hipStream_t stream,
                            uint64_t *trace = nullptr, void *workspace = nullptr, unsigned *wcount = nullptr);

// The attention kernel's epilogue stores alone (closed-form values).
hipError_t launch_epilogue_only(int64_t B, int64_t S, int64_t Hl, int d, const Placement &out,
                                hipStream_t stream);

// Bit copy of O_local [B][S][Hl][d] rows into `out`.
hipError_t launch_permute(const uint16_t *o_local, int64_t B, int64_t S, int64_t Hl, int d,
                          const Placement &out, hipStream_t stream);

// Bit copy of this rank's rows of a sequence-partitioned input (placed as
// `in` describes; base is only read) into x_local [B][S][Hl][d].
hipError_t launch_gather(const Placement &in, int64_t B, int64_t S, int64_t Hl, int d,
                         uint16_t *x_local, hipStream_t stream);

// Bytes of the fixed device scratch behind launch_attention_scratch.
constexpr int64_t kScratchBytes = (int64_t)128 << 20;

// launch_attention for the local-layout inputs with the key-split workspace
// in the library's fixed device scratch of the current device (no
// allocation; the caller checks workspace_bytes <= kScratchBytes).  Clears
// the scratch's arrival counts with a kernel on `stream` first.  Calls that
// overlap on one device race on the scratch.
hipError_t launch_attention_scratch(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t B,
                                    int64_t S, int64_t Hl, int d, float scale, const Placement &out,
                                    hipStream_t stream);

// XCDs of the current device (workgroups are dealt round robin over them);
// 8, the full MI355X, on a host without a device.
int device_xcd_count();

// Work units (one workgroup each) the attention launch uses for this shape
// without a key split (query tiles).
int64_t attention_units(int64_t B, int64_t S, int64_t Hl, int d);
// Workgroups of the launch given a workspace (the key split's, or the plain
// launch's when it does not split).
int64_t attention_units_ws(int64_t B, int64_t S, int64_t Hl, int d);

// Workgroups per query tile of a launch given a workspace (1: no split), and
// the workspace bytes that launch needs (0 when it does not split).
int key_split(int64_t B, int64_t S, int64_t Hl, int d);
// Iterations (query tile, key tile) per workgroup when that split is
// stream-K (one workgroup per CU); 0 otherwise.
int64_t stream_k_iters(int64_t B, int64_t S, int64_t Hl, int d);
int64_t workspace_bytes(int64_t B, int64_t S, int64_t Hl, int d);
// Leading bytes of that workspace that hold the arrival counts.
int64_t workspace_count_bytes(int64_t B, int64_t S, int64_t Hl, int d);

}  // namespace ua
