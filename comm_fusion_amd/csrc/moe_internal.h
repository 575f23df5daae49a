// moe_internal.h -- launch interface between the MoE C-ABI layer
// (moe_api.cpp) and its gfx950 kernels (moe_kernels.hip).  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxWave = 32;      // local experts per wave (MOE_MAX_WAVE)
constexpr int kInterleaved = 1;   // MOE_INTERLEAVED

// One call's operands (device pointers except `offsets`, a host array of
// E_l + 1 receive-row offsets, one expert's rows after another).
struct Problem {
    const uint16_t *x;         // [P][T][hidden]
    const int32_t *row_slot;   // [N]: (p*T + t)*k + j
    const float *topk_w;       // [P][T][k]
    const uint16_t *w1;        // [E_l][2*inter][hidden]
    const uint16_t *w2;        // [E_l][hidden][inter]
    uint16_t *act;             // [N][inter]
    uint16_t *out;             // Combine buffer [P][T][k][hidden], or y_local [N][hidden]
    const int64_t *offsets;    // host, [E_l + 1]
    int64_t E_l, hidden, inter, k;
};

// Linear-1 (+ activation) and Linear-2 (+ Combine, or local rows when
// `local`) of every local expert, in waves of per_wave experts under
// `schedule` (Expert-Wave, or interleaved; local output always runs
// Expert-Wave order).
hipError_t launch_moe(const Problem &p, int schedule, int per_wave, bool local, hipStream_t stream);

// The persistent form: the same tiles and arithmetic in one launch per
// kMaxWave experts, workgroups taking tiles in schedule order from a device
// queue, each Linear-2 tile waiting for its token tile's Linear-1 tiles.
// `ws` (device, 4-byte words): kWsHeader words of queue counters (one per
// launch) and the timeout count, then one word per token tile
// (token_tiles); the launch clears them first.
constexpr int kMaxLaunches = 32;  // launches of one call: one queue counter each
constexpr int kWsTimeouts = 32;   // header word counting bounded waits that gave up
constexpr int kWsHeader = 64;
int64_t token_tiles(const int64_t *offsets, int64_t E_l);
hipError_t launch_moe_persist(const Problem &p, int schedule, int per_wave, bool local, unsigned *ws,
                              hipStream_t stream);

// Bit copy of y_local rows into their Combine slots.
hipError_t launch_scatter(const uint16_t *y_local, const int32_t *row_slot, int64_t N, int64_t hidden,
                          uint16_t *combine, hipStream_t stream);

}  // namespace moe
