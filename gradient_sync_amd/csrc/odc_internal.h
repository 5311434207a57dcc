// Internal declarations of the on-demand-communication kernels (push and
// settle) shared by odc_kernels.hip and the entry points.
#pragma once

#include "dps_internal.h"

namespace dps {

// Scatter-accumulate of np pushes, each an n-element gradient of one rank,
// into the K owners' fp32 accumulators, applied in push order:
// acc[c][j] += f32(g_i[c*L + j]) for i = 0..np-1, j < n_c.
struct SaParams {
    const char *g[kMaxK];       // push i's gradient, element 0
    float *acc[kMaxK];          // owner c's accumulator, element 0 of its shard
    int aligned[kMaxK];         // set by the launcher: shard c takes the vector path
    long long n, L, tiles_per_shard;
    int np, k;
};
hipError_t launch_scatter_accumulate(const SaParams &p, int dt, hipStream_t stream);

// Settle: out[c][j] = cast(acc[c][j] / divisor) for j < n_c, zero for
// n_c <= j < L; with reset, acc[c][j] = 0 afterwards. mul: scale holds the exact
// reciprocal of a power-of-two divisor, else the divisor itself.
struct SettleParams {
    float *acc[kMaxK];
    char *out[kMaxK];
    int aligned[kMaxK];         // set by the launcher
    float scale;
    int reset;
    long long n, L, tiles_per_shard;
    int k;
};
hipError_t launch_settle(const SettleParams &p, int dt, bool mul, hipStream_t stream);

}  // namespace dps
