// Internal declarations of the sync kernels (ReduceScatter, AllGather,
// AllReduce and the fused ReduceScatter+AllGather launch), shared by
// sync_kernels.hip and the host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dps {

constexpr int kMaxK = 64;          // must equal DP_MAX_K in include/dpsync.h
constexpr int kBlock = 256;        // threads per workgroup of the sync kernels

enum Dtype { kF32 = 0, kBF16 = 1, kI32 = 2 };

// Reduction epilogues. kMul multiplies by an exactly representable 1/K (K a
// power of two), which gives the same correctly rounded result as dividing.
enum Epilogue { kSum = 0, kMul = 1, kDiv = 2, kWeighted = 3 };

inline int elem_size(int dt) { return dt == kBF16 ? 2 : 4; }

// ReduceScatter kernel arguments. Shard c's fold reads element (c*L + j) of
// every rank and writes element j of dst[c].
struct RsParams {
    const char *src[kMaxK];     // rank r input, element 0
    char *dst[kMaxK];           // shard c output, element 0 of the shard
    float w[kMaxK];             // per-rank weights f32(t_r) (kWeighted)
    // shard c: bit 8 set when all inputs and the output share one address phase
    // modulo 16 bytes; bits 0-7 hold the alignment anchor's address modulo 256
    // at shard element 0. 32-bit words so the kernel reads them with scalar
    // loads.
    int meta[kMaxK];
    float scale;                // 1/K (kMul), K (kDiv), sum of tokens (kWeighted)
    int write_pads;             // write zero into elements n_c..L-1 of every shard
    long long n, L;             // elements per rank, shard length
    long long sub;              // elements per sub-chunk, ceil(L/S)
    long long tiles_per_seg;    // tiles per (sub-chunk, shard) segment
    long long total_tiles;      // S * K * tiles_per_seg
    int max_blocks;             // persistent grid size (0: library default)
    int k, S;
    // set by the caller when an AllGather reads the shards next: then shard
    // sets small enough to stay in the caches are stored with ordinary
    // (cached) stores (the planner clears it for larger sets; capped-grid and
    // lean launches store nontemporally)
    int cache_out;
};

// AllGather kernel arguments. Shard c's valid elements go to element c*L + j
// of every rank's output.
struct AgParams {
    const char *src[kMaxK];     // shard c, element 0
    char *dst[kMaxK];           // rank r output, element 0
    int meta[kMaxK];            // as RsParams::meta, for shard c and the K outputs
    int skip_own;               // do not copy shard c to rank c (already in place)
    long long n, L, sub, tiles_per_seg, total_tiles;
    int max_blocks;
    int k, S;
};

// Fill the phase table and tiling of the parameter blocks; returns the grid size.
// The kernels are persistent: each workgroup walks tiles blockIdx.x,
// blockIdx.x + gridDim.x, ... of the flat (sub-chunk, shard, tile) space.
// lean: the variant with one vector per lane per rank and at most 64 VGPRs
// (same results), which fits beside a register-heavy kernel on one CU.
long long plan_rs(RsParams &p, int dt, bool lean = false);
long long plan_ag(AgParams &p, int dt);

hipError_t launch_rs(const RsParams &p, int dt, int ep, hipStream_t stream, bool lean = false);
// Fused AllReduce: RsParams with dst[r] = rank r's n-element output; every
// shard's fold goes straight to all K outputs (no shard buffer, no pads).
long long plan_ar(RsParams &p, int dt, bool lean = false);
hipError_t launch_ar(const RsParams &p, int dt, int ep, hipStream_t stream, bool lean = false);
hipError_t launch_ag(const AgParams &p, int dt, hipStream_t stream);
// A ReduceScatter (rp, epilogue ep) and an AllGather (ap) of disjoint buffer
// sets in one launch, one tile per workgroup, the two kinds interleaved.
hipError_t launch_rsag(const RsParams &rp, const AgParams &ap, int dt, int ep, hipStream_t stream);

}  // namespace dps
