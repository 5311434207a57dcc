// Internal declarations shared by the libdpsync translation units.
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

// Batched fp32 GEMM on MFMA: for each batch b < nb,
// C_b[M,N] = op(A_b)[M,Kd] * B_b[Kd,N], row-major; op(A) = A ([M,Kd]) or, with
// trans_a, A^T where A_b is stored [Kd,M].
struct GemmF32Batch {
    const float *a[kMaxK];
    const float *b[kMaxK];
    float *c[kMaxK];
    int nb;
    long long M, N, Kd;
    int trans_a;
    // b_rows > 0 (trans_a == 0): B is the same for every entry and given as row
    // shards, row k in b_shard[k / b_rows] (b ignored); entries with b_copy[i]
    // set also receive a copy of B there (the gathered matrix). Shapes:
    // gemm_f32_fusable_gather().
    const float *b_shard[kMaxK];
    long long b_rows;
    float *b_copy[kMaxK];
};
hipError_t launch_gemm_f32(const GemmF32Batch &g, hipStream_t stream);
bool gemm_f32_fusable_gather(const GemmF32Batch &g, int n_shards);

// FSDP backward in one launch: dw_full[r] = x[r]^T . dy[r] ([d, f], fp32 MFMA,
// the same bits as launch_gemm_f32 with trans_a) and dw_shard[c] = the ring-order
// fp32 sum of rows c*R .. (c+1)*R - 1 of every dw_full (the same bits as the
// ReduceScatter kernel). Shapes: fsdp_bwd_fusable().
struct FsdpBwdParams {
    const float *x[kMaxK];      // [m, d]
    const float *dy[kMaxK];     // [m, f]
    float *dw_full[kMaxK];      // [d, f]
    float *dw_shard[kMaxK];     // [R, f]
    int k;
    long long m, d, f, R;
};
bool fsdp_bwd_fusable(int k, long long m, long long d, long long f);
hipError_t launch_fsdp_bwd_fused(const FsdpBwdParams &p, hipStream_t stream);

// The whole FSDP step in one launch for K <= 8: the forward dot with the
// AllGather folded in (a GemmF32Batch in shard mode, cut to 8 entries) beside
// the fused backward. n_fwd = the forward's tile count, tiles_x = its tiles per
// row. Shapes: gemm_f32_fusable_gather() and fsdp_bwd_fusable().
struct FsdpFwd8 {
    const float *a[8];
    const float *b[8];
    float *c[8];
    int nb;
    long long M, N, Kd;
    int trans_a;
    const float *b_shard[8];
    long long b_rows;
    float *b_copy[8];
};
struct FsdpBwd8 {
    const float *x[8];
    const float *dy[8];
    float *dw_full[8];
    float *dw_shard[8];
    int k;
    long long m, d, f, R;
};
struct FsdpStepParams {
    FsdpFwd8 fwd;
    FsdpBwd8 bwd;
    int n_fwd, tiles_x;
};
hipError_t launch_fsdp_step(const FsdpStepParams &p, hipStream_t stream);

// bf16 GEMM, C[M,N] = A[M,Kd] * B[N,Kd]^T, row-major, fp32 accumulation.
// GEMM variants: kGemmFast = the 4-wave kernel (every register of each SIMD)
// where the shape allows, else the 8-wave one; kGemmCoresident = the 8-wave
// kernel with depth-64 stages (224 VGPRs: a lean sync workgroup fits beside it
// on a CU); kGemmShareCU = the 8-wave kernel with depth-32 stages (198 VGPRs: a
// default sync workgroup fits beside it).
enum GemmVariant { kGemmFast = 0, kGemmCoresident = 1, kGemmShareCU = 2 };
hipError_t launch_gemm_bf16(const void *a, const void *b, void *c, long long M, long long N,
                            long long Kd, int variant, hipStream_t stream);

}  // namespace dps
