// Internal declarations shared by the libdpsync translation units.
#pragma once

#include "sync_internal.h"

namespace dps {

// Batched fp32 GEMM on MFMA: for each batch b < nb,
// C_b[M,N] = op(A_b)[M,Kd] * op(B_b)[Kd,N], row-major; op(A) = A ([M,Kd]) or,
// with trans_a, A^T where A_b is stored [Kd,M]; op(B) = B ([Kd,N]) or, with
// trans_b, B^T where B_b is stored [N,Kd] (not both transposed).
struct GemmF32Batch {
    const float *a[kMaxK];
    const float *b[kMaxK];
    float *c[kMaxK];
    int nb;
    long long M, N, Kd;
    int trans_a;
    // b_rows > 0 (trans_a == 0): the stored B is the same for every entry and
    // given as row shards, row k in b_shard[k / b_rows] (b ignored); without
    // trans_b, entries with b_copy[i] set also receive a copy of B there (the
    // gathered matrix). Shapes: gemm_f32_fusable_gather().
    const float *b_shard[kMaxK];
    long long b_rows;
    float *b_copy[kMaxK];
    int trans_b;
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
    int trans_b;
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
    FsdpFwd8 fwd;       // y = x . W, W's rows from the shards, gathered copy written
    FsdpFwd8 dx;        // dx = dy . W^T, W's rows from the shards (n_dx = 0: none)
    FsdpBwd8 bwd;
    int n_fwd, tiles_x;
    int n_dx, tiles_x_dx;
};
hipError_t launch_fsdp_step(const FsdpStepParams &p, hipStream_t stream);
// the step kernel's forward blocks (32x32, x block in LDS, W from the shards):
// fwd.M, fwd.N multiples of 32, fwd.Kd 256 or 512, shards
// of a multiple of 32 rows
bool fsdp_fwd_direct_ok(const FsdpFwd8 &p);
// The step without dx as one wave of workgroups, each wave running a forward
// chain and a backward chain (fsdp_step2_kernel): the backward blocks'
// shapes, f a multiple of 64, d a multiple of 128 and at most 512. p.n_fwd =
// (k*m/32)*(f/64), p.n_dx = 0.
bool fsdp_step2_ok(int k, long long m, long long d, long long f);
// The fixture sizes (K = 8, m = 128, d = f = 512) with 16-byte aligned
// shards and outputs: the step as a compile-time-sized kernel, with dx = dy . W^T
// as well when p.n_dx != 0 (launch_fsdp_step2 then takes it).
bool fsdp_step_k8_ok(const FsdpStepParams &p);
hipError_t launch_fsdp_step2(const FsdpStepParams &p, hipStream_t stream);

// bf16 GEMM, row-major, fp32 accumulation: C[M,N] = A[M,Kd] * B[Kd,N] with
// b_kn, else C = A[M,Kd] * B[N,Kd]^T. Any element-aligned pointers and shapes;
// rows that are not 16-byte aligned take a slower kernel (same bits).
// GEMM variants: kGemmFast = the 4-wave kernel (every register of each SIMD)
// where the shape allows, else the 8-wave one; kGemmCoresident = the 8-wave
// kernel with depth-64 stages (224 VGPRs: a lean sync workgroup fits beside it
// on a CU); kGemmShareCU = the 8-wave kernel with depth-32 stages (198 VGPRs: a
// default sync workgroup fits beside it).
enum GemmVariant { kGemmFast = 0, kGemmCoresident = 1, kGemmShareCU = 2 };
hipError_t launch_gemm_bf16(const void *a, const void *b, void *c, long long M, long long N,
                            long long Kd, int variant, bool b_kn, hipStream_t stream);

}  // namespace dps
