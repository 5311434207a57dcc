// Batched fp32 GEMM on CDNA4 matrix cores, for the local dots of the FSDP
// layer step ("Sharding and Parallelism", "Real HLO before and after
// partitioning": after the weight AllGather each rank runs its local dot
// x_local[128,512] . w[512,512]; "FSDP and ZeRO": the backward pass produces the
// weight gradient that is then reduce-scattered).
//
// One workgroup (4 waves) computes a 64x64 tile of C for one batch entry
// (blockIdx.z = rank). Each wave owns a 32x32 quadrant and accumulates it with
// v_mfma_f32_32x32x2f32 over k in steps of 2; A and B tiles of depth 16 are
// staged through LDS, A stored k-major so each MFMA operand read is one
// contiguous 32-float row segment per half-wave.
//
// MFMA 32x32x2 f32 operand layout (lane l of the wave):
//   A operand: A[i = l % 32][k = l / 32]      B operand: B[k = l / 32][j = l % 32]
//   D register r: D[i = 8*(r/4) + 4*(l/32) + r%4][j = l % 32]
#include "dps_internal.h"

namespace dps {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 64, BN = 64, BK = 16;

template <int TA>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmF32Batch g)
{
    const int bz = blockIdx.z;
    const float *__restrict__ A = g.a[bz];
    const float *__restrict__ B = g.b[bz];
    float *__restrict__ C = g.c[bz];
    const long long M = g.M, N = g.N, Kd = g.Kd;
    const long long m0 = (long long)blockIdx.y * BM, n0 = (long long)blockIdx.x * BN;

    __shared__ float As[BK][BM + 4];   // As[k][i]
    __shared__ float Bs[BK][BN + 4];   // Bs[k][j]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wi = wave >> 1, wj = wave & 1;
    f32x16 acc = {};

    for (long long k0 = 0; k0 < Kd; k0 += BK) {
        if (TA == 0) {
            // A stored [M][Kd]: thread -> row tid/4, 4 consecutive k
            const int i = tid >> 2, kq = (tid & 3) * 4;
            const long long gi = m0 + i;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const long long gk = k0 + kq + e;
                As[kq + e][i] = (gi < M && gk < Kd) ? A[gi * Kd + gk] : 0.0f;
            }
        } else {
            // A stored [Kd][M]: thread -> k row tid/16, 4 consecutive i
            const int kr = tid >> 4, iq = (tid & 15) * 4;
            const long long gk = k0 + kr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const long long gi = m0 + iq + e;
                As[kr][iq + e] = (gk < Kd && gi < M) ? A[gk * M + gi] : 0.0f;
            }
        }
        {
            const int kr = tid >> 4, jq = (tid & 15) * 4;
            const long long gk = k0 + kr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const long long gj = n0 + jq + e;
                Bs[kr][jq + e] = (gk < Kd && gj < N) ? B[gk * N + gj] : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            const float a = As[kk + (lane >> 5)][wi * 32 + (lane & 31)];
            const float b = Bs[kk + (lane >> 5)][wj * 32 + (lane & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const long long gi = m0 + wi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const long long gj = n0 + wj * 32 + (lane & 31);
        if (gi < M && gj < N) C[gi * N + gj] = acc[r];
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmF32Batch &g, hipStream_t st)
{
    if (g.nb <= 0 || g.M <= 0 || g.N <= 0) return hipSuccess;
    const long long gx = (g.N + BN - 1) / BN, gy = (g.M + BM - 1) / BM;
    if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)g.nb);
    if (g.trans_a)
        hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, dim3(256), 0, st, g);
    else
        hipLaunchKernelGGL(gemm_f32_kernel<0>, grid, dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace dps
