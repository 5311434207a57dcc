// bf16 GEMM on CDNA4 matrix cores: C[M,N] = A[M,Kd] . B[N,Kd]^T, fp32
// accumulation, bf16 result (round to nearest even). This is the compute
// kernel of a (GEMM, collective) pair run concurrently with the sync kernels
// ("Optimizing ML Concurrent Computation and Communication with GPU DMA
// Engines", section "Problem Formulation": a GEMM and a collective with no data
// dependence between them).
//
// Both operands are k-contiguous (the linear-layer weight layout), so each
// lane's MFMA operand is one 16-byte run of 8 bf16 values in LDS.
// Workgroup: 256 threads = 2x2 waves, 128x128 tile of C, depth-32 k steps
// staged through LDS with the next step's global loads issued before the
// current step's MFMAs. Each wave owns 64x64 = 2x2 blocks of
// v_mfma_f32_32x32x16_bf16.
//
// MFMA 32x32x16 bf16 operand layout (lane l):
//   A operand: A[i = l % 32][k = 8*(l/32) + 0..7]
//   B operand: B[k = 8*(l/32) + 0..7][j = l % 32]
//   D register r: D[i = 8*(r/4) + 4*(l/32) + r%4][j = l % 32]
#include "dps_internal.h"

namespace dps {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 128, TN = 128, TK = 32, LDK = TK + 8;

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f)
{
    unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

__global__ __launch_bounds__(256) void gemm_bf16_kernel(const unsigned short *__restrict__ A,
                                                        const unsigned short *__restrict__ B,
                                                        unsigned short *__restrict__ C, long long M,
                                                        long long N, long long Kd)
{
    __shared__ __attribute__((aligned(16))) unsigned short As[TM][LDK];
    __shared__ __attribute__((aligned(16))) unsigned short Bs[TN][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wi = wave >> 1, wj = wave & 1;
    const long long m0 = (long long)blockIdx.y * TM, n0 = (long long)blockIdx.x * TN;

    // global -> register staging: two 16-byte chunks of A and of B per thread
    const int lr = tid >> 2, lk = (tid & 3) * 8;
    u32x4 ra[2], rb[2];
    auto gload = [&](long long k0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const long long gi = m0 + lr + 64 * h, gj = n0 + lr + 64 * h, gk = k0 + lk;
            const bool kin = gk + 8 <= Kd;
            ra[h] = (gi < M && kin) ? *reinterpret_cast<const u32x4 *>(A + gi * Kd + gk) : u32x4{0, 0, 0, 0};
            rb[h] = (gj < N && kin) ? *reinterpret_cast<const u32x4 *>(B + gj * Kd + gk) : u32x4{0, 0, 0, 0};
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<u32x4 *>(&As[lr + 64 * h][lk]) = ra[h];
            *reinterpret_cast<u32x4 *>(&Bs[lr + 64 * h][lk]) = rb[h];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    gload(0);
    sstore();
    __syncthreads();
    for (long long k0 = 0; k0 < Kd; k0 += TK) {
        const bool more = k0 + TK < Kd;
        if (more) gload(k0 + TK);
#pragma unroll
        for (int ks = 0; ks < TK / 16; ++ks) {
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                av[t] = *reinterpret_cast<const bf16x8 *>(&As[wi * 64 + t * 32 + (lane & 31)][ks * 16 + 8 * (lane >> 5)]);
                bv[t] = *reinterpret_cast<const bf16x8 *>(&Bs[wj * 64 + t * 32 + (lane & 31)][ks * 16 + 8 * (lane >> 5)]);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            sstore();
            __syncthreads();
        }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const long long gi = m0 + wi * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const long long gj = n0 + wj * 64 + b * 32 + (lane & 31);
                if (gi < M && gj < N) C[gi * N + gj] = f32_to_bf16_rne(acc[a][b][r]);
            }
}

}  // namespace

hipError_t launch_gemm_bf16(const void *a, const void *b, void *c, long long M, long long N,
                            long long Kd, hipStream_t st)
{
    const long long gx = (N + TN - 1) / TN, gy = (M + TM - 1) / TM;
    if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st,
                       (const unsigned short *)a, (const unsigned short *)b, (unsigned short *)c,
                       M, N, Kd);
    return hipGetLastError();
}

}  // namespace dps
