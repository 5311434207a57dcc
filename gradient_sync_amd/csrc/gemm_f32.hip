// Batched fp32 GEMM launches (the tile code is in gemm_f32_tile.h).
#include "gemm_f32_tile.h"

namespace dps {
namespace {

using namespace f32tile;

template <int TA, int NT, bool WHOLE, int FUSE>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(const GemmF32Batch g, const int tiles_x)
{
    __shared__ __attribute__((aligned(16))) float As[2][BK][LDP];   // As[buf][k][i]
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][LDP];   // Bs[buf][k][j]
    gemm_f32_tile<TA, NT, WHOLE, FUSE>(g, tiles_x, (int)blockIdx.x, As, Bs);
}

template <int TA, int NT>
void launch_f32(const GemmF32Batch &g, long long blocks, long long gx, bool whole, hipStream_t st)
{
    if constexpr (TA == 0 || TA == 2) {
        if (g.b_rows > 0) {
            hipLaunchKernelGGL((gemm_f32_kernel<TA, NT, true, TA == 0 ? 1 : 2>), dim3((unsigned)blocks), dim3(NT), 0, st, g, (int)gx);
            return;
        }
    }
    if (whole)
        hipLaunchKernelGGL((gemm_f32_kernel<TA, NT, true, 0>), dim3((unsigned)blocks), dim3(NT), 0, st, g, (int)gx);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<TA, NT, false, 0>), dim3((unsigned)blocks), dim3(NT), 0, st, g, (int)gx);
}

// whole tiles, whole stage groups and 16-byte aligned rows everywhere
bool f32_whole(const GemmF32Batch &g)
{
    bool whole = g.M % BM == 0 && g.N % BN == 0 && g.Kd % (BK * kDepth) == 0 &&
                 (g.trans_b ? g.Kd % 4 == 0 : g.N % 4 == 0) &&
                 (g.trans_a ? g.M % 4 == 0 : g.Kd % 4 == 0);
    for (int i = 0; i < g.nb && whole; ++i)
        whole = ((uintptr_t)g.a[i] & 15) == 0 && (g.b_rows > 0 || ((uintptr_t)g.b[i] & 15) == 0);
    return whole;
}

}  // namespace

bool gemm_f32_fusable_gather(const GemmF32Batch &g, int n_shards)
{
    if (g.trans_a || g.b_rows <= 0 || !f32_whole(g)) return false;
    // B's rows along k (each k stage in one shard), or B^T's rows along n (each
    // 64-row tile in one shard)
    if (g.trans_b ? (g.b_rows % BN != 0 || g.b_rows * n_shards < g.N)
                  : (g.b_rows % BK != 0 || g.b_rows * n_shards < g.Kd))
        return false;
    for (int c = 0; c < n_shards; ++c)
        if (((uintptr_t)g.b_shard[c] & 15) != 0) return false;
    for (int i = 0; i < g.nb; ++i)
        if (!g.trans_b && g.b_copy[i] && ((uintptr_t)g.b_copy[i] & 15) != 0) return false;
    return true;
}

hipError_t launch_gemm_f32(const GemmF32Batch &g, hipStream_t st)
{
    if (g.nb <= 0 || g.M <= 0 || g.N <= 0) return hipSuccess;
    const long long gx = (g.N + BN - 1) / BN, gy = (g.M + BM - 1) / BM;
    const long long blocks = gx * gy * g.nb;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (g.trans_a && g.trans_b) return hipErrorInvalidValue;
    const bool whole = f32_whole(g);
    if (g.b_rows > 0 && (g.trans_a || !whole ||
                         (g.trans_b ? g.b_rows % BN != 0 : g.b_rows % BK != 0)))
        return hipErrorInvalidValue;
    // grids that leave CUs idle get eight waves per tile (k split in two)
    const bool split = blocks <= kSplitMax;
    if (g.trans_a) {
        if (split) launch_f32<1, 512>(g, blocks, gx, whole, st);
        else launch_f32<1, 256>(g, blocks, gx, whole, st);
    } else if (g.trans_b) {
        if (split) launch_f32<2, 512>(g, blocks, gx, whole, st);
        else launch_f32<2, 256>(g, blocks, gx, whole, st);
    } else {
        if (split) launch_f32<0, 512>(g, blocks, gx, whole, st);
        else launch_f32<0, 256>(g, blocks, gx, whole, st);
    }
    return hipGetLastError();
}

}  // namespace dps
