// Batched fp32 GEMM on CDNA4 matrix cores, for the local dots of the FSDP
// layer step ("Sharding and Parallelism", "Real HLO before and after
// partitioning": after the weight AllGather each rank runs its local dot
// x_local[128,512] . w[512,512]; "FSDP and ZeRO": the backward pass produces the
// weight gradient that is then reduce-scattered).
//
// One workgroup (4 waves) computes a 64x64 tile of C for one batch entry
// (rank = workgroup id mod K). Each wave owns a 32x32 quadrant and accumulates
// it with v_mfma_f32_32x32x2f32. The k dimension is walked in stages of 32: the
// next two stages' A and B tiles are in flight from global memory into
// registers (16-byte loads where the tile is whole and aligned) while the
// current stage's MFMAs run from LDS; LDS is double-buffered so one barrier per
// stage suffices. A is
// kept k-major in LDS so each MFMA operand read is one contiguous 32-float row
// segment per half-wave.
//
// MFMA 32x32x2 f32 operand layout (lane l of the wave):
//   A operand: A[i = l % 32][k = l / 32]      B operand: B[k = l / 32][j = l % 32]
//   D register r: D[i = 8*(r/4) + 4*(l/32) + r%4][j = l % 32]
// (Shared by gemm_f32.hip and fsdp_kernels.hip.)
#pragma once

#include "dps_internal.h"

namespace dps {
namespace f32tile {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64, BN = 64, BK = 32, LDP = 64 + 4;

constexpr int kDepth = 2;            // k stages in flight from global memory (even)
static_assert(kDepth >= 2 && kDepth % 2 == 0, "an even number of register stages");

constexpr int kSplitMax = 256;       // largest grid that gets eight waves per tile

// Stage loader: the 64x32 A and 32x64 B tiles of one stage as 2 x 256 float4
// each; with NT threads every thread takes 512/NT of them (h = 0, 1 for 256
// threads; h = threadIdx.x / 256 for 512).
// TA: bit 0 = A stored [Kd][M] (else [M][Kd]); bit 1 = B stored [N][Kd] (else
// [Kd][N]). LDS always holds A k-major (As[k][i]) and B k-major (Bs[k][j]).
template <int TA, int NT>
struct Stage {
    static constexpr int NH = 512 / NT;
    static constexpr bool TRA = TA & 1, TRB = (TA & 2) != 0;
    f32x4 a[NH], b[NH];
    long long kb;                       // k0 of the stage held

    // the B tile held, written to rows kb.. of the [Kd][N] matrix W (whole
    // tiles, B not transposed)
    __device__ __forceinline__ void copy_b(float *__restrict__ W, long long N, long long n0) const
    {
        const int t = threadIdx.x & 255;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const int h = NH == 2 ? hh : (int)(threadIdx.x >> 8);
            const long long k = kb + (t >> 4) + 16 * h, j = n0 + (t & 15) * 4;
            *reinterpret_cast<f32x4 *>(W + k * N + j) = b[hh];
        }
    }

    // WHOLE: every tile is inside the matrices and 16-byte aligned, so all
    // loads are unconditional 16-byte loads (the guarded form, if-converted by
    // the compiler, would issue both forms and wait on all of them)
    // Bk0: address of row k0 of B, or with B transposed of row n0 (B may be
    // split into row shards).
    template <bool WHOLE>
    __device__ __forceinline__ void load(const float *__restrict__ A, const float *__restrict__ Bk0,
                                         long long M, long long N, long long Kd, long long m0,
                                         long long n0, long long k0, bool vec_a, bool vec_b)
    {
        if (WHOLE) vec_a = vec_b = true;
        kb = k0;
        const int t = threadIdx.x & 255;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const int h = NH == 2 ? hh : (int)(threadIdx.x >> 8);
            if (!TRA) {
                // A stored [M][Kd]: row m0 + t/8 + 32h, k k0 + (t%8)*4 .. +3
                const long long i = m0 + (t >> 3) + 32 * h, k = k0 + (t & 7) * 4;
                if (vec_a) {
                    a[hh] = *reinterpret_cast<const f32x4 *>(A + i * Kd + k);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[hh][e] = (i < M && k + e < Kd) ? A[i * Kd + k + e] : 0.0f;
                }
            } else {
                // A stored [Kd][M]: k row k0 + t/16 + 16h, i m0 + (t%16)*4 .. +3
                const long long k = k0 + (t >> 4) + 16 * h, i = m0 + (t & 15) * 4;
                if (vec_a) {
                    a[hh] = *reinterpret_cast<const f32x4 *>(A + k * M + i);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[hh][e] = (k < Kd && i + e < M) ? A[k * M + i + e] : 0.0f;
                }
            }
            if (TRB) {
                // B stored [N][Kd]: row n0 + t/8 + 32h, k k0 + (t%8)*4 .. +3
                const long long jr = (t >> 3) + 32 * h, j = n0 + jr, k = k0 + (t & 7) * 4;
                if (vec_b) {
                    b[hh] = *reinterpret_cast<const f32x4 *>(Bk0 + jr * Kd + k);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) b[hh][e] = (j < N && k + e < Kd) ? Bk0[jr * Kd + k + e] : 0.0f;
                }
            } else {
                // B stored [Kd][N]: k row k0 + t/16 + 16h, j n0 + (t%16)*4 .. +3
                const long long kr = (t >> 4) + 16 * h, k = k0 + kr, j = n0 + (t & 15) * 4;
                if (vec_b) {
                    b[hh] = *reinterpret_cast<const f32x4 *>(Bk0 + kr * N + j);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) b[hh][e] = (k < Kd && j + e < N) ? Bk0[kr * N + j + e] : 0.0f;
                }
            }
        }
    }

    __device__ __forceinline__ void store(float (*As)[LDP], float (*Bs)[LDP]) const
    {
        const int t = threadIdx.x & 255;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const int h = NH == 2 ? hh : (int)(threadIdx.x >> 8);
            if (!TRA) {
                const int i = (t >> 3) + 32 * h, k = (t & 7) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) As[k + e][i] = a[hh][e];
            } else {
                *reinterpret_cast<f32x4 *>(&As[(t >> 4) + 16 * h][(t & 15) * 4]) = a[hh];
            }
            if (TRB) {
                const int j = (t >> 3) + 32 * h, k = (t & 7) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) Bs[k + e][j] = b[hh][e];
            } else {
                *reinterpret_cast<f32x4 *>(&Bs[(t >> 4) + 16 * h][(t & 15) * 4]) = b[hh];
            }
        }
    }
};

// NT = 256: four waves, one 32x32 quadrant each over the whole k range.
// NT = 512 (grids too small to fill the CUs): eight waves; waves 4-7 take the
// upper half of every 32-deep stage for the same quadrants, and their partial
// tiles are added to those of waves 0-3 through LDS at the end (a fixed order:
// lower half + upper half), so twice as many SIMDs run half-length MFMA chains.
// FUSE = 1 (whole tiles, B not transposed): B's rows come from row shards (row
// k in b_shard[k / b_rows], each k stage inside one shard) and every B tile
// loaded is also written to b_copy[entry] by one of the tiles that load it, so
// one launch does the AllGather of the shards and the dot that consumes it.
// FUSE = 2 (whole tiles, B transposed): B^T's rows (the N dimension) come from
// row shards (row j in b_shard[j / b_rows], each 64-row tile inside one
// shard): a dot with the transpose of a row-sharded matrix, without gathering
// it first.
// The LDS stage buffers (As, Bs: 2 x BK x LDP floats each) are the caller's, so
// different tile kinds in one kernel can share them.
// One tile of C, for workgroup number id of the launch (NT threads). Batch is
// GemmF32Batch or a struct with the same fields and fewer entries.
template <int TA, int NT, bool WHOLE, int FUSE, class Batch>
__device__ __forceinline__ void gemm_f32_tile(const Batch &g, const int tiles_x, const int id,
                                              float (*__restrict__ As)[BK][LDP],
                                              float (*__restrict__ Bs)[BK][LDP])
{
    constexpr bool TRA = TA & 1, TRB = (TA & 2) != 0;
    // 1-D grid, batch entry = id mod nb: with 8 ranks, workgroup ids round-robin
    // over the 8 XCDs put every tile of rank r on XCD r, so a rank's A and B
    // stay in one XCD's L2
    const int bz = id % g.nb;
    const int tile = id / g.nb;
    const float *__restrict__ A = g.a[bz];
    const float *__restrict__ B = g.b[bz];
    float *__restrict__ C = g.c[bz];
    const long long M = g.M, N = g.N, Kd = g.Kd;
    const long long m0 = (long long)(tile / tiles_x) * BM, n0 = (long long)(tile % tiles_x) * BN;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wi = (wave & 3) >> 1, wj = wave & 1;
    constexpr int KSPAN = NT == 512 ? BK / 2 : BK;     // k values of a stage per wave
    const int kbase = NT == 512 ? (wave >> 2) * KSPAN : 0;
    // whole-tile 16-byte loads need the tile inside the matrix, 16-byte aligned
    // base pointers and row lengths that keep every row 16-byte aligned
    const bool rows_a = ((uintptr_t)A & 15) == 0 && m0 + BM <= M &&
                        (!TRA ? (Kd & 3) == 0 : (M & 3) == 0);
    const bool rows_b = ((uintptr_t)B & 15) == 0 && n0 + BN <= N &&
                        (TRB ? (Kd & 3) == 0 : (N & 3) == 0);
    const long long stages = (Kd + BK - 1) / BK;

    f32x16 acc = {};
    // DEPTH register sets: while stage s is multiplied from LDS, stages
    // s+1 .. s+DEPTH-1 are in flight from global memory and the set that held
    // stage s (already in LDS) takes stage s+DEPTH, so every load has DEPTH-1
    // stages of compute to arrive in
    Stage<TA, NT> r[kDepth];
    auto load = [&](Stage<TA, NT> &st, long long s) {
        const long long k0 = s * BK;
        const float *Bk0 = TRB ? B + n0 * Kd : B + k0 * N;
        if (FUSE == 1) {
            const long long c = k0 / g.b_rows;
            Bk0 = g.b_shard[c] + (k0 - c * g.b_rows) * N;
        } else if (FUSE == 2) {
            const long long c = n0 / g.b_rows;
            Bk0 = g.b_shard[c] + (n0 - c * g.b_rows) * Kd;
        }
        st.template load<WHOLE>(A, Bk0, M, N, Kd, m0, n0, k0, rows_a && k0 + BK <= Kd,
                                rows_b && k0 + BK <= Kd);
    };
    // the copy of a B tile is written by one of the tiles_y tiles that load
    // it: stage s by the tile in tile row s mod tiles_y, so the extra writes
    // are spread evenly over the tile rows
    float *__restrict__ Wc = FUSE == 1 ? g.b_copy[bz] : nullptr;
    const long long tiles_y = (M + BM - 1) / BM, ty = m0 / BM;
    auto put = [&](const Stage<TA, NT> &st, int buf) {
        st.store(As[buf], Bs[buf]);
        if (FUSE == 1 && Wc && (st.kb / BK) % tiles_y == ty) st.copy_b(Wc, N, n0);
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int kk = kbase; kk < kbase + KSPAN; kk += 2) {
            const float a = As[buf][kk + (lane >> 5)][wi * 32 + (lane & 31)];
            const float b = Bs[buf][kk + (lane >> 5)][wj * 32 + (lane & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
    };
    if (WHOLE) {
        // stages is a multiple of kDepth (checked by the launcher); the body has
        // no branch, so no load can be moved down to its use: past the end the
        // loads repeat the last stage and the last store lands in a buffer that
        // is never read
#pragma unroll
        for (int i = 0; i < kDepth; ++i) load(r[i], i);
        put(r[0], 0);
        __syncthreads();
        for (long long s = 0; s < stages; s += kDepth) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) {
                const long long st = s + i;
                load(r[i], min(st + kDepth, stages - 1));
                mma(i & 1);
                put(r[(i + 1) % kDepth], (i + 1) & 1);
                __syncthreads();
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kDepth; ++i)
            if (i < stages) load(r[i], i);
        r[0].store(As[0], Bs[0]);
        __syncthreads();
        // unrolled by kDepth (even) so that each register set and LDS buffer has
        // a fixed role: stage s + i uses set i and LDS buffer i & 1
        for (long long s = 0; s < stages; s += kDepth) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) {
                const long long st = s + i;
                if (st >= stages) break;
                if (st + kDepth < stages) load(r[i], st + kDepth);
                mma(i & 1);
                if (st + 1 >= stages) break;
                r[(i + 1) % kDepth].store(As[(i + 1) & 1], Bs[(i + 1) & 1]);
                __syncthreads();
            }
        }
    }
    if (NT == 512) {
        // upper-half partial tiles through LDS (reusing the stage buffers)
        float *red = &As[0][0][0];          // 4 quadrants x 16 x 64 floats = 16 KiB
        __syncthreads();
        if (wave >= 4) {
#pragma unroll
            for (int r = 0; r < 16; ++r) red[((wave & 3) * 16 + r) * 64 + lane] = acc[r];
        }
        __syncthreads();
        if (wave >= 4) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = acc[r] + red[(wave * 16 + r) * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const long long gi = m0 + wi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const long long gj = n0 + wj * 32 + (lane & 31);
        if (gi < M && gj < N) C[gi * N + gj] = acc[r];
    }
}

}  // namespace f32tile
}  // namespace dps
