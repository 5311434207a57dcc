// bf16 GEMM on CDNA4 matrix cores: C[M,N] = A[M,Kd] . op(B), fp32
// accumulation, bf16 result (round to nearest even). This is the compute
// kernel of a (GEMM, collective) pair run concurrently with the sync kernels
// ("Optimizing ML Concurrent Computation and Communication with GPU DMA
// Engines", section "Problem Formulation": a GEMM and a collective with no data
// dependence between them).
//
// B layouts (template parameter BKN):
//   BKN = true : B stored [Kd, N] row-major (C = A . B, the plain product).
//   BKN = false: B stored [N, Kd] row-major (C = A . B^T, both operands
//                k-contiguous, the linear-layer weight layout).
// A is always [M, Kd] (k-contiguous). The MFMA operands need 8 consecutive k
// values per lane. A k-contiguous operand gives them as one 16-byte run in LDS;
// for an n-contiguous B the stage is stored in LDS as [k][n] rows (coalesced
// 16-byte global loads along n) and each lane's 8 k values are assembled with
// two ds_read_b64_tr_b16 transposing reads, gfx950's LDS load that hands each
// lane of a 16-lane group one 16-bit column of the 4 rows its neighbours
// address (lane i of the group receives element i % 4 of the 8-byte rows
// addressed by lanes 4e + i / 4, e = 0..3; verified on the GPU with an
// in-bounds probe). Every variant and layout walks k in ascending order (16-
// element steps of v_mfma_f32_32x32x16_bf16, or 32-element steps of
// v_mfma_f32_16x16x32_bf16, which accumulate the same products in the same
// order), zero-padded past Kd, so all of them produce the same bits.
//
// Five designs over a tile of C:
//
// * gemm_bf16_w4d_kernel (the default for B stored [N, Kd] where M and N are
//   multiples of 256 and Kd a multiple of 128, at least 384): the operands go
//   from global memory straight into LDS, 4 waves of 128x128 with 16x16x32
//   MFMAs; described at the kernel.
//
// * gemm_bf16_w4dn_kernel (the same for B stored [Kd, N], Kd at least 256):
//   the same loads into LDS and 16x16x32 MFMAs, B's fragments assembled with
//   transposing LDS reads; described at the kernel.
//
// * gemm_bf16_w4_kernel (the default where M and N are multiples of 256, Kd a
//   multiple of 64 and at least 1024, and the direct-to-LDS kernels do not
//   apply): 4 waves, one per SIMD, each owning a 128x128 quarter (4x4 MFMA
//   blocks, 256 fp32 accumulators per lane held in the accumulation registers).
//   A 128x128 wave tile reads 8 fragments from LDS per 16 MFMAs, against 6
//   per 8 for a 128x64 wave tile, so the LDS read traffic per flop drops by a
//   third, which is what bounds the 8-wave design below. With one wave per SIMD
//   nothing hides an LDS wait, so the stage is software-pipelined by hand: the
//   fragments of the next k step are read while the current step's MFMAs run
//   (two fragment register sets), and each of the 16 groups of 4 MFMAs also
//   carries one 16-byte LDS store of the next stage and one global load three
//   stages ahead (scheduling fences keep that interleave). The loads alternate
//   between two staging register sets, so each has two stages to arrive before
//   its LDS store needs it. Global loads use a buffer descriptor on the tile's
//   first row (first column for an n-contiguous B), so their addresses are one
//   per-lane offset register plus a scalar offset.
//
// * gemm_bf16_kernel: 8 waves arranged 2 (rows) x 4 (columns), each wave
//   128x64 = 4x2 MFMA blocks (128 fp32 accumulators per lane), k stages of TK
//   (32 or 64) through double-buffered LDS. It fits in 224 (TK=64) or 198
//   (TK=32) VGPRs, which leaves room for a sync workgroup on the same CU; it also
//   takes any shape whose rows are 16-byte aligned (edge tiles on a guarded
//   path). With EARLY, a stage's operands are loaded into registers two stages
//   ahead and written to the idle LDS buffer at the start of the next stage, so
//   the LDS writes overlap that stage's MFMAs instead of standing between the
//   MFMAs and the barrier.
//
// * gemm_bf16_any_kernel: any shape, any element-aligned pointers, any Kd: 64x64
//   tiles of 4 waves, each lane gathering its MFMA operands straight from
//   global memory with guarded 2-byte loads. Slow; it serves what the two
//   kernels above cannot take (rows that are not 16-byte aligned).
//
// A 256x256 tile does 128 flop per byte loaded, which keeps the kernels off the
// L2 bandwidth limit a 128x128 tile (64 flop/byte) runs into. Tiles are ordered
// so that the workgroups running together on one XCD (ids round-robin over 8
// XCDs) cover a compact block of C and share A and B rows in that XCD's L2.
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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Padded LDS row of an n-contiguous B stage: 256 + 32 elements = 576 bytes, so
// consecutive k rows start 64 bytes apart modulo 256 and the 8 rows x 64 bytes
// one transposing read of a wave touches fall on every bank exactly twice.
constexpr int BKN_LDN = 256 + 32;

// MFMA B operand of lane `lane` for the 32 columns starting at column `col` of
// an [k][n] LDS stage whose row `row0` is the block's first k: lane group g =
// lane / 16 covers columns 16 (g % 2) .. + 15 and k 8 (g / 2) .. + 7; within
// the group lane jj addresses row jj / 4 (+4 for the second read) at column
// 4 (jj % 4), and receives its own column's 4 k values from each read.
__device__ __forceinline__ bf16x8 b_operand_kn(const unsigned short *stage, int ldn, int row0,
                                               int col, int lane)
{
    const int g = lane >> 4, jj = lane & 15;
    const unsigned short *p = stage + (row0 + 8 * (g >> 1) + (jj >> 2)) * ldn + col +
                              16 * (g & 1) + 4 * (jj & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * ldn));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

constexpr int TM = 256, TN = 256;                           // workgroup tile of C
constexpr int NT = 512;                                     // threads per workgroup
constexpr int WM = 128, WN = 64;                            // per-wave tile
constexpr int BI = WM / 32, BJ = WN / 32;                   // MFMA blocks per wave

// written as a select, so that an epilogue converting many values has no
// branches: NaN -> quiet NaN with its sign and upper payload bits, otherwise
// round to nearest even (overflow to infinity)
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f)
{
    const unsigned u = __float_as_uint(f);
    const unsigned nan = (u >> 16) | 0x40u;
    const unsigned rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (unsigned short)((u & 0x7fffffffu) > 0x7f800000u ? nan : rne);
}

// Workgroup id -> (tile row, tile col). Ids go round-robin to the 8 XCDs; the
// ids of one XCD are handed a compact group of tiles (GROUP tile rows at a
// time, column-major inside the group) so that concurrently running
// workgroups of one XCD reuse A and B rows from its L2.
__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int total = tiles_m * tiles_n;
    constexpr int XCDS = 8, GROUP = 4;
    if (total % XCDS == 0) {
        const int per = total / XCDS;
        id = (id % XCDS) * per + id / XCDS;      // contiguous range per XCD
    }
    const int group_tiles = GROUP * tiles_n;
    const int g = id / group_tiles;
    const int first_m = g * GROUP;
    const int rows = min(GROUP, tiles_m - first_m);
    const int in = id - g * group_tiles;
    tm = first_m + in % rows;
    tn = in / rows;
}

// TK: k depth of one LDS stage (64: full 128-byte rows per load, 228 VGPRs,
// 144 KiB LDS; 32: 198 VGPRs and 80 KiB, which leaves room on the CU for a
// sync workgroup beside the GEMM workgroup). BKN: B stored [Kd, N] (see above);
// then N must be a multiple of 8 (16-byte rows) as Kd must for A.
template <bool EDGE, int TK, bool EARLY, bool BKN>
__global__ __launch_bounds__(NT) void gemm_bf16_kernel(const unsigned short *__restrict__ A,
                                                       const unsigned short *__restrict__ B,
                                                       unsigned short *__restrict__ C, int M, int N,
                                                       int Kd, int tiles_m, int tiles_n)
{
    constexpr int LDK = TK + 8;      // LDS row padded by 16 bytes
    constexpr int CH = TK / 8;       // 16-byte chunks per tile row
    constexpr int RPP = NT / CH;     // rows loaded per pass
    constexpr int HP = TM / RPP;     // passes per tile
    // B stage: [TN][LDK] (k-contiguous) or [TK][BKN_LDN] (n-contiguous)
    constexpr int BR = BKN ? TK : TN, BC = BKN ? BKN_LDN : LDK;
    // n-contiguous B: thread -> 16-byte chunk bc of k rows br + 16h
    constexpr int BHP = BKN ? TK / 16 : HP;
    static_assert(!BKN || BHP * 16 * 32 == TK * TN / 8, "B chunks per thread");
    __shared__ __attribute__((aligned(16))) unsigned short As[2][TM][LDK];
    __shared__ __attribute__((aligned(16))) unsigned short Bs[2][BR][BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wi = wave >> 2, wj = wave & 3;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const long long m0 = (long long)tm * TM, n0 = (long long)tn * TN;

    // global -> register staging: rows lr + RPP*h of A (and of a k-contiguous
    // B), 8 bf16 at k lk; an n-contiguous B: k rows br + 16h, 8 bf16 at column 8*bc
    const int lr = tid / CH, lk = (tid % CH) * 8;
    const int bc = tid & 31, br = tid >> 5;
    u32x4 ra[HP], rb[BHP];
    auto gload = [&](int k0) {
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            const long long gi = m0 + lr + RPP * h;
            const int gk = k0 + lk;
            if (EDGE) {
                const bool kin = gk + 8 <= Kd;
                ra[h] = (gi < M && kin) ? *reinterpret_cast<const u32x4 *>(A + gi * Kd + gk) : u32x4{0, 0, 0, 0};
            } else {
                ra[h] = *reinterpret_cast<const u32x4 *>(A + gi * Kd + gk);
            }
        }
#pragma unroll
        for (int h = 0; h < BHP; ++h) {
            if constexpr (BKN) {
                const long long gk = k0 + br + 16 * h, gj = n0 + 8 * bc;
                if (EDGE)
                    rb[h] = (gk < Kd && gj < N) ? *reinterpret_cast<const u32x4 *>(B + gk * N + gj)
                                                : u32x4{0, 0, 0, 0};
                else
                    rb[h] = *reinterpret_cast<const u32x4 *>(B + gk * N + gj);
            } else {
                const long long gj = n0 + lr + RPP * h;
                const int gk = k0 + lk;
                if (EDGE)
                    rb[h] = (gj < N && gk + 8 <= Kd) ? *reinterpret_cast<const u32x4 *>(B + gj * Kd + gk)
                                                     : u32x4{0, 0, 0, 0};
                else
                    rb[h] = *reinterpret_cast<const u32x4 *>(B + gj * Kd + gk);
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int h = 0; h < HP; ++h)
            *reinterpret_cast<u32x4 *>(&As[buf][lr + RPP * h][lk]) = ra[h];
#pragma unroll
        for (int h = 0; h < BHP; ++h) {
            if constexpr (BKN)
                *reinterpret_cast<u32x4 *>(&Bs[buf][br + 16 * h][8 * bc]) = rb[h];
            else
                *reinterpret_cast<u32x4 *>(&Bs[buf][lr + RPP * h][lk]) = rb[h];
        }
    };

    f32x16 acc[BI][BJ];
#pragma unroll
    for (int a = 0; a < BI; ++a)
#pragma unroll
        for (int b = 0; b < BJ; ++b) acc[a][b] = f32x16{};

    const int stages = (Kd + TK - 1) / TK;
    gload(0);
    sstore(0);
    if (EARLY && stages > 1) gload(TK);
    __syncthreads();
    int buf = 0;
    for (int s = 0; s < stages; ++s) {
        const bool more = s + 1 < stages;
        if (EARLY) {
            // stage s+1 (loaded during the previous stage) goes to the other
            // buffer now, overlapping this stage's MFMAs; that buffer was last
            // read before the previous barrier
            if (more) {
                sstore(buf ^ 1);
                if (s + 2 < stages) gload((s + 2) * TK);
            }
        } else if (more) {
            gload((s + 1) * TK);
        }
#pragma unroll
        for (int ks = 0; ks < TK / 16; ++ks) {
            bf16x8 av[BI], bv[BJ];
#pragma unroll
            for (int a = 0; a < BI; ++a)
                av[a] = *reinterpret_cast<const bf16x8 *>(&As[buf][wi * WM + a * 32 + (lane & 31)][ks * 16 + 8 * (lane >> 5)]);
#pragma unroll
            for (int b = 0; b < BJ; ++b) {
                if constexpr (BKN)
                    bv[b] = b_operand_kn(&Bs[buf][0][0], BKN_LDN, ks * 16, wj * WN + b * 32, lane);
                else
                    bv[b] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][wj * WN + b * 32 + (lane & 31)][ks * 16 + 8 * (lane >> 5)]);
            }
#pragma unroll
            for (int a = 0; a < BI; ++a)
#pragma unroll
                for (int b = 0; b < BJ; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
        if (more) {
            if (!EARLY) sstore(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }
#pragma unroll
    for (int a = 0; a < BI; ++a)
#pragma unroll
        for (int b = 0; b < BJ; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const long long gi = m0 + wi * WM + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const long long gj = n0 + wj * WN + b * 32 + (lane & 31);
                if (!EDGE || (gi < M && gj < N)) C[gi * N + gj] = f32_to_bf16_rne(acc[a][b][r]);
            }
}


// ----------------------------------------------------------- 4-wave kernel

constexpr int W4_NT = 256;                  // 4 waves
constexpr int W4_TK = 64;                   // k per stage
constexpr int W4_LDK = W4_TK + 8;           // LDS row padded by 16 bytes (no bank conflicts)
constexpr int W4_CH = W4_TK / 8;            // 16-byte chunks per tile row
constexpr int W4_RPP = W4_NT / W4_CH;       // rows loaded per pass (32)
constexpr int W4_HP = TM / W4_RPP;          // passes per operand tile (8)
constexpr int W4_KS = W4_TK / 16;           // MFMA k steps per stage (4)
constexpr int W4_B = 4;                     // 32x32 MFMA blocks per wave side (128 = 4 x 32)
constexpr long long kW4MinK = 1024;         // shortest k range given to the register-staged 4-wave kernel
constexpr long long kDirectMinK = 256;      // shortest k range given to the direct-to-LDS kernel for B [Kd, N]
constexpr long long kDirectMinKNk = 384;    // and to the one for B [N, Kd]
constexpr long long kNtcMinK = 8192;        // k range from which C leaves in nontemporal stores
static_assert(W4_HP * 2 == W4_KS * W4_B, "one staged 16-byte load per group of MFMAs");

// keeps the compiler's scheduler from moving instructions across it, so the
// interleave of LDS reads, LDS stores, global loads and MFMAs stays as written
#define W4_FENCE() __builtin_amdgcn_sched_barrier(0)

template <bool BKN>
__global__ __launch_bounds__(W4_NT) void gemm_bf16_w4_kernel(const unsigned short *__restrict__ A,
                                                             const unsigned short *__restrict__ B,
                                                             unsigned short *__restrict__ C, int M,
                                                             int N, int Kd, int tiles_m,
                                                             int tiles_n)
{
    // B stage: [TN][W4_LDK] (k-contiguous) or [W4_TK][BKN_LDN] (n-contiguous);
    // the same 73,728 bytes either way
    constexpr int BR = BKN ? W4_TK : TN, BC = BKN ? BKN_LDN : W4_LDK;
    __shared__ __attribute__((aligned(16))) unsigned short As[2][TM][W4_LDK];
    __shared__ __attribute__((aligned(16))) unsigned short Bs[2][BR][BC];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wi = wave >> 1, wj = wave & 1;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const long long m0 = (long long)tm * TM, n0 = (long long)tn * TN;

    // Staging: two sets of 16 registers of 16 bytes per lane; st[t][h] holds A
    // row lr + 32h at k chunk lk, and st[t][8 + h] B row lr + 32h at k chunk lk
    // (k-contiguous B) or B's k row br + 8h at columns 8*bc (n-contiguous B),
    // of one stage. Byte offsets from the descriptors' bases fit 31 bits
    // (checked by the launcher).
    const int lr = tid / W4_CH, lk = (tid % W4_CH) * 8;
    const int bc = tid & 31, br = tid >> 5;
    const unsigned voff = (unsigned)((lr * Kd + lk) * 2);
    const unsigned voff_b = BKN ? (unsigned)((br * N + 8 * bc) * 2) : voff;
    const __amdgpu_buffer_rsrc_t rA =
        __builtin_amdgcn_make_buffer_rsrc((void *)(A + m0 * Kd), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(BKN ? B + n0 : B + n0 * Kd), (short)0, 0x7fffffff, 0x00020000);
    u32x4 st[2][2 * W4_HP];
    auto gload1 = [&](int t, int j, int k0) __attribute__((always_inline)) {
        if (j < W4_HP) {
            const int so = (W4_RPP * j * Kd + k0) * 2;
            st[t][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, voff, so, 0));
        } else if (BKN) {
            const int so = ((k0 + 8 * (j - W4_HP)) * N) * 2;
            st[t][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, voff_b, so, 0));
        } else {
            const int so = (W4_RPP * (j - W4_HP) * Kd + k0) * 2;
            st[t][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, voff_b, so, 0));
        }
    };
    auto sstore1 = [&](int t, int buf, int j) __attribute__((always_inline)) {
        unsigned short *row = j < W4_HP ? &As[buf][lr + W4_RPP * j][lk]
                              : BKN     ? &Bs[buf][br + 8 * (j - W4_HP)][8 * bc]
                                        : &Bs[buf][lr + W4_RPP * (j - W4_HP)][lk];
        *reinterpret_cast<u32x4 *>(row) = st[t][j];
    };

    f32x16 acc[W4_B][W4_B];
#pragma unroll
    for (int a = 0; a < W4_B; ++a)
#pragma unroll
        for (int b = 0; b < W4_B; ++b) acc[a][b] = f32x16{};

    // two fragment sets: k step ks computes from set ks & 1 while the next
    // step's fragments arrive in the other
    bf16x8 av[2][W4_B], bv[2][W4_B];
    auto rd = [&](int set, int buf, int ks, int x) __attribute__((always_inline)) {
        const int r = lane & 31, kc = ks * 16 + 8 * (lane >> 5);
        av[set][x] = *reinterpret_cast<const bf16x8 *>(&As[buf][wi * 128 + x * 32 + r][kc]);
        if constexpr (BKN)
            bv[set][x] = b_operand_kn(&Bs[buf][0][0], BKN_LDN, ks * 16, wj * 128 + x * 32, lane);
        else
            bv[set][x] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][wj * 128 + x * 32 + r][kc]);
    };

    // One stage from LDS buffer buf: 16 groups of 4 MFMAs (k step ks, A block a);
    // group j also reads fragment pair a of step ks+1, stores staging register
    // st[buf][j] (the next stage, loaded two stages ago) into the idle buffer
    // and reloads it from k offset kload (three stages ahead). Called with
    // literal arguments only, so every register and LDS index is fixed at
    // compile time; io = false (an odd last stage) leaves the staging alone.
    auto stage = [&](int buf, int kload, bool io) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < W4_B; ++x) rd(0, buf, 0, x);
        W4_FENCE();
#pragma unroll
        for (int ks = 0; ks < W4_KS; ++ks) {
#pragma unroll
            for (int a = 0; a < W4_B; ++a) {
                const int j = ks * W4_B + a;
                if (ks + 1 < W4_KS) rd((ks + 1) & 1, buf, ks + 1, a);
                if (io) {
                    sstore1(buf, buf ^ 1, j);
                    gload1(buf, j, kload);
                }
#pragma unroll
                for (int b = 0; b < W4_B; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks & 1][a], bv[ks & 1][b],
                                                                        acc[a][b], 0, 0, 0);
                W4_FENCE();
            }
        }
    };

    // Stage s computes from LDS buffer s & 1. Before it, stage s+1 sits in
    // staging set s & 1 and stage s+2 in the other set (or, for s = 0, stage 1
    // in set 0 and stage 2 in set 1). Past the end the loads repeat the last
    // stage and the stores land in a buffer that is never read again, so the
    // loop body has no branch.
    const int stages = Kd / W4_TK;
    const int last = (stages - 1) * W4_TK;
#pragma unroll
    for (int j = 0; j < 2 * W4_HP; ++j) gload1(0, j, 0);
#pragma unroll
    for (int j = 0; j < 2 * W4_HP; ++j) sstore1(0, 0, j);
#pragma unroll
    for (int j = 0; j < 2 * W4_HP; ++j) gload1(0, j, min(W4_TK, last));
#pragma unroll
    for (int j = 0; j < 2 * W4_HP; ++j) gload1(1, j, min(2 * W4_TK, last));
    __syncthreads();
    int s = 0;
    for (; s + 2 <= stages; s += 2) {
        stage(0, min((s + 3) * W4_TK, last), true);
        __syncthreads();
        stage(1, min((s + 4) * W4_TK, last), true);
        __syncthreads();
    }
    if (s < stages) stage(0, 0, false);
#pragma unroll
    for (int a = 0; a < W4_B; ++a)
#pragma unroll
        for (int b = 0; b < W4_B; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const long long gi = m0 + wi * 128 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const long long gj = n0 + wj * 128 + b * 32 + (lane & 31);
                C[gi * N + gj] = f32_to_bf16_rne(acc[a][b][r]);
            }
}

// ------------------------------------------- 4-wave direct-to-LDS kernel

// For B stored [N, Kd] (both operands k-contiguous). 256x256 tile, 4 waves of
// 128x128 (8x8 blocks of v_mfma_f32_16x16x32_bf16, 256 fp32 accumulators per
// lane), k stages of 64 through two LDS buffers that the operands reach
// straight from global memory (buffer_load ... lds): no staging registers and
// no LDS store instructions. A stage row of 64 bf16 is one 128-byte line;
// each load instruction writes 1 KiB of LDS, lane l's 16 bytes at offset 16 l,
// and moves 8 rows, lane l fetching chunk (l % 8) ^ (l / 8) of row l / 8, so
// chunk c of row r sits at position c ^ (r % 8) and the fragment reads of 16
// rows at one chunk hit distinct banks. Wave w loads rows 64w .. 64w + 63 of
// both operands.
//
// Stage t computes from buffer t & 1 in two k steps of 32: step 0 while the
// fragments of step 1 are read (one read per 4 MFMAs); then each wave waits
// for its own loads of stage t + 1 and the workgroup meets at the barrier;
// then step 1 while the step-0 fragments of stage t + 1 are read (one per 4
// MFMAs) and the 16 loads of stage t + 2 go into buffer t & 1 (all its reads
// finished before the barrier), one per 3 MFMAs over the first 46 of the
// step's 64: early enough to land before the next barrier, spread enough to
// keep the address unit's queues from filling (one per 4 MFMAs: 2.4% slower;
// one per 2 or 1: 21% slower). The k steps add the same products in the same
// order as the 32x32x16 kernels, and the results are the same bits.
// Measured at 8192^3: 724 us (1518 TFLOP/s) against 804 us for the
// register-staged kernel and 673 us for the vendor library on the same GPU.
// The MFMAs take B's fragment first, so each lane ends with four consecutive
// columns of a row of C per block and C leaves in 16-byte stores (store_c_tr).
// An n-contiguous B takes the kernel after this one.
constexpr int D_NT = 256, D_TK = 64;
constexpr int D_ELEMS = TM * D_TK;          // one operand's stage: 16,384 bf16 = 32 KiB

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// C of one wave's 128x128 block (rows wi*128.., columns wj*128.. of the tile at
// rC) from accumulators holding transposed 16x16 blocks: the direct-to-LDS
// kernels pass B's fragment as the MFMA's first operand and A's as its second,
// which yields the same products and sums (bf16 products are exact in fp32 and
// each output element adds its 32 products in the same order) with register r
// of block (a, b) in lane l holding C[16a + l%16][16b + 4(l/16) + r]: four
// consecutive columns of one row. With C16 (C 16-byte aligned, N a multiple of
// 8) pairs of values become bf16 pairs in one v_cvt_pk_bf16_f32 (round to
// nearest even, NaN quieted with sign and upper payload kept: the same bits as
// f32_to_bf16_rne for every one of the 2^32 inputs, checked exhaustively on the
// GPU), and v_permlane16_swap_b32 trades the halves of blocks b and b+1 between
// lane rows g and g^1 of 16, so that each lane holds 8 consecutive columns of
// one row: one 16-byte store per two blocks, 32 per lane instead of 256 2-byte
// stores (8192^3: 733 -> 720 us; 4096 x 8192 x 1024: 71 -> 62 us). Otherwise
// 2-byte stores of any alignment. NTC marks the 16-byte stores nontemporal:
// faster where the k range is long (8192^3: 1.1-2.2% for both layouts), slower
// where C's writes weigh more (kk = 4096: +1-1.7% for B [k, n]; kk = 2048: +6%;
// kk = 1024: +11%), so the launcher sets it from kk = 8192.
template <bool C16, bool NTC>
__device__ __forceinline__ void store_c_tr(const f32x4 (&acc)[8][8], const __amdgpu_buffer_rsrc_t rC,
                                           int N, int wi, int wj, int lane)
{
    const int row = wi * 128 + (lane & 15), g = lane >> 4;
    if constexpr (C16) {
        const int coff = (row * N + wj * 128 + 16 * (g & 1) + 8 * (g >> 1)) * 2;
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int b = 0; b < 8; b += 2) {
                const f32x2 x0 = {acc[a][b][0], acc[a][b][1]}, x1 = {acc[a][b][2], acc[a][b][3]};
                const f32x2 y0 = {acc[a][b + 1][0], acc[a][b + 1][1]}, y1 = {acc[a][b + 1][2], acc[a][b + 1][3]};
                // rows g even keep block b's pair and receive the next row's;
                // rows g odd receive the previous row's pair of block b + 1
                const auto s0 = __builtin_amdgcn_permlane16_swap(
                    __builtin_bit_cast(unsigned, __builtin_convertvector(x0, bf16x2)),
                    __builtin_bit_cast(unsigned, __builtin_convertvector(y0, bf16x2)), false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(
                    __builtin_bit_cast(unsigned, __builtin_convertvector(x1, bf16x2)),
                    __builtin_bit_cast(unsigned, __builtin_convertvector(y1, bf16x2)), false, false);
                const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
                __builtin_amdgcn_raw_buffer_store_b128(v, rC, coff, (a * 16 * N + b * 16) * 2, NTC ? 2 : 0);
            }
    } else {
        const int coff = (row * N + wj * 128 + 4 * g) * 2;
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(acc[a][b][r]), rC, coff,
                                                          (a * 16 * N + b * 16 + r) * 2, 0);
    }
}

template <bool C16, bool NTC>
__global__ __launch_bounds__(D_NT) void gemm_bf16_w4d_kernel(const unsigned short *__restrict__ A,
                                                             const unsigned short *__restrict__ B,
                                                             unsigned short *__restrict__ C, int M,
                                                             int N, int Kd, int tiles_m, int tiles_n)
{
    // one array per buffer and operand: the compiler then sees that fragment
    // reads of one buffer do not alias loads in flight into another, and
    // waits for those loads only at the barrier
    __shared__ __attribute__((aligned(1024))) unsigned short A0[D_ELEMS], A1[D_ELEMS];
    __shared__ __attribute__((aligned(1024))) unsigned short B0[D_ELEMS], B1[D_ELEMS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave >> 1, wj = wave & 1;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const long long m0 = (long long)tm * TM, n0 = (long long)tn * TN;
    // byte offsets from the descriptors' bases (a tile's 256 rows: 512 Kd
    // bytes) fit 31 bits (checked by the launcher)
    const __amdgpu_buffer_rsrc_t rA =
        __builtin_amdgcn_make_buffer_rsrc((void *)(A + m0 * Kd), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB =
        __builtin_amdgcn_make_buffer_rsrc((void *)(B + n0 * Kd), (short)0, 0x7fffffff, 0x00020000);
    auto abuf = [&](int buf) __attribute__((always_inline)) { return buf ? A1 : A0; };
    auto bbuf = [&](int buf) __attribute__((always_inline)) { return buf ? B1 : B0; };

    // load q (0..15) of a stage: rows 64 wave + 8 (q % 8) of A (q < 8) or B
    const int lr = lane >> 3;
    const int voff = lr * Kd * 2 + (((lane & 7) ^ lr) << 4);
    auto dtl = [&](int buf, int k0, int q) __attribute__((always_inline)) {
        const int row0 = wave * 64 + (q & 7) * 8;
        const int so = __builtin_amdgcn_readfirstlane((row0 * Kd + k0) * 2);
        if (q < 8)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void *)(abuf(buf) + row0 * D_TK), 16, voff, so, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void *)(bbuf(buf) + row0 * D_TK), 16, voff, so, 0, 0);
    };

    // fragments per k step, two sets: k step ks computes from set ks while
    // the other set is filled. Read q (0..15): q < 8 B block q, else A block
    // q - 8; lane l reads row l % 16 of the block at chunk 4 ks + l / 16.
    bf16x8 af[2][8], bf[2][8];
    const int fp0 = (lane & 15) * D_TK, fx = lane & 7, fc = lane >> 4;
    auto rdq = [&](int set, int buf, int ks, int q) __attribute__((always_inline)) {
        const int x = q & 7;
        const int p = ((ks * 4 + fc) ^ fx) * 8;
        if (q >= 8)
            af[set][x] = *reinterpret_cast<const bf16x8 *>(abuf(buf) + (wi * 128 + x * 16) * D_TK + fp0 + p);
        else
            bf[set][x] = *reinterpret_cast<const bf16x8 *>(bbuf(buf) + (wj * 128 + x * 16) * D_TK + fp0 + p);
    };
    f32x4 acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{};
    auto mf = [&](int set, int a, int b) __attribute__((always_inline)) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[set][b], af[set][a], acc[a][b], 0, 0, 0);
    };

    const int stages = Kd / D_TK;
    const int last = (stages - 1) * D_TK;
    // stage t from buffer buf = t & 1; k2: k offset of stage t + 2 (past the
    // end the loads repeat the last stage into a buffer no MFMA reads again).
    // Called with literal buffer indices only.
    auto stage = [&](int buf, int k2) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            if ((i & 3) == 0) rdq(1, buf, 1, i >> 2);
            mf(0, i >> 3, i & 7);
            W4_FENCE();
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of stage t + 1 landed
        __syncthreads();
        W4_FENCE();
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            if ((i & 3) == 0) rdq(0, buf ^ 1, 0, i >> 2);
            if (i % 3 == 0 && i / 3 < 16) dtl(buf, k2, i / 3);
            mf(1, i >> 3, i & 7);
            W4_FENCE();
        }
    };
#pragma unroll
    for (int q = 0; q < 16; ++q) dtl(0, 0, q);
#pragma unroll
    for (int q = 0; q < 16; ++q) dtl(1, min(D_TK, last), q);
    __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16): this wave's loads of stage 0 landed
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) rdq(0, 0, 0, q);
    W4_FENCE();
    // an even number of stages (the launcher's condition): a loop of stage
    // pairs with no odd stage after it keeps every accumulator in one
    // accumulation register for the whole loop
    for (int s = 0; s < stages; s += 2) {
        stage(0, min((s + 2) * D_TK, last));
        stage(1, min((s + 3) * D_TK, last));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    // the accumulators named as accumulation registers where the loop ends:
    // without this the compiler keeps some of them in architectural registers
    // for the epilogue's conversions and copies them around every loop pass
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) asm volatile("" : "+a"(acc[a][b]));
    // C through a buffer descriptor on the tile's first element: one per-lane
    // offset register, the block and row offsets as scalar offsets (256 N
    // bytes from the base fit 31 bits: checked by the launcher)
    const __amdgpu_buffer_rsrc_t rC =
        __builtin_amdgcn_make_buffer_rsrc((void *)(C + m0 * N + n0), (short)0, 0x7fffffff, 0x00020000);
    store_c_tr<C16, NTC>(acc, rC, N, wi, wj, lane);
}

// ------------------------------------------- 4-wave direct-to-LDS kernel, B stored [Kd, N]

// For B stored [Kd, N] (the plain product). Same tile, waves, LDS buffers,
// 16x16x32 MFMAs (8x8 blocks per wave) and direct-to-LDS loads as the kernel
// above; what differs:
// - B's stage is 64 k rows of 256 n (512 bytes each, one load instruction
//   moving two rows), 16-byte chunk c of row r at position
//   c ^ (4 (r % 4) + 2 ((r / 8) % 2)), which puts the four 16-lane groups of
//   one transposing read on two disjoint halves of the banks
//   (SQ_LDS_BANK_CONFLICT: 0 per 8192^3 product);
// - each B fragment (the 8 k values of one column per lane) is two
//   ds_read_b64_tr_b16 reads, gfx950's transposing LDS load: lane i of a
//   16-lane group receives element i % 4 of the 8-byte rows addressed by lanes
//   4e + i / 4 (e = 0..3) of its group, so lane 4e + h addresses k row e (+4
//   for the second read) at columns 4h .. 4h + 3 and lane i receives 4 k
//   values of column i;
// - a k step walks the 8 column blocks in turn (8 MFMAs each, one per row
//   block); all 8 A fragments of a step are read during the step before, the B
//   fragment of block G two blocks ahead, each into a register set of its own;
// - every LDS read is inline assembly and every wait for one is written out
//   (s_waitcnt lgkmcnt naming the fragments it makes valid): the compiler
//   counts neither the transposing reads nor, here, the others, and its own
//   waits would wait for reads issued after the ones needed. The barrier sits
//   after block 13 of a stage (the last reads of its buffer issued and waited
//   for); the loads of stage t + 2 go into that buffer from then on, one per 3
//   MFMAs, 6 in blocks 14-15 and 10 in step 0 of the next stage;
// - the MFMAs are inline assembly too, with the accumulators as "+a"
//   operands: with builtins the compiler keeps part of the 256 accumulators in
//   architectural registers and copies them through the accumulation
//   registers around every MFMA (~600 moves per loop pass). As it sees neither
//   their latency nor their hazards, every read of the accumulators outside
//   the MFMAs is ordered after a fence asm that names all of them and waits
//   24 cycles.
// Every MFMA chain adds the same products in the same order as the other
// kernels (ascending k, 16x16x32 over 32-wide steps), so the results are the
// same bits. Measured at 8192^3: 718-733 us (1500-1531 TFLOP/s) against
// 759-768 us for the 32x32x16 form of this kernel on the same GPUs (which
// holds a lower clock), level with it from kk = 1024 to 1152 and 3-6% faster
// from 2048. Like the kernel above, its MFMAs take B's fragment first and C
// leaves in 16-byte stores (store_c_tr).

__device__ __forceinline__ bf16x8 lds_read_b128(unsigned addr)
{
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ i16x4 lds_read_tr_b64(unsigned addr)
{
    i16x4 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

#define DN_ACC_ROW(A, TXT)                                                                    \
    asm volatile(TXT : "+a"(acc[A][0]), "+a"(acc[A][1]), "+a"(acc[A][2]), "+a"(acc[A][3]),    \
                 "+a"(acc[A][4]), "+a"(acc[A][5]), "+a"(acc[A][6]), "+a"(acc[A][7]))
#define DN_ACC_FENCE()                                                                        \
    do {                                                                                      \
        DN_ACC_ROW(0, "s_nop 7\n\ts_nop 7\n\ts_nop 7");                                         \
        DN_ACC_ROW(1, ""); DN_ACC_ROW(2, ""); DN_ACC_ROW(3, ""); DN_ACC_ROW(4, "");             \
        DN_ACC_ROW(5, ""); DN_ACC_ROW(6, ""); DN_ACC_ROW(7, "");                                \
    } while (0)
#define DN_WAIT_A(N, S, Q)                                                                    \
    asm volatile("s_waitcnt lgkmcnt(" #N ")"                                                  \
                 : "+v"(af[S][0]), "+v"(af[S][1]), "+v"(af[S][2]), "+v"(af[S][3]),             \
                   "+v"(af[S][4]), "+v"(af[S][5]), "+v"(af[S][6]), "+v"(af[S][7]), "+v"(bq[Q]))

template <bool C16, bool NTC>
__global__ __launch_bounds__(D_NT) void gemm_bf16_w4dn_kernel(const unsigned short *__restrict__ A,
                                                              const unsigned short *__restrict__ B,
                                                              unsigned short *__restrict__ C, int M,
                                                              int N, int Kd, int tiles_m, int tiles_n)
{
    // A stages at LDS bytes 0 and 32768, B stages at 65536 and 98304
    __shared__ __attribute__((aligned(1024))) unsigned short L[4 * D_ELEMS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave >> 1, wj = wave & 1;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const long long m0 = (long long)tm * TM, n0 = (long long)tn * TN;
    const __amdgpu_buffer_rsrc_t rA =
        __builtin_amdgcn_make_buffer_rsrc((void *)(A + m0 * Kd), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB =
        __builtin_amdgcn_make_buffer_rsrc((void *)(B + n0), (short)0, 0x7fffffff, 0x00020000);
    const unsigned lb = (unsigned)(size_t)(const __attribute__((address_space(3))) unsigned short *)L;

    // load q (0..15) of a stage: q < 8: A rows 64 wave + 8q (as the [N, Kd]
    // kernel); q >= 8: B k rows r = 16 wave + 2 (q - 8) + h, h = lane / 32, the
    // lane's LDS chunk p = lane % 32 holding global chunk p ^ (4 (r % 4) + 2 ((r / 8) % 2))
    const int lr = lane >> 3;
    const int voff = lr * Kd * 2 + (((lane & 7) ^ lr) << 4);
    const int hb = lane >> 5;
    const int vbh = hb * N * 2, vbc = lane & 31;
    auto dtl = [&](int buf, int k0, int q) __attribute__((always_inline)) {
        if (q < 8) {
            const int row0 = wave * 64 + q * 8;
            const int so = __builtin_amdgcn_readfirstlane((row0 * Kd + k0) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void *)(L + buf * D_ELEMS + row0 * D_TK), 16, voff, so, 0, 0);
        } else {
            const int qq = q - 8, r0 = wave * 16 + 2 * qq;
            const int so = __builtin_amdgcn_readfirstlane((k0 + r0) * N * 2);
            const int vb = vbh + 16 * (vbc ^ (8 * (qq & 1) + 4 * hb + 2 * (qq >> 2)));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void *)(L + (2 + buf) * D_ELEMS + r0 * TN), 16, vb, so, 0, 0);
        }
    };

    // A fragment x of k step ks: row wi*128 + 16x + lane % 16, chunk 4 ks +
    // lane / 16, stored at chunk ^ (row % 8)
    const unsigned aa0 = lb + (wi * 128 + (lane & 15)) * 128 + 16 * ((lane >> 4) ^ (lane & 7));
    const unsigned aa1 = lb + (wi * 128 + (lane & 15)) * 128 + 16 * ((4 + (lane >> 4)) ^ (lane & 7));
    // B fragment of column block b (columns wj*128 + 16b ..) in k step ks:
    // lane group g = lane / 16 covers k 8g .. 8g + 7; lane m = lane % 16
    // addresses k row 8g + m / 4 (+4 for the second read) at columns 4 (m % 4)
    // .. + 3, which sit 32 (b ^ s) + 16 ((m % 4) / 2) + 8 (m % 2) bytes into the
    // row's 256-byte half wj, s = 2 (m / 4) + g % 2
    const int g = lane >> 4, mm = lane & 15, e = mm >> 2, h4 = mm & 3;
    const int sx = 2 * e + (g & 1);
    const unsigned bb = lb + 65536 + 512 * (8 * g + e) + 256 * wj + 16 * (h4 >> 1) + 8 * (h4 & 1);

    // af[ks][x]: A fragments of k step ks; bq[G]: B fragment of block G = 8 ks + b
    bf16x8 af[2][8], bq[16];
    auto rdA = [&](int set, int buf, int x) __attribute__((always_inline)) {
        af[set][x] = lds_read_b128((set ? aa1 : aa0) + buf * 32768 + x * 2048);
    };
    auto rdB = [&](int G, int buf, int hi) __attribute__((always_inline)) {
        const int ks = G >> 3, b = G & 7;
        const i16x4 v = lds_read_tr_b64(bb + ((unsigned)(b ^ sx) << 5) + buf * 32768 + ks * 16384 + hi * 2048);
        i16x8 w = __builtin_bit_cast(i16x8, bq[G]);
        if (hi) { w[4] = v[0]; w[5] = v[1]; w[6] = v[2]; w[7] = v[3]; }
        else    { w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3]; }
        bq[G] = __builtin_bit_cast(bf16x8, w);
    };
    f32x4 acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{};
    DN_ACC_FENCE();

    const int stages = Kd / D_TK;
    const int last = (stages - 1) * D_TK;
    // Block G (0..15) of stage t from buffer buf (literal): 8 MFMAs, one per
    // row block. LDS reads issued in block G: G < 8: A fragment G of step 1 and
    // the B fragment of block G + 2; 8 <= G < 14: the B fragment of block G + 2;
    // G = 14, 15: A fragments 4 (G - 14) .. + 3 of stage t + 1's step 0 and its
    // B fragment of block G - 14, from buf ^ 1. The wait at the start of a
    // block counts the reads issued after the ones it needs (3 per block in
    // step 0, 2 in step 1). k1: k of stage t + 1 (its loads 6..15 go into buf
    // ^ 1 during step 0); k2: k of stage t + 2 (its loads 0..5 go into buf after
    // the barrier).
    auto block = [&](int buf, int k1, int k2, int G) __attribute__((always_inline)) {
        const int ks = G >> 3, b = G & 7;
        if (G == 0) DN_WAIT_A(2, 0, 0);
        else if (G == 8) DN_WAIT_A(2, 1, 8);
        else if (G < 8) asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(bq[G]));
        else if (G <= 13) asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(bq[G]));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = 8 * G + j;
            if (G < 8) {
                if (j == 0) rdA(1, buf, G);
                else if (j <= 2) rdB(G + 2, buf, j - 1);
            } else if (G < 14) {
                if (j <= 1) rdB(G + 2, buf, j);
            } else {
                if (j < 4) rdA(0, buf ^ 1, 4 * (G - 14) + j);
                else if (j <= 5) rdB(G - 14, buf ^ 1, j - 4);
            }
            if (i >= 2 && i < 32 && (i - 2) % 3 == 0) dtl(buf ^ 1, k1, 6 + (i - 2) / 3);
            if (i >= 112 && (i - 112) % 3 == 0) dtl(buf, k2, (i - 112) / 3);
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                         : "+a"(acc[j][b]) : "v"(bq[G]), "v"(af[ks][j]));
            W4_FENCE();
        }
        if (G == 13) {
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bq[12]), "+v"(bq[13]), "+v"(bq[14]), "+v"(bq[15]));
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of stage t + 1 landed
            __syncthreads();
            W4_FENCE();
        }
    };
    auto stage = [&](int buf, int k1, int k2) __attribute__((always_inline)) {
#pragma unroll
        for (int G = 0; G < 16; ++G) block(buf, k1, k2, G);
    };
#pragma unroll
    for (int q = 0; q < 16; ++q) dtl(0, 0, q);
#pragma unroll
    for (int q = 0; q < 6; ++q) dtl(1, min(D_TK, last), q);
    __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6): this wave's loads of stage 0 landed
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 8; ++x) rdA(0, 0, x);
    rdB(0, 0, 0);
    rdB(0, 0, 1);
    rdB(1, 0, 0);
    rdB(1, 0, 1);
    W4_FENCE();
    // an even number of stages (the launcher's condition); past the end the
    // loads repeat the last stage into a buffer no MFMA reads again
    for (int s = 0; s < stages; s += 2) {
        stage(0, min((s + 1) * D_TK, last), min((s + 2) * D_TK, last));
        stage(1, min((s + 2) * D_TK, last), min((s + 3) * D_TK, last));
    }
    // the reads issued for the stage past the end land before their registers
    // are reused, and the loads before the workgroup's LDS is released
    DN_WAIT_A(0, 0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bq[1]));
    __builtin_amdgcn_s_waitcnt(0x0F70);
    DN_ACC_FENCE();
    // C through a buffer descriptor on the tile's first element
    const __amdgpu_buffer_rsrc_t rC =
        __builtin_amdgcn_make_buffer_rsrc((void *)(C + m0 * N + n0), (short)0, 0x7fffffff, 0x00020000);
    const int el = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    store_c_tr<C16, NTC>(acc, rC, N, wi, wj, el);
}
#undef DN_ACC_ROW
#undef DN_ACC_FENCE
#undef DN_WAIT_A

// ------------------------------------------------------ any-shape kernel

// 64x64 tile of C per workgroup of 4 waves (2x2 blocks of 32x32); every lane
// gathers its 8 A and 8 B operand values of each 16-wide k step with guarded
// 2-byte loads (zero past M, N or Kd), so any shape and any element alignment
// works. Same MFMA sequence as the kernels above.
template <bool BKN>
__global__ __launch_bounds__(256) void gemm_bf16_any_kernel(const unsigned short *__restrict__ A,
                                                            const unsigned short *__restrict__ B,
                                                            unsigned short *__restrict__ C,
                                                            long long M, long long N, long long Kd,
                                                            long long tiles_n)
{
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
    const long long i = tm * 64 + (wave >> 1) * 32 + (lane & 31);
    const long long j = tn * 64 + (wave & 1) * 32 + (lane & 31);
    const int kq = 8 * (lane >> 5);
    f32x16 acc = f32x16{};
    for (long long k0 = 0; k0 < Kd; k0 += 16) {
        u16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const long long k = k0 + kq + e;
            const bool kin = k < Kd;
            a[e] = (kin && i < M) ? A[i * Kd + k] : (unsigned short)0;
            b[e] = (kin && j < N) ? (BKN ? B[k * N + j] : B[j * Kd + k]) : (unsigned short)0;
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const long long gi = tm * 64 + (wave >> 1) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const long long gj = tn * 64 + (wave & 1) * 32 + (lane & 31);
        if (gi < M && gj < N) C[gi * N + gj] = f32_to_bf16_rne(acc[r]);
    }
}

template <int TK, bool EARLY, bool BKN>
void launch_tk(const void *a, const void *b, void *c, int M, int N, int Kd, int tm, int tn,
               hipStream_t st)
{
    const bool edge = (M % TM) || (N % TN) || (Kd % TK);
    const unsigned grid = (unsigned)tm * (unsigned)tn;
    const auto *A = (const unsigned short *)a;
    const auto *B = (const unsigned short *)b;
    auto *C = (unsigned short *)c;
    if (edge)
        hipLaunchKernelGGL((gemm_bf16_kernel<true, TK, EARLY, BKN>), dim3(grid), dim3(NT), 0, st, A, B, C, M, N, Kd, tm, tn);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<false, TK, EARLY, BKN>), dim3(grid), dim3(NT), 0, st, A, B, C, M, N, Kd, tm, tn);
}

template <bool BKN>
hipError_t launch_layout(const void *a, const void *b, void *c, long long M, long long N,
                         long long Kd, int variant, hipStream_t st)
{
    // rows of A (and of B) must be 16-byte aligned for the staged kernels
    const bool rows16 = ((uintptr_t)a & 15) == 0 && ((uintptr_t)b & 15) == 0 && Kd % 8 == 0 &&
                        (!BKN || N % 8 == 0);
    if (!rows16) {
        const long long tm = (M + 63) / 64, tn = (N + 63) / 64;
        if (tm * tn > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((gemm_bf16_any_kernel<BKN>), dim3((unsigned)(tm * tn)), dim3(256), 0, st,
                           (const unsigned short *)a, (const unsigned short *)b, (unsigned short *)c,
                           M, N, Kd, tn);
        return hipGetLastError();
    }
    if (M > 0x7fffffffLL || N > 0x7fffffffLL || Kd > 0x7fffffffLL) return hipErrorInvalidValue;
    const long long tm = (M + TM - 1) / TM, tn = (N + TN - 1) / TN;
    if (tm * tn > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // the 4-wave kernels: whole tiles only, byte offsets from their buffer
    // descriptors' bases (a tile's 256 rows of A, 512 * Kd bytes; an
    // n-contiguous B's Kd rows, 2 * Kd * N bytes) within 31 bits, and a k range
    // long enough that the main loop outweighs the per-tile prologue and
    // epilogue, which one wave per SIMD cannot overlap with another workgroup's
    // MFMAs. The register-staged kernel from kk = 1024 (measured against the
    // 8-wave kernel: 1.2x at 8192^3, 1.08x at kk = 1536, 1.02-1.07x at 1024,
    // 0.93x at 512, 0.8x at 256); the direct-to-LDS kernels (an even number of
    // k stages) from kk = 256 for B [k, n] (at 4096 x 14336: 0.87-0.90x the
    // 8-wave kernel's time at kk = 256, 0.83x at 384, 0.81x at 512) and from
    // kk = 384 for B [n, k] (0.98-1.04x at 256, 0.94x at 384, 0.88x at 512;
    // 1.12x at 128)
    const bool whole = variant == kGemmFast && M % TM == 0 && N % TN == 0 && 512 * Kd < 0x7fffffffLL &&
                       (BKN ? 2 * Kd * N < 0x7fffffffLL : true);
    const bool w4 = whole && Kd % W4_TK == 0 && Kd >= kW4MinK;
    const bool direct = whole && Kd % (2 * D_TK) == 0 && Kd >= (BKN ? kDirectMinK : kDirectMinKNk) &&
                        512 * N < 0x7fffffffLL;
    // the direct-to-LDS kernels: C in 16-byte stores where C is 16-byte aligned
    // and N a multiple of 8, nontemporal from kk = 8192, else in 2-byte stores
    // (512 N bytes cover a tile's rows of C)
    const bool c16 = ((uintptr_t)c & 15) == 0 && N % 8 == 0, ntc = Kd >= kNtcMinK;
    const auto *A = (const unsigned short *)a;
    const auto *B = (const unsigned short *)b;
    auto *C = (unsigned short *)c;
    const dim3 grid((unsigned)(tm * tn));
    if (direct && BKN) {
        auto *kern = c16 ? (ntc ? gemm_bf16_w4dn_kernel<true, true> : gemm_bf16_w4dn_kernel<true, false>)
                         : gemm_bf16_w4dn_kernel<false, false>;
        hipLaunchKernelGGL(kern, grid, dim3(D_NT), 0, st, A, B, C, (int)M, (int)N, (int)Kd, (int)tm, (int)tn);
    } else if (direct && !BKN) {
        auto *kern = c16 ? (ntc ? gemm_bf16_w4d_kernel<true, true> : gemm_bf16_w4d_kernel<true, false>)
                         : gemm_bf16_w4d_kernel<false, false>;
        hipLaunchKernelGGL(kern, grid, dim3(D_NT), 0, st, A, B, C, (int)M, (int)N, (int)Kd, (int)tm, (int)tn);
    } else if (w4) {
        hipLaunchKernelGGL(gemm_bf16_w4_kernel<BKN>, dim3((unsigned)(tm * tn)), dim3(W4_NT), 0, st,
                           (const unsigned short *)a, (const unsigned short *)b, (unsigned short *)c,
                           (int)M, (int)N, (int)Kd, (int)tm, (int)tn);
    } else if (variant == kGemmShareCU) {
        launch_tk<32, true, BKN>(a, b, c, (int)M, (int)N, (int)Kd, (int)tm, (int)tn, st);
    } else {
        launch_tk<64, true, BKN>(a, b, c, (int)M, (int)N, (int)Kd, (int)tm, (int)tn, st);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const void *a, const void *b, void *c, long long M, long long N,
                            long long Kd, int variant, bool b_kn, hipStream_t st)
{
    return b_kn ? launch_layout<true>(a, b, c, M, N, Kd, variant, st)
                : launch_layout<false>(a, b, c, M, N, Kd, variant, st);
}

}  // namespace dps
