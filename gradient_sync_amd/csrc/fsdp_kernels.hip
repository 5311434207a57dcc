// Backward half of the FSDP layer step in one launch: every rank's weight
// gradient dW_r = x_r^T . dy_r and its ReduceScatter back to the row shards
// ("Sharding and Parallelism", section "FSDP and ZeRO": the backward pass
// produces the gradient of the gathered weight and reduce-scatters it so each
// rank keeps the rows it owns; section "The cost of the inserted collectives":
// the collective that follows the dot).
//
// A workgroup owns one 32x32 block (rows i0.., columns j0..) of the [d, f]
// gradient for all K ranks: wave r computes rank r's block with
// v_mfma_f32_32x32x2f32 over the m tokens in ascending order (the same chain as
// the stand-alone GEMM, so dW_r has the same bits), writes it to dw_full[r] and
// to LDS, and after one barrier the workgroup folds the K blocks in the ring
// order of the block's shard into dw_shard (the same fold as the ReduceScatter
// kernel, so the shard has the same bits as ReduceScatter(dw_full)). One launch
// replaces a GEMM launch and a ReduceScatter launch, and the K blocks are
// folded from LDS instead of being read back from HBM.
//
// The MFMA operands come straight from global memory into registers: for a k
// pair, lanes 0-31 read x_r[k][i0 .. i0+31] and lanes 32-63 x_r[k+1][...] (two
// 128-byte rows), and the same for dy_r, which is already the operand layout
// of the 32x32x2 instruction (A[i][k] = x[k][i], B[k][j] = dy[k][j]):
//   A operand: A[i = l % 32][k = l / 32]      B operand: B[k = l / 32][j = l % 32]
//   D register q: D[i = 8*(q/4) + 4*(l/32) + q%4][j = l % 32]
#include "gemm_f32_tile.h"

namespace dps {
namespace {

using f32tile::f32x16;

constexpr int FB = 32;       // block edge
constexpr int FQ = 16;       // k pairs per chunk of operands

// Block id of the backward half for NTH threads (NTH >= 64 K; waves K.. only
// join the fold). P is FsdpBwdParams or a struct with the same fields. T: the
// caller's LDS, K blocks of 32x32 floats (rank r's block, element i*32 + j).
template <int K, int NTH, class P>
__device__ __forceinline__ void fsdp_bwd_block(const P &p, const long long id,
                                               float (*__restrict__ T)[FB * FB])
{
    const int lane = threadIdx.x & 63;
    const int r = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long nbj = p.f / FB;
    const long long i0 = (id / nbj) * FB, j0 = (id % nbj) * FB;
    const long long kh = lane >> 5, col = lane & 31;

    if (r < K) {
        const float *__restrict__ x = p.x[r] + kh * p.d + i0 + col;
        const float *__restrict__ dy = p.dy[r] + kh * p.f + j0 + col;
        // chunks of FQ k pairs: a chunk's 2*FQ operand loads are issued
        // together, then its FQ MFMAs run (two waves per SIMD overlap one
        // wave's loads with the other's MFMAs; keeping 2 or 4 chunks in flight
        // per wave measured slower, chunks of 4 to 32 pairs the same)
        const long long chunks = p.m / (2 * FQ);
        f32x16 acc = {};
        for (long long c = 0; c < chunks; ++c) {
            float a[FQ], b[FQ];
#pragma unroll
            for (int q = 0; q < FQ; ++q) {
                const long long k = (c * FQ + q) * 2;
                a[q] = x[k * p.d];
                b[q] = dy[k * p.f];
            }
            // keep the scheduler from moving the loads down next to their MFMAs
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < FQ; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
        }
        float *__restrict__ dwf = p.dw_full[r];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = 8 * (q >> 2) + 4 * (int)kh + (q & 3);
            dwf[(i0 + i) * p.f + j0 + col] = acc[q];
            T[r][i * FB + col] = acc[q];
        }
    }
    __syncthreads();

    // shard c holds rows c*R ..; its fold visits ranks c+1, c+2, ..., c (mod K)
    const int c = (int)(i0 / p.R);
    float *__restrict__ out = p.dw_shard[c] + (i0 - (long long)c * p.R) * p.f + j0;
    for (int e = threadIdx.x; e < FB * FB; e += NTH) {
        int rr = c + 1 >= K ? c + 1 - K : c + 1;
        float s = T[rr][e];
#pragma unroll
        for (int m = 1; m < K; ++m) {
            rr = rr + 1 >= K ? 0 : rr + 1;
            s = s + T[rr][e];
        }
        out[(e / FB) * p.f + (e % FB)] = s;
    }
}

// Forward block with the AllGather folded in: one workgroup (8 waves) computes a
// 32x32 block (rows i0.., columns j0..) of y_r = x_r . W. The block's 32 rows of
// x_r are loaded into LDS once, k-major (Xs[k][i], odd row pitch: the 4-byte
// stores of consecutive k and the reads of 32 consecutive i are free of bank
// conflicts); wave w then runs the MFMA chain over its eighth of the k range
// with the B operand read straight from W's row shards into registers (lanes
// 0-31 and 32-63 read 128-byte row pieces of W, the 32x32x2 operand layout),
// and the eight partial blocks are added through LDS in wave order. There is
// no k-stage loop, so no per-stage barrier and LDS round trip. Wave w of block
// row it also writes the W rows it loaded to the gathered copy w_full[r] when
// w mod (m/32) == it, so every W element is written once per rank.
constexpr int XP = FB + 1;   // LDS row pitch of the x block (floats)

template <class P>
__device__ __forceinline__ void fsdp_fwd_block(const P &p, const int id, float *__restrict__ smem)
{
    const int K = p.nb;
    const int r = id % K;                     // with K = 8 a rank's blocks share an XCD
    const long long t = id / K;
    const long long nbj = p.N / FB, nbi = p.M / FB;
    const long long it = t / nbj, i0 = it * FB, j0 = (t % nbj) * FB;
    const long long Kd = p.Kd, N = p.N;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long kh = lane >> 5, col = lane & 31;

    // x_r[i0 .. i0+31][0 .. Kd-1] -> Xs[k][i]: thread k loads column k of the
    // block (Kd <= 512 threads), each row read by the workgroup as one
    // coalesced 4-byte-per-lane sweep
    // (buffer loads: one per-lane offset register, the row offset scalar)
    if (threadIdx.x < Kd) {
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.a[r] + i0 * Kd), (short)0, 0x7fffffff, 0x00020000);
        const int vo = (int)threadIdx.x * 4;
#pragma unroll
        for (int h = 0; h < FB; h += 16) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, vo, (int)((h + i) * Kd * 4), 0));
#pragma unroll
            for (int i = 0; i < 16; ++i) smem[threadIdx.x * XP + h + i] = v[i];
        }
    }
    __syncthreads();

    const long long span = Kd / 8, kb = w * span;
    float *__restrict__ wc = (w % nbi) == it ? p.b_copy[r] : nullptr;
    f32x16 acc = {};
    for (long long c0 = kb; c0 < kb + span; c0 += 2 * FQ) {
        // the chunk's 32 rows of W lie in one shard (R is a multiple of 32)
        const long long sh = c0 / p.b_rows;
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.b_shard[sh] + (c0 - sh * p.b_rows) * N + j0), (short)0, 0x7fffffff, 0x00020000);
        const int vo = (int)((kh * N + col) * 4);
        float b[FQ];
#pragma unroll
        for (int q = 0; q < FQ; ++q)
            b[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, vo, (int)(2 * q * N * 4), 0));
        __builtin_amdgcn_sched_barrier(0);
        if (wc) {
            const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(wc + c0 * N + j0), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
            for (int q = 0; q < FQ; ++q)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, b[q]), rc, vo, (int)(2 * q * N * 4), 0);
        }
#pragma unroll
        for (int q = 0; q < FQ; ++q) {
            const float a = smem[(c0 + 2 * q + kh) * XP + col];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b[q], acc, 0, 0, 0);
        }
    }
    __syncthreads();
    // partial blocks of the 8 waves, added in wave order
#pragma unroll
    for (int q = 0; q < 16; ++q) smem[(w * 16 + q) * 64 + lane] = acc[q];
    __syncthreads();
    float *__restrict__ y = p.c[r];
    for (int e = threadIdx.x; e < 16 * 64; e += 512) {
        const int q = e >> 6, l = e & 63;
        float s = smem[q * 64 + l];
#pragma unroll
        for (int v = 1; v < 8; ++v) s = s + smem[(v * 16 + q) * 64 + l];
        const int i = 8 * (q >> 2) + 4 * (l >> 5) + (q & 3), j = l & 31;
        y[(i0 + i) * N + j0 + j] = s;
    }
}

template <class P>
bool fwd_direct_ok(const P &p)
{
    // whole 32x32 blocks, k split in 8 waves of whole 32-deep chunks, each chunk
    // inside one shard, and one thread per k for the x block (Kd <= 512, which
    // also keeps the block's LDS at 66 KiB: two workgroups per CU)
    return p.M % FB == 0 && p.N % FB == 0 && p.Kd % (8 * 2 * FQ) == 0 && p.Kd <= 512 &&
           p.b_rows % (2 * FQ) == 0 && p.N <= (1 << 20);   // buffer offsets in 31 bits
}

template <int K>
__global__ __launch_bounds__(64 * K) void fsdp_bwd_kernel(const FsdpBwdParams p)
{
    __shared__ float T[K][FB * FB];
    fsdp_bwd_block<K, 64 * K>(p, (long long)blockIdx.x, T);
}

// The whole layer step in one launch, three kinds of workgroups: tiles of the
// input gradient dx = dy . W^T (W's rows read from the shards as the columns
// of W^T; n_dx of them, none without dx), blocks of the backward weight
// gradient with its ReduceScatter, and 32x32 blocks of the forward dot with
// the AllGather folded in (fsdp_fwd_block: W's rows read from the shards, the
// gathered copy written as it is loaded; n_fwd of them). The parts share no data, so they run
// side by side on the CUs instead of one after the other; the ReduceScatter of
// dW overlaps the dx dot (the FSDP backward overlap). A workgroup runs one
// part, so the parts share one LDS allocation.
// DX: with the dx tiles. Their 16 dependent k stages are then the long pole,
// and the forward runs as the same 64x64 k-stage tiles (34 KiB of LDS, so
// more workgroups fit beside the dx tiles); without dx, the forward runs as
// fsdp_fwd_block (66 KiB: the x block in LDS, no k-stage loop), which is
// shorter alone (22.8 against 26.2 us for the step; with dx 26.5 against 29.0
// the other way round).
template <int K, bool DX>
__global__ __launch_bounds__(512) void fsdp_step_kernel(const FsdpStepParams p)
{
    using namespace f32tile;
    constexpr int kOp = 2 * BK * LDP;                    // floats of one operand's buffers
    constexpr int kA = 2 * kOp > K * FB * FB ? 2 * kOp : K * FB * FB;
    constexpr int kWords = DX ? kA : (kA > 512 * XP ? kA : 512 * XP);
    __shared__ __attribute__((aligned(16))) float smem[kWords];
    auto As = reinterpret_cast<float (*)[BK][LDP]>(smem);
    auto Bs = reinterpret_cast<float (*)[BK][LDP]>(smem + kOp);
    // longest parts first, so the workgroup dispatcher starts them first and
    // the short forward blocks fill in behind them: the dx tiles (16 dependent
    // k stages each), the backward blocks, then the forward blocks
    const int id = (int)blockIdx.x;
    const int n_bwd = (int)((p.bwd.d / FB) * (p.bwd.f / FB));
    if (id < p.n_dx)
        gemm_f32_tile<2, 512, true, 2>(p.dx, p.tiles_x_dx, id, As, Bs);
    else if (id < p.n_dx + n_bwd)
        fsdp_bwd_block<K, 512>(p.bwd, (long long)id - p.n_dx,
                               reinterpret_cast<float (*)[FB * FB]>(smem));
    else if (DX)
        gemm_f32_tile<0, 512, true, 1>(p.fwd, p.tiles_x, id - p.n_dx - n_bwd, As, Bs);
    else
        fsdp_fwd_block(p.fwd, id - p.n_dx - n_bwd, smem);
}

// The FSDP step (without dx) in one wave of workgroups: G = max(n_fwd, n_bwd)
// workgroups of 8 waves, where n_fwd = (K*m/32)*(f/64) forward tiles of 32x64
// and n_bwd = (d/32)*(f/32) backward positions; with the fixture's shapes both
// are 256, one workgroup per CU, all resident from the start (no second round
// of workgroups). Every wave runs two independent MFMA chains side by side:
//   forward: a 32x32 block (column half w & 1 of the tile) over a quarter
//     (w >> 1) of the k range, A from the tile's x rows staged once in LDS
//     (k-major, odd pitch), B straight from W's row shards into registers; the
//     four quarter partials are added in quarter order through LDS. The waves
//     also write the W rows they load to the gathered copy w_full (each chunk
//     of 32 rows by one tile row of each rank, so each element once per rank);
//   backward: rank w's 32x32 block of dW_w = x_w^T dy_w over the tokens in
//     ascending pairs (the same chain as the stand-alone GEMM, so the same
//     bits), written to dw_full[w] and to LDS; after one barrier the block's K
//     rank blocks are folded in the ring order of its shard into dw_shard (the
//     ReduceScatter's fold, same bits).
// Operands move in chunks of 16 k pairs, the next chunk's loads issued before
// the current chunk's MFMAs. Workgroup ids go round-robin over the 8 XCDs; the
// tiles are permuted so that an XCD's workgroups take one rank's forward tiles
// (its x rows and all of W in that XCD's L2) and adjacent backward positions.
// The outputs (y, the gathered W copies, dw_full, dw_shard) are stored with the
// nontemporal hint: nothing in the launch reads them back, and ordinary stores
// leave them dirty in L2 to be written back when the kernel ends (K = 8, 128
// tokens, d = f = 512: 21.2 against 19.8 us).
constexpr int S2_XP = FB + 1;     // LDS pitch of the x block (floats)
constexpr int kNtAux = 2;         // cache-policy bits of a buffer store: nontemporal

__device__ __forceinline__ long long xcd_major(long long id, long long n, long long grid)
{
    return (grid == n && n % 8 == 0) ? (id % 8) * (n / 8) + id / 8 : id;
}

template <int K>
__global__ __launch_bounds__(512) void fsdp_step2_kernel(const FsdpStepParams p)
{
    const FsdpFwd8 &fw = p.fwd;
    const FsdpBwd8 &bw = p.bwd;
    const long long m = bw.m, d = bw.d, f = bw.f, R = bw.R;
    const long long grid = gridDim.x;
    const long long n_bwd = (d / FB) * (f / FB);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long kh = lane >> 5, col = lane & 31;
    __shared__ float Xs[512 * S2_XP];          // forward tile's x rows, k-major
    __shared__ float Pf[8][16 * 64];            // forward partial blocks
    __shared__ float T[K][FB * FB];             // backward rank blocks

    // ---- forward tile
    const bool has_f = blockIdx.x < p.n_fwd;
    const long long tf = has_f ? xcd_major(blockIdx.x, p.n_fwd, grid) : 0;
    const long long nbj2 = f / 64, rows_per_rank = m / FB;
    const long long trow = tf / nbj2, jb = tf % nbj2;
    const int rf = (int)(trow / rows_per_rank);
    const long long it = trow % rows_per_rank;
    const long long jf = jb * 64 + (w & 1) * FB;            // this wave's 32 columns
    const long long pq = d / 8;                              // k pairs per quarter
    const long long pf0 = (w >> 1) * pq;                     // first k pair of the quarter
    // ---- backward position
    const bool has_b = blockIdx.x < n_bwd && w < K;
    const long long tb = blockIdx.x < n_bwd ? xcd_major(blockIdx.x, n_bwd, grid) : 0;
    const long long i0 = (tb / (f / FB)) * FB, j0 = (tb % (f / FB)) * FB;

    // x rows of the forward tile: thread t loads column t of the 32 rows; they
    // go into LDS after the backward chain's first chunk, which does not need
    // them, so the loads' latency is spent on MFMAs
    const bool xcol = has_f && (long long)threadIdx.x < d;
    float xv[FB];

    const long long nfc = has_f ? pq / FQ : 0;               // forward chunks
    const long long nbc = has_b ? m / (2 * FQ) : 0;          // backward chunks
    const long long nc = nfc > nbc ? nfc : nbc;
    // Buffer descriptors on this wave's columns: a lane's offset is fixed
    // (row kh, column col) and a load's row offset is a scalar. The backward
    // operands of rank w: x_w[.][i0 + col] and dy_w[.][j0 + col]; byte offsets
    // stay below 2^31 (checked by the launcher).
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(has_b ? bw.x[w] + i0 : bw.x[0]), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(has_b ? bw.dy[w] + j0 : bw.dy[0]), (short)0, 0x7fffffff, 0x00020000);
    const int vox = (int)((kh * d + col) * 4), voy = (int)((kh * f + col) * 4);
    const int vow = (int)((kh * f + jf + col) * 4);
    // staging: two sets (chunk parity) of FQ forward B values and FQ pairs of
    // backward operands per lane
    float fb0[FQ], ba0[FQ], bb0[FQ], fb1[FQ], ba1[FQ], bb1[FQ];
    auto load = [&](long long c, float (&fb)[FQ], float (&ba)[FQ], float (&bb)[FQ], int parts = 3)
        __attribute__((always_inline)) {
        if ((parts & 1) && c < nfc) {
            // W rows 2*(pf0 + c*FQ) .. + 31 lie in one shard
            const long long k0 = 2 * (pf0 + c * FQ);
            const long long sh = k0 / R;
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(fw.b_shard[sh] + (k0 - sh * R) * f), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
            for (int q = 0; q < FQ; ++q)
                fb[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      rw, vow, (int)(2 * q * f * 4), 0));
        }
        if ((parts & 2) && c < nbc) {
#pragma unroll
            for (int q = 0; q < FQ; ++q) {
                const int k = (int)((c * FQ + q) * 2);
                ba[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      rx, vox, (int)(k * d * 4), 0));
                bb[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      rdy, voy, (int)(k * f * 4), 0));
            }
        }
    };
    // loads in the order their results are needed (vmcnt counts in order):
    // the backward operands of chunk 0, the x columns, the forward operands
    load(0, fb0, ba0, bb0, 2);
    __builtin_amdgcn_sched_barrier(0);
    if (xcol) {
        const float *xr = fw.a[rf] + it * FB * d + threadIdx.x;
#pragma unroll
        for (int i = 0; i < FB; ++i) xv[i] = xr[i * d];
    }
    __builtin_amdgcn_sched_barrier(0);
    load(0, fb0, ba0, bb0, 1);

    f32tile::f32x16 accf = {}, accb = {};
    if (nbc > 0) {
#pragma unroll
        for (int q = 0; q < FQ; ++q)
            accb = __builtin_amdgcn_mfma_f32_32x32x2f32(ba0[q], bb0[q], accb, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (xcol) {
#pragma unroll
        for (int i = 0; i < FB; ++i) Xs[threadIdx.x * S2_XP + i] = xv[i];
    }
    __syncthreads();                                         // the x block is in LDS
    load(1, fb1, ba1, bb1);

    // chunk cc from one staging set: the two chains' MFMAs alternate (each
    // depends only on the one two back), then the W rows go to the gathered
    // copy where this tile row writes them; bwd = false: the backward part of
    // the chunk is already done
    auto chunk = [&](long long cc, const float (&fb)[FQ], const float (&ba)[FQ],
                     const float (&bb)[FQ], bool bwd = true) __attribute__((always_inline)) {
        const bool on_b = bwd && cc < nbc, on_f = cc < nfc;
        const long long k0 = 2 * (pf0 + cc * FQ);
        const float *xs = &Xs[(k0 + kh) * S2_XP + col];
        if (on_b && on_f) {
#pragma unroll
            for (int q = 0; q < FQ; ++q) {
                accb = __builtin_amdgcn_mfma_f32_32x32x2f32(ba[q], bb[q], accb, 0, 0, 0);
                accf = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[2 * q * S2_XP], fb[q], accf, 0, 0, 0);
            }
        } else if (on_b) {
#pragma unroll
            for (int q = 0; q < FQ; ++q)
                accb = __builtin_amdgcn_mfma_f32_32x32x2f32(ba[q], bb[q], accb, 0, 0, 0);
        } else if (on_f) {
#pragma unroll
            for (int q = 0; q < FQ; ++q)
                accf = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[2 * q * S2_XP], fb[q], accf, 0, 0, 0);
        }
        if (on_f && (k0 / FB) % rows_per_rank == it) {
            const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(fw.b_copy[rf] + k0 * f), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
            for (int q = 0; q < FQ; ++q)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, fb[q]), rc, vow,
                                                      (int)(2 * q * f * 4), kNtAux);
        }
    };
    __builtin_amdgcn_sched_barrier(0);
    chunk(0, fb0, ba0, bb0, false);
    load(2, fb0, ba0, bb0);
    __builtin_amdgcn_sched_barrier(0);
    chunk(1, fb1, ba1, bb1);
    for (long long c = 2; c < nc; c += 2) {
        load(c + 1, fb1, ba1, bb1);
        __builtin_amdgcn_sched_barrier(0);
        chunk(c, fb0, ba0, bb0);
        load(c + 2, fb0, ba0, bb0);
        __builtin_amdgcn_sched_barrier(0);
        chunk(c + 1, fb1, ba1, bb1);
    }
    if (has_f) {
#pragma unroll
        for (int q = 0; q < 16; ++q) Pf[w][q * 64 + lane] = accf[q];
    }
    if (has_b) {
        float *__restrict__ dwf = bw.dw_full[w];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = 8 * (q >> 2) + 4 * (int)kh + (q & 3);
            __builtin_nontemporal_store(accb[q], &dwf[(i0 + i) * f + j0 + col]);
            T[w][i * FB + col] = accb[q];
        }
    }
    __syncthreads();
    if (has_f) {
        // y block (column half ch): the quarters' partials in quarter order
        float *__restrict__ y = fw.c[rf];
        for (int e = threadIdx.x; e < 2 * 16 * 64; e += 512) {
            const int ch = e >> 10, q = (e >> 6) & 15, l = e & 63;
            float s = Pf[ch][q * 64 + l];
#pragma unroll
            for (int h = 1; h < 4; ++h) s = s + Pf[2 * h + ch][q * 64 + l];
            const int i = 8 * (q >> 2) + 4 * (l >> 5) + (q & 3), j = l & 31;
            __builtin_nontemporal_store(s, &y[(it * FB + i) * f + jb * 64 + ch * FB + j]);
        }
    }
    if (blockIdx.x < n_bwd) {
        // shard c holds rows c*R ..; its fold visits ranks c+1, c+2, ..., c (mod K)
        const int c = (int)(i0 / R);
        float *__restrict__ out = bw.dw_shard[c] + (i0 - (long long)c * R) * f + j0;
        for (int e = threadIdx.x; e < FB * FB; e += 512) {
            int rr = c + 1 >= K ? c + 1 - K : c + 1;
            float s = T[rr][e];
#pragma unroll
            for (int mm = 1; mm < K; ++mm) {
                rr = rr + 1 >= K ? 0 : rr + 1;
                s = s + T[rr][e];
            }
            __builtin_nontemporal_store(s, &out[(e / FB) * f + (e % FB)]);
        }
    }
}

// The same step with every size fixed at compile time: K = 8 ranks of 128
// tokens, d = f = 512 (the layer of "Real HLO before and after partitioning":
// x[1024,512] and W[512,512] row-sharded over 8 devices). One workgroup per CU
// (256), each with the forward tile and the backward position of
// fsdp_step2_kernel and the same arithmetic, so the same bits; what differs is
// the order of the work and how the results leave:
//   1. the backward chain first: wave w's 64 MFMAs over rank w's tokens (the x
//      rows of the forward tile are loaded meanwhile and stored to LDS after
//      the first chunk), then the block goes to LDS and on to dw_full[w] as
//      16-byte row pieces, read back by the wave that wrote them;
//   2. one workgroup barrier (the x block complete), then the forward chain of
//      64 MFMAs over the wave's k quarter; the gathered copies of W are written
//      meanwhile, each workgroup copying one 32 KiB piece of W into one rank's
//      copy in 16-byte pieces (instead of the W rows its waves load);
//   3. the final barrier, then the y tile (quarter partials added in quarter
//      order) and the fold of the K rank blocks into dw_shard, both from LDS in
//      16-byte pieces.
// Every output store is nontemporal. All indices are compile-time shifts and
// masks (the runtime-shaped kernel spends about 3 us of this step in 64-bit
// index arithmetic). The launcher takes it only for these sizes and 16-byte
// aligned W shards and outputs.
namespace k8 {
constexpr int K = 8, M = 128, D = 512, F = 512, R = D / K;
constexpr int kPiece = 8192;               // floats of W one workgroup copies
constexpr int kGrid = (D / FB) * (F / FB);
static_assert((K * M / FB) * (F / 64) == kGrid, "a forward tile beside every backward position");
static_assert(K * (D * F / kPiece) == kGrid && R * F % kPiece == 0, "one piece of one W copy per workgroup");
static_assert(D == 512, "one thread per k column of the x block");
}

template <bool DX>
__global__ __launch_bounds__(512) void fsdp_step_k8_kernel(const FsdpStepParams p)
{
    using namespace k8;
    using f32tile::f32x4;
    const FsdpFwd8 &fw = p.fwd;
    const FsdpBwd8 &bw = p.bwd;
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int kh = lane >> 5, col = lane & 31;
    __shared__ float Xs[D * S2_XP];                                   // the tile's x rows, k-major
    __shared__ __attribute__((aligned(16))) float Pf[8][16 * 64];      // forward partial blocks
    __shared__ __attribute__((aligned(16))) float T[K][FB * FB];       // backward rank blocks

    const int b = blockIdx.x;
    const int tpos = (b % 8) * (kGrid / 8) + b / 8;                     // XCD-major
    const int trow = tpos / (F / 64), jb = tpos % (F / 64);
    const int rf = trow / (M / FB), it = trow % (M / FB);
    const int jf = jb * 64 + (w & 1) * FB, kq = (w >> 1) * (D / 4);
    const int i0 = (tpos / (F / FB)) * FB, j0 = (tpos % (F / FB)) * FB;

    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(bw.x[w] + i0), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(bw.dy[w] + j0), (short)0, 0x7fffffff, 0x00020000);
    const int vox = (kh * D + col) * 4, voy = (kh * F + col) * 4, vow = (kh * F + jf + col) * 4;
    // chunk c of the backward operands: token pairs 16c .. 16c+15
    auto loadb = [&](int c, float (&ba)[FQ], float (&bb)[FQ]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < FQ; ++q) {
            const int k = (c * FQ + q) * 2;
            ba[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, vox, k * D * 4, 0));
            bb[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, voy, k * F * 4, 0));
        }
    };
    // chunk c of the forward B operand: W rows kq + 32c .. + 31 (one shard)
    auto loadf = [&](int c, float (&fb)[FQ]) __attribute__((always_inline)) {
        const int k0 = kq + c * 2 * FQ;
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(fw.b_shard[k0 / R] + (k0 % R) * F), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int q = 0; q < FQ; ++q)
            fb[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, vow, 2 * q * F * 4, 0));
    };
    f32tile::f32x16 accb = {}, accf = {};
    auto mfb = [&](const float (&ba)[FQ], const float (&bb)[FQ]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < FQ; ++q) accb = __builtin_amdgcn_mfma_f32_32x32x2f32(ba[q], bb[q], accb, 0, 0, 0);
    };
    auto mff = [&](int c, const float (&fb)[FQ]) __attribute__((always_inline)) {
        const float *xs = &Xs[(kq + c * 2 * FQ + kh) * S2_XP + col];
#pragma unroll
        for (int q = 0; q < FQ; ++q)
            accf = __builtin_amdgcn_mfma_f32_32x32x2f32(xs[2 * q * S2_XP], fb[q], accf, 0, 0, 0);
    };
    float ba0[FQ], bb0[FQ], ba1[FQ], bb1[FQ], fb0[FQ], fb1[FQ], xv[FB];

    // 1. backward chain; the x block (thread t: column t of the tile's 32 rows)
    //    loads behind the first chunk's operands and goes to LDS after its MFMAs
    loadb(0, ba0, bb0);
    __builtin_amdgcn_sched_barrier(0);
    {
        const float *xr = fw.a[rf] + it * FB * D + t;
#pragma unroll
        for (int i = 0; i < FB; ++i) xv[i] = xr[i * D];
    }
    __builtin_amdgcn_sched_barrier(0);
    loadb(1, ba1, bb1);
    mfb(ba0, bb0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FB; ++i) Xs[t * S2_XP + i] = xv[i];
    loadb(2, ba0, bb0);
    __builtin_amdgcn_sched_barrier(0);
    mfb(ba1, bb1);
    loadb(3, ba1, bb1);
    __builtin_amdgcn_sched_barrier(0);
    mfb(ba0, bb0);
    loadf(0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mfb(ba1, bb1);
    loadf(1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    // dx = dy . W^T (DX): wave w's partial of the dx tile's column half w % 2
    // over the f quarter w / 2, in 4 chunks of 32 f. A k step pairs f0 + s
    // with f0 + 16 + s (s = 0..15), so each lane's operands are 16 consecutive
    // floats of one dy row and one W row: lane l loads row l % 32 at f0 + 16 (l / 32)
    // with four 16-byte loads per operand.
    const int fq = (w >> 1) * (F / 4), jd = jb * 64 + (w & 1) * FB;
    const float *dyr = bw.dy[rf] + (it * FB + col) * F + fq + 16 * kh;
    const float *wr = fw.b_shard[jd / R] + (jd % R + col) * F + fq + 16 * kh;
    auto loadx = [&](int c, f32x4 (&da)[4], f32x4 (&db)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            da[u] = *reinterpret_cast<const f32x4 *>(dyr + c * 32 + 4 * u);
            db[u] = *reinterpret_cast<const f32x4 *>(wr + c * 32 + 4 * u);
        }
    };
    [[maybe_unused]] f32x4 da0[4], db0[4], da1[4], db1[4];
    if constexpr (DX) loadx(0, da0, db0);
#pragma unroll
    for (int q = 0; q < 16; ++q) T[w][(8 * (q >> 2) + 4 * kh + (q & 3)) * FB + col] = accb[q];
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0): the wave's block is in LDS
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < FB * FB / 4 / 64; ++u) {
        const int e = (u * 64 + lane) * 4;
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4 *>(&T[w][e]),
                                    reinterpret_cast<f32x4 *>(&bw.dw_full[w][(i0 + e / FB) * F + j0 + e % FB]));
    }
    __syncthreads();                                    // the x block is in LDS

    // 2. forward chain, with this workgroup's piece of the gathered W copies
    f32x4 wcp[kPiece / 4 / 512];
    {
        const int pc = b / K;
        const float *src = fw.b_shard[pc / (R * F / kPiece)] + (pc % (R * F / kPiece)) * kPiece;
#pragma unroll
        for (int u = 0; u < kPiece / 4 / 512; ++u) wcp[u] = *reinterpret_cast<const f32x4 *>(src + (u * 512 + t) * 4);
    }
    // with DX, the dx chain's chunks alternate with the forward chain's (two
    // independent accumulators; each chunk's operands load behind the other
    // chain's MFMAs)
    [[maybe_unused]] f32tile::f32x16 accx = {};
    auto mfx = [&](const f32x4 (&da)[4], const f32x4 (&db)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 16; ++q)
            accx = __builtin_amdgcn_mfma_f32_32x32x2f32(da[q >> 2][q & 3], db[q >> 2][q & 3], accx, 0, 0, 0);
    };
    __builtin_amdgcn_sched_barrier(0);
    mff(0, fb0);
    loadf(2, fb0);
    if constexpr (DX) {
        loadx(1, da1, db1);
        __builtin_amdgcn_sched_barrier(0);
        mfx(da0, db0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mff(1, fb1);
    {
        float *dst = fw.b_copy[b % K] + (b / K) * kPiece;
#pragma unroll
        for (int u = 0; u < kPiece / 4 / 512; ++u)
            __builtin_nontemporal_store(wcp[u], reinterpret_cast<f32x4 *>(dst + (u * 512 + t) * 4));
    }
    loadf(3, fb1);
    if constexpr (DX) {
        loadx(2, da0, db0);
        __builtin_amdgcn_sched_barrier(0);
        mfx(da1, db1);
    }
    __builtin_amdgcn_sched_barrier(0);
    mff(2, fb0);
    if constexpr (DX) {
        loadx(3, da1, db1);
        __builtin_amdgcn_sched_barrier(0);
        mfx(da0, db0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mff(3, fb1);
    if constexpr (DX) {
        __builtin_amdgcn_sched_barrier(0);
        mfx(da1, db1);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) Pf[w][q * 64 + lane] = accf[q];
    __syncthreads();
    if constexpr (DX) {
        // every forward chain is done with the x block: its LDS takes the dx partials
        float *Px = Xs + w * (16 * 64);
#pragma unroll
        for (int q = 0; q < 16; ++q) Px[q * 64 + lane] = accx[q];
    }

    // 3. y tile: register q of lane l is row 8(q/4) + 4(l/32) + q%4, column l%32
    //    of column half ch; the quarters' partials in quarter order
    {
        const int ch = t >> 8, q = (t >> 4) & 15, l = (t & 15) * 4;
        f32x4 s = *reinterpret_cast<const f32x4 *>(&Pf[ch][q * 64 + l]);
#pragma unroll
        for (int h = 1; h < 4; ++h) s = s + *reinterpret_cast<const f32x4 *>(&Pf[2 * h + ch][q * 64 + l]);
        const int i = 8 * (q >> 2) + 4 * (l >> 5) + (q & 3), j = l & 31;
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4 *>(&fw.c[rf][(it * FB + i) * F + jb * 64 + ch * FB + j]));
    }
    if (t < FB * FB / 4) {
        // shard c holds rows c*R ..; its fold visits ranks c+1, c+2, ..., c (mod K)
        const int c = i0 / R, e = t * 4;
        int rr = c + 1 >= K ? c + 1 - K : c + 1;
        f32x4 s = *reinterpret_cast<const f32x4 *>(&T[rr][e]);
#pragma unroll
        for (int mm = 1; mm < K; ++mm) {
            rr = rr + 1 >= K ? 0 : rr + 1;
            s = s + *reinterpret_cast<const f32x4 *>(&T[rr][e]);
        }
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4 *>(
                                           &bw.dw_shard[c][(i0 - c * R + e / FB) * F + j0 + e % FB]));
    }
    if constexpr (DX) {
        // 4. the dx tile, from the partials in the x block's LDS
        __syncthreads();
        // dx tile: the quarters' partials in quarter order, as the y tile
        const int ch = t >> 8, q = (t >> 4) & 15, l = (t & 15) * 4;
        f32x4 s = *reinterpret_cast<const f32x4 *>(&Xs[ch * (16 * 64) + q * 64 + l]);
#pragma unroll
        for (int h = 1; h < 4; ++h) s = s + *reinterpret_cast<const f32x4 *>(&Xs[(2 * h + ch) * (16 * 64) + q * 64 + l]);
        const int i = 8 * (q >> 2) + 4 * (l >> 5) + (q & 3), j = l & 31;
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4 *>(&p.dx.c[rf][(it * FB + i) * D + jb * 64 + ch * FB + j]));
    }
}

template <int K>
hipError_t go_step2(const FsdpStepParams &p, long long grid, hipStream_t st)
{
    hipLaunchKernelGGL((fsdp_step2_kernel<K>), dim3((unsigned)grid), dim3(512), 0, st, p);
    return hipGetLastError();
}

template <int K>
hipError_t go(const FsdpBwdParams &p, hipStream_t st)
{
    const long long blocks = (p.d / FB) * (p.f / FB);
    hipLaunchKernelGGL((fsdp_bwd_kernel<K>), dim3((unsigned)blocks), dim3(64 * K), 0, st, p);
    return hipGetLastError();
}

template <int K>
hipError_t go_step(const FsdpStepParams &p, long long blocks, hipStream_t st)
{
    if (p.n_dx > 0)
        hipLaunchKernelGGL((fsdp_step_kernel<K, true>), dim3((unsigned)blocks), dim3(512), 0, st, p);
    else
        hipLaunchKernelGGL((fsdp_step_kernel<K, false>), dim3((unsigned)blocks), dim3(512), 0, st, p);
    return hipGetLastError();
}

}  // namespace

bool fsdp_fwd_direct_ok(const FsdpFwd8 &p) { return fwd_direct_ok(p); }

bool fsdp_step2_ok(int k, long long m, long long d, long long f)
{
    // the backward blocks' shape conditions, forward tiles of 32x64 with a k
    // quarter of whole 16-pair chunks, and the x rows of a tile in LDS (d <= 512)
    return fsdp_bwd_fusable(k, m, d, f) && f % 64 == 0 && d % 128 == 0 && d <= 512 &&
           (k * m / FB) * (f / 64) <= 0x7fffffffLL &&
           m * d * 4 < 0x7fffffffLL && m * f * 4 < 0x7fffffffLL && d * f * 4 < 0x7fffffffLL;
}

static bool aligned16(const void *q) { return ((uintptr_t)q & 15) == 0; }

bool fsdp_step_k8_ok(const FsdpStepParams &p)
{
    const int k = p.bwd.k;
    bool ok = k == k8::K && p.fwd.nb == k && p.bwd.m == k8::M && p.bwd.d == k8::D && p.bwd.f == k8::F &&
              p.bwd.R == k8::R;
    for (int r = 0; ok && r < k; ++r) {
        ok = aligned16(p.fwd.b_shard[r]) && aligned16(p.fwd.b_copy[r]) && aligned16(p.fwd.c[r]) &&
             aligned16(p.bwd.dw_full[r]) && aligned16(p.bwd.dw_shard[r]);
        if (p.n_dx != 0) ok = ok && aligned16(p.bwd.dy[r]) && aligned16(p.dx.c[r]);
    }
    return ok;
}

hipError_t launch_fsdp_step2(const FsdpStepParams &p, hipStream_t st)
{
    const int k = p.bwd.k;
    if (k < 1 || k > 8 || p.fwd.nb != k || (p.n_dx != 0 && !fsdp_step_k8_ok(p)) ||
        !fsdp_step2_ok(k, p.bwd.m, p.bwd.d, p.bwd.f) ||
        p.n_fwd != (k * p.bwd.m / FB) * (p.bwd.f / 64))
        return hipErrorInvalidValue;
    if (fsdp_step_k8_ok(p)) {
        if (p.n_dx != 0) hipLaunchKernelGGL(fsdp_step_k8_kernel<true>, dim3(k8::kGrid), dim3(512), 0, st, p);
        else hipLaunchKernelGGL(fsdp_step_k8_kernel<false>, dim3(k8::kGrid), dim3(512), 0, st, p);
        return hipGetLastError();
    }
    const long long n_bwd = (p.bwd.d / FB) * (p.bwd.f / FB);
    const long long grid = p.n_fwd > n_bwd ? p.n_fwd : n_bwd;
    switch (k) {
    case 1: return go_step2<1>(p, grid, st);
    case 2: return go_step2<2>(p, grid, st);
    case 3: return go_step2<3>(p, grid, st);
    case 4: return go_step2<4>(p, grid, st);
    case 5: return go_step2<5>(p, grid, st);
    case 6: return go_step2<6>(p, grid, st);
    case 7: return go_step2<7>(p, grid, st);
    default: return go_step2<8>(p, grid, st);
    }
}

bool fsdp_bwd_fusable(int k, long long m, long long d, long long f)
{
    // whole 32x32 blocks, no shard pad rows, each block inside one shard, whole
    // operand chunks, and at most 8 ranks (one wave per rank)
    return k >= 1 && k <= 8 && d % k == 0 && (d / k) % FB == 0 && f % FB == 0 &&
           m % (2 * FQ) == 0 && (d / FB) * (f / FB) <= 0x7fffffffLL;
}

hipError_t launch_fsdp_bwd_fused(const FsdpBwdParams &p, hipStream_t st)
{
    if (!fsdp_bwd_fusable(p.k, p.m, p.d, p.f)) return hipErrorInvalidValue;
    switch (p.k) {
    case 1: return go<1>(p, st);
    case 2: return go<2>(p, st);
    case 3: return go<3>(p, st);
    case 4: return go<4>(p, st);
    case 5: return go<5>(p, st);
    case 6: return go<6>(p, st);
    case 7: return go<7>(p, st);
    default: return go<8>(p, st);
    }
}

hipError_t launch_fsdp_step(const FsdpStepParams &p, hipStream_t st)
{
    const int k = p.bwd.k;
    if (k < 1 || k > 8 || p.fwd.nb != k || !fsdp_bwd_fusable(k, p.bwd.m, p.bwd.d, p.bwd.f))
        return hipErrorInvalidValue;
    // forward as 32x32 blocks without dx, as 64x64 tiles with it
    if (p.n_dx > 0 ? p.n_fwd != (p.fwd.M / 64) * (p.fwd.N / 64) * k || p.tiles_x != p.fwd.N / 64
                   : !fwd_direct_ok(p.fwd) || p.n_fwd != (p.fwd.M / FB) * (p.fwd.N / FB) * k ||
                         p.tiles_x != p.fwd.N / FB)
        return hipErrorInvalidValue;
    const long long blocks = (long long)p.n_fwd + p.n_dx + (p.bwd.d / FB) * (p.bwd.f / FB);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    switch (k) {
    case 1: return go_step<1>(p, blocks, st);
    case 2: return go_step<2>(p, blocks, st);
    case 3: return go_step<3>(p, blocks, st);
    case 4: return go_step<4>(p, blocks, st);
    case 5: return go_step<5>(p, blocks, st);
    case 6: return go_step<6>(p, blocks, st);
    case 7: return go_step<7>(p, blocks, st);
    default: return go_step<8>(p, blocks, st);
    }
}

}  // namespace dps
