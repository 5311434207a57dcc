// ReduceScatter and AllGather kernels for K ranks emulated as K HBM buffers.
//
// ReduceScatter (CMU 11-868 L14-L15 notes, "Ring AllReduce: ReduceScatter,
// then AllGather", phase 1; "Sharding and Parallelism", "The cost of the
// inserted collectives", T_RS,ring): shard c of the result is the sum over
// ranks of elements [cL, cL + n_c). On one GPU the ring's K-1 hops become K
// streaming reads of the same element range, folded in the order the ring
// would add them: rho_c = (c+1, ..., c+K-1, c) mod K, left fold, fp32
// accumulation (wrapping uint32 for int32).
//
// AllGather (same sources, phase 2 and T_AG,ring): every rank receives every
// shard's valid elements at their global offset.
//
// Both are HBM-bound streams: per 16-byte vector of shard elements the
// ReduceScatter reads K vectors and writes one; the AllGather reads one and
// writes K. The work is cut into tiles of one (sub-chunk, shard) segment, so
// the fold order rho_c and the alignment decision are uniform per tile; a
// persistent grid of workgroups walks the tiles. ReduceScatter inputs are read
// once, so they are loaded with the nontemporal hint. The per-shard phase
// table is kept in 32-bit words so that it is read with scalar loads.
//
// Where the K inputs and the output of a shard share their address
// phase modulo 16 bytes, the body of the tile moves 128-bit vectors (one
// global_load/store_dwordx4 per lane, consecutive lanes on consecutive
// vectors) and the unaligned head and the tail are done element by element;
// otherwise the tile is done element by element with consecutive lanes on
// consecutive elements (still coalesced).
#include "sync_internal.h"

#pragma clang fp contract(off)

namespace dps {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Tr;
template <> struct Tr<kF32>  { using Acc = float;    static constexpr int ES = 4, V = 4; };
template <> struct Tr<kBF16> { using Acc = float;    static constexpr int ES = 2, V = 8; };
template <> struct Tr<kI32>  { using Acc = unsigned; static constexpr int ES = 4, V = 4; };

// vectors per thread per tile
// One 16-byte vector per lane and rank in every ReduceScatter tile. In the
// fused ReduceScatter + AllGather launch this makes the two kinds' tiles the
// same size, so they pair up one for one across the grid (the pipelined layer
// step 1.3483 -> 1.3128 ms against 2 per lane, interleaved in one process).
template <int DT> struct RsU { static constexpr int U = 1; };
// The one-pass AllReduce stores each folded vector to all K outputs; there, too,
// one vector per lane and rank measured best (25M bf16, K=8: 72.1% of peak
// against 70.6% with 2 and 69.3% with 4).
constexpr int kArU = 1;
// The AllGather, too, stores each loaded vector K times; one vector per lane
// measured best (the pipelined layer step 1.3508 -> 1.3382 ms against 2).
constexpr int kAgU = 1;
// With a capped grid (dp_launch_opts_t.max_workgroups) a few resident
// workgroups walk many tiles, and two vectors per lane keep twice the loads in
// flight per workgroup (1 GiB/rank fp32 RS + AG on 256 workgroups: 3.78 ms
// against 4.01 with one; on the default grid one is faster: 3.42 against 3.53).
constexpr int kUCapped = 2;
constexpr int kAgBlock = 256;   // threads per AllGather workgroup
// AllGather shards are loaded with ordinary loads and the outputs stored with
// the nontemporal hint: with ordinary output stores the 400 MB a bucket's
// AllGather writes displace the next bucket's shards from the Infinity Cache
// (pipelined layer step 81.52% -> 74.70% of HBM peak).
// Default grid: one workgroup per tile (a wave that finishes its tile exits
// instead of waiting for its stores before loading the next tile); measured
// faster than persistent grids of 1, 2 or 4 workgroups per CU. A caller's
// dp_launch_opts_t.max_workgroups caps it instead.

// Where an AllGather reads the shards next, the ReduceScatter stores them with
// ordinary stores, which leave them in the caches (the 256 MB Infinity Cache
// holds a 25,000,000-value bf16 bucket's 50 MB of shards) where nontemporal
// stores do not: always in the fused ReduceScatter + AllGather launch of the
// bucket pipeline (its AllGather half reads the previous launch's shards), and
// in a ReduceScatter launched with cache_out (the two-phase AllReduce, the
// pipeline call's single phases) when the K shards together fit in
// kCacheOutBytes. Measured on MI355X, K = 8 bf16 layer step: pipelined 75.98%
// -> 78.59% of HBM peak (same bits). Every other ReduceScatter stores
// nontemporally: ordinary stores slowed the standalone kernel from 76.75 to
// 84.32 us per 25M bf16 bucket (K = 8). The store kind is a template
// parameter: chosen at run time inside the kernel, the two stores were merged
// into one ordinary store by the compiler.
constexpr long long kCacheOutBytes = 128ll << 20;

// Tile bodies start on a kAlign-byte boundary of the dominant stream: the K
// inputs for ReduceScatter, the K outputs for AllGather (anchoring the
// ReduceScatter on its output measured slower).
constexpr int kAlign = 128;
constexpr int kFastBit = 256;
constexpr int kOutAlignBit = 512;   // AllGather: the K outputs share one 16-byte phase

// Residency caps for launches over small shards. At full residency a launch
// keeps ~2,048 workgroups of 4 KiB tiles in flight (8 waves per SIMD on 256
// CUs); where a shard has fewer tiles than about twice that, the resident
// workgroups span two shards most of the time, and the write-heavy kernels then
// stream into twice as many output regions at once. Holding them to fewer
// workgroups per CU keeps them mostly within one shard. The cap is LDS the
// kernels never touch, reserved per workgroup at launch (160 KiB per CU,
// allocated in 2 KiB blocks: 80 KiB -> 2 workgroups, 40 KiB -> 4). Measured on
// MI355X, same bits, interleaved processes on one box per comparison
// (25,000,000-value bf16 buckets, K = 8: 1,526 tiles per shard):
//   AllGather 85.4-86.4 -> 79.7-80.1 us with 2 per CU (3: 80.3-80.6, 4: 84.3,
//   1: 116; the plain layer step 70.4 -> 72.7-73.0% of HBM peak); one-pass
//   AllReduce of the layer 1.191-1.193 -> 1.161-1.162 ms with 2 (3: 1.210-
//   1.213, slower; 4 to 6: unchanged); fused ReduceScatter + AllGather, the
//   pipelined layer step 78.4-78.5 -> 79.2-79.4% with 4 (2: 66%; 5, 6:
//   78.8-79.0%); token-weighted fp32, 10,000,019 values (1,221 tiles per
//   shard): two-phase 117.4-118.5 -> 114.2-115.0 us, one pass 111.8-114.2 ->
//   110.8-112.6 us.
// Shards of 131,072 tiles (1 GiB fp32 per rank) lose 1% with the cap, and the
// standalone ReduceScatter (K reads per write) loses 5% (79 -> 83 us): both run
// uncapped. A persistent grid of as few workgroups is no substitute (AllGather
// on 512-1,024 workgroups: 90-97 us): the cap keeps one tile per workgroup.
constexpr long long kCapSegTiles = 4096;   // shards of fewer tiles take the cap ...
constexpr long long kCapMinTiles = 4096;   // ... in launches of at least this many tiles
constexpr unsigned kCapLds2 = 80u << 10;   // AllGather and one-pass AllReduce: 2 per CU
constexpr unsigned kCapLds4 = 40u << 10;   // fused ReduceScatter + AllGather: 4 per CU
static_assert(kAlign >= 16 && kAlign <= 256 && (kAlign & (kAlign - 1)) == 0, "alignment");

__device__ __forceinline__ u32x4 load_stream(const char *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

template <bool CACHED>
__device__ __forceinline__ void store_rs(char *p, u32x4 v)
{
    if constexpr (CACHED) *reinterpret_cast<u32x4 *>(p) = v;
    else __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ void store_ag(char *p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN (sign kept).
__device__ __forceinline__ unsigned f32_to_bf16_bits(float f)
{
    unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <int DT>
__device__ __forceinline__ typename Tr<DT>::Acc load1(const char *p)
{
    if constexpr (DT == kF32) return *reinterpret_cast<const float *>(p);
    else if constexpr (DT == kBF16) return bf16_bits_to_f32(*reinterpret_cast<const unsigned short *>(p));
    else return *reinterpret_cast<const unsigned *>(p);
}

template <int DT>
__device__ __forceinline__ void store1(char *p, typename Tr<DT>::Acc v)
{
    if constexpr (DT == kF32) *reinterpret_cast<float *>(p) = v;
    else if constexpr (DT == kBF16) *reinterpret_cast<unsigned short *>(p) = (unsigned short)f32_to_bf16_bits(v);
    else *reinterpret_cast<unsigned *>(p) = v;
}

template <int DT>
__device__ __forceinline__ void unpack(const u32x4 v, typename Tr<DT>::Acc (&o)[Tr<DT>::V])
{
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
    } else if constexpr (DT == kBF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(v[i] << 16);
            o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = v[i];
    }
}

template <int DT>
__device__ __forceinline__ u32x4 pack(const typename Tr<DT>::Acc (&a)[Tr<DT>::V])
{
    u32x4 v;
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(a[i]);
    } else if constexpr (DT == kBF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = f32_to_bf16_bits(a[2 * i]) | (f32_to_bf16_bits(a[2 * i + 1]) << 16);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = a[i];
    }
    return v;
}

// operand m of shard c's fold is rank (c + 1 + m) mod K
__device__ __forceinline__ int fold_rank(int c, int m, int K)
{
    int r = c + 1 + m;
    return r >= K ? r - K : r;
}

template <int EP, typename A>
__device__ __forceinline__ A term(A x, float w)
{
    if constexpr (EP == kWeighted) return x * w;
    else return x;
}

template <int EP, typename A>
__device__ __forceinline__ A finish(A acc, float scale)
{
    if constexpr (EP == kMul) return acc * scale;
    else if constexpr (EP == kDiv || EP == kWeighted) return acc / scale;
    else return acc;
}

// One element of shard c at global index g: the ring-order fold and the
// epilogue. Stored to `out`, or with AR (fused AllReduce) to element g of every
// rank's output dst[r].
template <int DT, int EP, int KT, bool AR>
__device__ __forceinline__ void rs_elem(const RsParams &p, int K, int c, long long g, char *out)
{
    using A = typename Tr<DT>::Acc;
    constexpr int ES = Tr<DT>::ES;
    const int r0 = fold_rank(c, 0, K);
    A acc = term<EP>(load1<DT>(p.src[r0] + g * ES), p.w[r0]);
#pragma unroll
    for (int m = 1; m < (KT ? KT : kMaxK); ++m) {
        if (!KT && m >= K) break;
        const int r = fold_rank(c, m, K);
        acc = acc + term<EP>(load1<DT>(p.src[r] + g * ES), p.w[r]);
    }
    acc = finish<EP>(acc, p.scale);
    if constexpr (AR) {
#pragma unroll
        for (int i = 0; i < (KT ? KT : kMaxK); ++i) {
            if (!KT && i >= K) break;
            store1<DT>(p.dst[fold_rank(c, i, K)] + g * ES, acc);
        }
    } else {
        store1<DT>(out, acc);
    }
}

template <int DT, int EP, int KT, bool AR>
__device__ __forceinline__ void rs_scalar_range(const RsParams &p, int K, int c, long long base,
                                                long long nc, long long lo, long long hi)
{
    constexpr int ES = Tr<DT>::ES;
    char *dst = AR ? nullptr : p.dst[c];
    for (long long j = lo + threadIdx.x; j < hi; j += kBlock) {
        if (j < nc) rs_elem<DT, EP, KT, AR>(p, K, c, base + j, AR ? nullptr : dst + j * ES);
        else if (!AR && p.write_pads) store1<DT>(dst + j * ES, typename Tr<DT>::Acc(0));
    }
}

// The 128-bit body of a tile: nv vectors (nv == kBlock*U when FULL). The FULL
// variant has no per-lane conditions, so all loads are issued back to back and
// the stores are not separated by waits on earlier memory operations. With AR
// the packed result goes to offset `off` of all K outputs (ranks c+1, c+2, ...,
// c, no per-rank branch) instead of to `dst`.
template <int DT, int EP, int KT, int U, bool FULL, bool AR, bool CACHED>
__device__ __forceinline__ void rs_vectors(const RsParams &p, const int K, const int c,
                                           const long long off, char *dst, const long long nv)
{
    using A = typename Tr<DT>::Acc;
    constexpr int V = Tr<DT>::V;
    const int tid = threadIdx.x;
    A acc[U][V];
    if constexpr (KT != 0) {
        // issue all U*K loads, then fold in ring order
        u32x4 v[U][KT];
#pragma unroll
        for (int m = 0; m < KT; ++m) {
            const char *ps = p.src[fold_rank(c, m, KT)] + off;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const long long q = FULL ? (long long)tid + u * kBlock
                                         : min((long long)tid + u * kBlock, nv - 1);
                v[u][m] = load_stream(ps + q * 16);
            }
        }
#pragma unroll
        for (int m = 0; m < KT; ++m) {
            const float w = p.w[fold_rank(c, m, KT)];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                A x[V];
                unpack<DT>(v[u][m], x);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    acc[u][e] = m == 0 ? term<EP>(x[e], w) : acc[u][e] + term<EP>(x[e], w);
            }
        }
    } else {
        for (int m = 0; m < K; ++m) {
            const int r = fold_rank(c, m, K);
            const char *ps = p.src[r] + off;
            const float w = p.w[r];
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const long long q = FULL ? (long long)tid + u * kBlock
                                         : min((long long)tid + u * kBlock, nv - 1);
                v[u] = load_stream(ps + q * 16);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                A x[V];
                unpack<DT>(v[u], x);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    acc[u][e] = m == 0 ? term<EP>(x[e], w) : acc[u][e] + term<EP>(x[e], w);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const long long q = (long long)tid + u * kBlock;
#pragma unroll
        for (int e = 0; e < V; ++e) acc[u][e] = finish<EP>(acc[u][e], p.scale);
        if constexpr (AR) {
            const u32x4 o = pack<DT>(acc[u]);
#pragma unroll
            for (int i = 0; i < (KT ? KT : kMaxK); ++i) {
                if (!KT && i >= K) break;
                if (FULL || q < nv) store_ag(p.dst[fold_rank(c, i, K)] + off + q * 16, o);
            }
        } else {
            if (FULL || q < nv) store_rs<CACHED>(dst + q * 16, pack<DT>(acc[u]));
        }
    }
}

template <int DT, int EP, int KT, int U, bool AR, bool CACHED>
__device__ __forceinline__ void rs_tile(const RsParams &p, const int K, const long long bid)
{
    using A = typename Tr<DT>::Acc;
    constexpr int ES = Tr<DT>::ES, V = Tr<DT>::V;
    constexpr long long TE = (long long)kBlock * U * V;
    const long long seg = bid / p.tiles_per_seg;
    const long long t = bid - seg * p.tiles_per_seg;
    const int s = (int)(seg / K);
    const int c = (int)(seg - (long long)s * K);
    const long long j0 = (long long)s * p.sub;
    const long long j1 = min(j0 + p.sub, p.L);
    if (j0 >= j1) return;
    const long long base = (long long)c * p.L;
    const long long nc = max(0LL, min(p.L, p.n - base));
    const int meta = p.meta[c];
    const bool fast = (meta & kFastBit) != 0;
    const long long head = fast ? (long long)(((kAlign - (((meta & 255) + j0 * ES) & (kAlign - 1))) &
                                               (kAlign - 1)) / ES) : 0;
    const long long body = min(j0 + head, j1);
    const long long e0 = body + t * TE;
    const long long e1 = min(e0 + TE, j1);

    if (t == 0 && body > j0) rs_scalar_range<DT, EP, KT, AR>(p, K, c, base, nc, j0, body);
    if (e0 >= e1) return;
    if (!fast) {
        rs_scalar_range<DT, EP, KT, AR>(p, K, c, base, nc, e0, e1);
        return;
    }
    const long long ve = min(e1, nc);
    const long long nv = ve > e0 ? (ve - e0) / V : 0;
    char *dst = AR ? nullptr : p.dst[c] + e0 * ES;
    const long long off = (base + e0) * ES;
    if (nv == (long long)kBlock * U)
        rs_vectors<DT, EP, KT, U, true, AR, CACHED>(p, K, c, off, dst, nv);
    else if (nv > 0)
        rs_vectors<DT, EP, KT, U, false, AR, CACHED>(p, K, c, off, dst, nv);
    rs_scalar_range<DT, EP, KT, AR>(p, K, c, base, nc, e0 + nv * V, e1);
}

template <int DT, int EP, int KT, int U, bool AR, bool CACHED>
__global__ __launch_bounds__(kBlock) void rs_kernel(const RsParams p)
{
    const int K = KT ? KT : p.k;
    for (long long bid = blockIdx.x; bid < p.total_tiles; bid += gridDim.x)
        rs_tile<DT, EP, KT, U, AR, CACHED>(p, K, bid);
}

// Lean variant: one vector per lane per rank and at most 64 VGPRs (8 waves per
// SIMD), so one of its workgroups fits in the registers a 224-VGPR GEMM
// workgroup (two waves per SIMD) leaves free on a CU.
template <int DT, int EP, int KT, bool AR>
__global__ __launch_bounds__(kBlock, 8) void rs_kernel_lean(const RsParams p)
{
    const int K = KT ? KT : p.k;
    for (long long bid = blockIdx.x; bid < p.total_tiles; bid += gridDim.x)
        rs_tile<DT, EP, KT, 1, AR, false>(p, K, bid);
}

// ------------------------------------------------------------------ AllGather

template <int ES, int KT>
__device__ __forceinline__ void ag_scalar_range(const AgParams &p, int K, int c, long long base,
                                                long long lo, long long hi)
{
    const char *src = p.src[c];
    for (long long j = lo + threadIdx.x; j < hi; j += kAgBlock) {
        unsigned short h = 0;
        unsigned w = 0;
        if constexpr (ES == 2) h = *reinterpret_cast<const unsigned short *>(src + j * ES);
        else w = *reinterpret_cast<const unsigned *>(src + j * ES);
#pragma unroll
        for (int r = 0; r < (KT ? KT : kMaxK); ++r) {
            if (!KT && r >= K) break;
            if (p.skip_own && r == c) continue;
            char *d = p.dst[r] + (base + j) * ES;
            if constexpr (ES == 2) *reinterpret_cast<unsigned short *>(d) = h;
            else *reinterpret_cast<unsigned *>(d) = w;
        }
    }
}

// The 128-bit body of an AllGather tile. Destinations are visited as ranks
// c+1, c+2, ... (mod K), with rank c itself last and left out when SKIP_OWN, so
// the store sequence has no per-rank branch.
template <int ES, int KT, int U, bool FULL, bool SKIP_OWN>
__device__ __forceinline__ void ag_vectors(const AgParams &p, const int K, const int c,
                                           const char *src, const long long off, const long long nv)
{
    const int tid = threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const long long q = FULL ? (long long)tid + u * kAgBlock : min((long long)tid + u * kAgBlock, nv - 1);
        v[u] = *reinterpret_cast<const u32x4 *>(src + q * 16);
    }
    const int nr = SKIP_OWN ? K - 1 : K;
#pragma unroll
    for (int i = 0; i < (KT ? (SKIP_OWN ? KT - 1 : KT) : kMaxK); ++i) {
        if (!KT && i >= nr) break;
        int r = c + 1 + i;
        r = r >= K ? r - K : r;
        char *d = p.dst[r] + off;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long q = (long long)tid + u * kAgBlock;
            if (FULL || q < nv) store_ag(d + q * 16, v[u]);
        }
    }
}

// The AllGather body when the K outputs share a 16-byte phase but the shard
// does not: stores stay 16-byte aligned, and each lane assembles its 16 source
// bytes from dword-aligned loads (for 2-byte elements at an odd element
// address, five dwords joined with a byte shift). src is the shard address of
// chunk 0; the caller keeps every dword read inside the shard's valid range.
template <int ES, int KT, int U, bool FULL, bool SKIP_OWN>
__device__ __forceinline__ void ag_vectors_shifted(const AgParams &p, const int K, const int c,
                                                   const char *src, const long long off,
                                                   const long long nv)
{
    const int tid = threadIdx.x;
    const unsigned shift = (unsigned)((uintptr_t)src & 3);      // 0, or 2 for 2-byte elements
    const unsigned *w0 = reinterpret_cast<const unsigned *>(src - shift);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const long long q = FULL ? (long long)tid + u * kAgBlock : min((long long)tid + u * kAgBlock, nv - 1);
        const unsigned *w = w0 + q * 4;
        if (ES == 2 && shift) {
            unsigned a[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) a[i] = w[i];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[u][i] = __builtin_amdgcn_alignbyte(a[i + 1], a[i], 2);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[u][i] = w[i];
        }
    }
    const int nr = SKIP_OWN ? K - 1 : K;
#pragma unroll
    for (int i = 0; i < (KT ? (SKIP_OWN ? KT - 1 : KT) : kMaxK); ++i) {
        if (!KT && i >= nr) break;
        int r = c + 1 + i;
        r = r >= K ? r - K : r;
        char *d = p.dst[r] + off;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long q = (long long)tid + u * kAgBlock;
            if (FULL || q < nv) store_ag(d + q * 16, v[u]);
        }
    }
}

template <int ES, int KT, int U>
__device__ __forceinline__ void ag_tile(const AgParams &p, const int K, const long long bid)
{
    constexpr int V = 16 / ES;
    constexpr long long TE = (long long)kAgBlock * U * V;
    const long long seg = bid / p.tiles_per_seg;
    const long long t = bid - seg * p.tiles_per_seg;
    const int s = (int)(seg / K);
    const int c = (int)(seg - (long long)s * K);
    const long long base = (long long)c * p.L;
    const long long nc = max(0LL, min(p.L, p.n - base));
    const long long j0 = (long long)s * p.sub;
    const long long j1 = min(min(j0 + p.sub, p.L), nc);   // valid elements only
    if (j0 >= j1) return;
    const int meta = p.meta[c];
    const bool fast = (meta & kFastBit) != 0;
    const bool out_aligned = (meta & kOutAlignBit) != 0;
    const long long head = (fast || out_aligned)
                               ? (long long)(((kAlign - (((meta & 255) + j0 * ES) & (kAlign - 1))) &
                                              (kAlign - 1)) / ES)
                               : 0;
    const long long body = min(j0 + head, j1);
    const long long e0 = body + t * TE;
    const long long e1 = min(e0 + TE, j1);

    if (t == 0 && body > j0) ag_scalar_range<ES, KT>(p, K, c, base, j0, body);
    if (e0 >= e1) return;
    if (!fast && !out_aligned) {
        ag_scalar_range<ES, KT>(p, K, c, base, e0, e1);
        return;
    }
    if (!fast) {
        // outputs aligned, shard not: shifted loads. A 2-byte shift reads the
        // dword before a chunk and the one after it, so the first chunk of the
        // shard and a chunk ending at the last valid element go element-wise.
        const bool shifted = ES == 2 && (((uintptr_t)p.src[c] + (uintptr_t)(e0 * ES)) & 3) != 0;
        long long v0 = e0;
        if (shifted && v0 == 0) v0 += V;
        long long nv = v0 < e1 ? (e1 - v0) / V : 0;
        if (shifted && nv > 0 && v0 + nv * V >= nc) --nv;
        if (v0 > e0) ag_scalar_range<ES, KT>(p, K, c, base, e0, min(v0, e1));
        if (nv > 0) {
            const char *src = p.src[c] + v0 * ES;
            const long long off = (base + v0) * ES;
            if (nv == (long long)kAgBlock * U) {
                if (p.skip_own) ag_vectors_shifted<ES, KT, U, true, true>(p, K, c, src, off, nv);
                else ag_vectors_shifted<ES, KT, U, true, false>(p, K, c, src, off, nv);
            } else {
                if (p.skip_own) ag_vectors_shifted<ES, KT, U, false, true>(p, K, c, src, off, nv);
                else ag_vectors_shifted<ES, KT, U, false, false>(p, K, c, src, off, nv);
            }
        }
        ag_scalar_range<ES, KT>(p, K, c, base, max(v0, e0) + max(nv, 0LL) * V, e1);
        return;
    }
    const long long nv = (e1 - e0) / V;
    const char *src = p.src[c] + e0 * ES;
    const long long off = (base + e0) * ES;
    if (nv == (long long)kAgBlock * U) {
        if (p.skip_own) ag_vectors<ES, KT, U, true, true>(p, K, c, src, off, nv);
        else ag_vectors<ES, KT, U, true, false>(p, K, c, src, off, nv);
    } else if (nv > 0) {
        if (p.skip_own) ag_vectors<ES, KT, U, false, true>(p, K, c, src, off, nv);
        else ag_vectors<ES, KT, U, false, false>(p, K, c, src, off, nv);
    }
    ag_scalar_range<ES, KT>(p, K, c, base, e0 + nv * V, e1);
}

template <int ES, int KT, int U>
__global__ __launch_bounds__(kAgBlock) void ag_kernel(const AgParams p)
{
    const int K = KT ? KT : p.k;
    for (long long bid = blockIdx.x; bid < p.total_tiles; bid += gridDim.x)
        ag_tile<ES, KT, U>(p, K, bid);
}

// ------------------------------------------- ReduceScatter + AllGather fused

static_assert(kAgBlock == kBlock, "the fused kernel runs both tile kinds with one block size");

// A ReduceScatter of one buffer set and an AllGather of another in one launch
// (bucket b+1 reduced while bucket b is gathered): the ReduceScatter reads K
// bytes per byte written and the AllGather the reverse, so running their tiles
// side by side gives HBM a copy-like read/write mix. In each run of 16
// workgroup ids the first 8 (one per XCD, ids go round-robin over the 8 XCDs)
// take ReduceScatter tiles and the next 8 AllGather tiles; the tiles left over
// when one kind runs out go to the other.
template <int DT, int EP, int KT>
__global__ __launch_bounds__(kBlock) void rsag_kernel(const RsParams rp, const AgParams ap)
{
    constexpr int ES = Tr<DT>::ES;
    constexpr long long G = 8;
    const int K = KT ? KT : rp.k;
    const long long nr = rp.total_tiles, na = ap.total_tiles;
    const long long paired = ((nr < na ? nr : na) / G) * G;
    const long long bid = blockIdx.x;
    if (bid < 2 * paired) {
        const long long idx = (bid / (2 * G)) * G + bid % G;
        if ((bid / G) & 1) ag_tile<ES, KT, kAgU>(ap, K, idx);
        else rs_tile<DT, EP, KT, RsU<DT>::U, false, true>(rp, K, idx);
        return;
    }
    const long long rem = bid - 2 * paired;
    if (rem < nr - paired) rs_tile<DT, EP, KT, RsU<DT>::U, false, true>(rp, K, paired + rem);
    else ag_tile<ES, KT, kAgU>(ap, K, paired + rem - (nr - paired));
}

// ------------------------------------------------------------------ launchers

bool small_shards(long long tiles_per_seg, long long total_tiles)
{
    return tiles_per_seg < kCapSegTiles && total_tiles >= kCapMinTiles;
}

template <int DT, int EP, int KT, bool AR>
hipError_t rs_go(const RsParams &p, long long grid, bool lean, hipStream_t st)
{
    if (lean)
        hipLaunchKernelGGL((rs_kernel_lean<DT, EP, KT, AR>), dim3((unsigned)grid), dim3(kBlock), 0, st, p);
    else if (p.max_blocks > 0)
        hipLaunchKernelGGL((rs_kernel<DT, EP, KT, kUCapped, AR, false>), dim3((unsigned)grid), dim3(kBlock), 0, st, p);
    else if (!AR && p.cache_out)
        hipLaunchKernelGGL((rs_kernel<DT, EP, KT, RsU<DT>::U, false, true>), dim3((unsigned)grid), dim3(kBlock), 0, st, p);
    else
        hipLaunchKernelGGL((rs_kernel<DT, EP, KT, AR ? kArU : RsU<DT>::U, AR, false>), dim3((unsigned)grid), dim3(kBlock),
                           AR && small_shards(p.tiles_per_seg, p.total_tiles) ? kCapLds2 : 0u, st, p);
    return hipGetLastError();
}

template <int DT, int EP, bool AR>
hipError_t rs_k(const RsParams &p, long long grid, bool lean, hipStream_t st)
{
    switch (p.k) {
    case 2: return rs_go<DT, EP, 2, AR>(p, grid, lean, st);
    case 4: return rs_go<DT, EP, 4, AR>(p, grid, lean, st);
    case 8: return rs_go<DT, EP, 8, AR>(p, grid, lean, st);
    default: return rs_go<DT, EP, 0, AR>(p, grid, lean, st);
    }
}

template <bool AR>
hipError_t rs_dispatch(const RsParams &q, int dt, int ep, long long grid, bool lean, hipStream_t st)
{
    if (dt == kF32) {
        switch (ep) {
        case kSum: return rs_k<kF32, kSum, AR>(q, grid, lean, st);
        case kMul: return rs_k<kF32, kMul, AR>(q, grid, lean, st);
        case kDiv: return rs_k<kF32, kDiv, AR>(q, grid, lean, st);
        default: return rs_k<kF32, kWeighted, AR>(q, grid, lean, st);
        }
    }
    if (dt == kBF16) {
        switch (ep) {
        case kSum: return rs_k<kBF16, kSum, AR>(q, grid, lean, st);
        case kMul: return rs_k<kBF16, kMul, AR>(q, grid, lean, st);
        case kDiv: return rs_k<kBF16, kDiv, AR>(q, grid, lean, st);
        default: return rs_k<kBF16, kWeighted, AR>(q, grid, lean, st);
        }
    }
    return rs_k<kI32, kSum, AR>(q, grid, lean, st);
}

template <int ES, int KT>
hipError_t ag_go(const AgParams &p, long long grid, hipStream_t st)
{
    if (p.max_blocks > 0)
        hipLaunchKernelGGL((ag_kernel<ES, KT, kUCapped>), dim3((unsigned)grid), dim3(kAgBlock), 0, st, p);
    else
        hipLaunchKernelGGL((ag_kernel<ES, KT, kAgU>), dim3((unsigned)grid), dim3(kAgBlock),
                           small_shards(p.tiles_per_seg, p.total_tiles) ? kCapLds2 : 0u, st, p);
    return hipGetLastError();
}

template <int ES>
hipError_t ag_k(const AgParams &p, long long grid, hipStream_t st)
{
    switch (p.k) {
    case 2: return ag_go<ES, 2>(p, grid, st);
    case 4: return ag_go<ES, 4>(p, grid, st);
    case 8: return ag_go<ES, 8>(p, grid, st);
    default: return ag_go<ES, 0>(p, grid, st);
    }
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// vectors per lane of the tiles a launch will run (the kernel choice in rs_go)
int rs_vectors_per_thread(int dt, bool lean, bool capped)
{
    if (lean) return 1;
    if (capped) return kUCapped;
    return dt == kF32 ? RsU<kF32>::U : dt == kBF16 ? RsU<kBF16>::U : RsU<kI32>::U;
}

}  // namespace

namespace {

// kFastBit: every stream ins[r] + in_off and `out` share one 16-byte phase.
// Bits 0-7: the address phase modulo 256 of the anchor stream (ins[0] + in_off
// when anchor_ins, else out) at shard element 0; tile bodies start where the
// anchor is kAlign-byte aligned, so its wave-wide 1 KiB accesses cover whole
// cache lines.
int phase_meta(const char *const *ins, long long in_off_bytes, int k, const char *out,
               bool anchor_ins)
{
    const unsigned ph = (unsigned)((uintptr_t)out & 15);
    bool same = true;
    for (int r = 0; r < k; ++r)
        same = same && (unsigned)(((uintptr_t)ins[r] + (uintptr_t)in_off_bytes) & 15) == ph;
    const uintptr_t anchor = anchor_ins ? (uintptr_t)ins[0] + (uintptr_t)in_off_bytes : (uintptr_t)out;
    return (same ? kFastBit : 0) | (int)(anchor & 255);
}

long long grid_for(long long total_tiles, int max_blocks)
{
    const long long cap = max_blocks > 0 ? max_blocks : 0x7fffffffLL;
    return total_tiles < cap ? total_tiles : cap;
}

}  // namespace

long long plan_rs(RsParams &p, int dt, bool lean)
{
    const int es = elem_size(dt);
    for (int c = 0; c < p.k; ++c)
        p.meta[c] = phase_meta(p.src, (long long)c * p.L * es, p.k, p.dst[c], true);
    p.sub = ceil_div(p.L, p.S);
    const long long te = (long long)kBlock * rs_vectors_per_thread(dt, lean, p.max_blocks > 0) * (16 / es);
    p.tiles_per_seg = p.sub > 0 ? ceil_div(p.sub, te) : 1;
    p.total_tiles = (long long)p.S * p.k * p.tiles_per_seg;
    p.cache_out = p.cache_out && (long long)p.k * p.L * es <= kCacheOutBytes;
    return grid_for(p.total_tiles, p.max_blocks);
}

long long plan_ag(AgParams &p, int dt)
{
    const int es = elem_size(dt);
    for (int c = 0; c < p.k; ++c) {
        // the K outputs at element c*L against the shard (the "input" here)
        const char *outs[kMaxK];
        for (int r = 0; r < p.k; ++r) outs[r] = p.dst[r];
        const long long off = (long long)c * p.L * es;
        p.meta[c] = phase_meta(outs, off, p.k, p.src[c], true);
        bool same = true;
        for (int r = 1; r < p.k; ++r)
            same = same && (((uintptr_t)outs[r] + (uintptr_t)off) & 15) ==
                               (((uintptr_t)outs[0] + (uintptr_t)off) & 15);
        if (same) p.meta[c] |= kOutAlignBit;
    }
    p.sub = ceil_div(p.L, p.S);
    const long long te = (long long)kAgBlock * (p.max_blocks > 0 ? kUCapped : kAgU) * (16 / es);
    p.tiles_per_seg = p.sub > 0 ? ceil_div(p.sub, te) : 1;
    p.total_tiles = (long long)p.S * p.k * p.tiles_per_seg;
    return grid_for(p.total_tiles, p.max_blocks);
}

hipError_t launch_rs(const RsParams &p, int dt, int ep, hipStream_t st, bool lean)
{
    RsParams q = p;
    const long long grid = plan_rs(q, dt, lean);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return rs_dispatch<false>(q, dt, ep, grid, lean, st);
}

long long plan_ar(RsParams &p, int dt, bool lean)
{
    const int es = elem_size(dt);
    for (int c = 0; c < p.k; ++c) {
        // the K inputs and the K outputs at element c*L; anchor: output 0
        const long long off = (long long)c * p.L * es;
        const int m_in = phase_meta(p.src, off, p.k, p.dst[0] + off, false);
        const int m_out = phase_meta(p.dst, off, p.k, p.dst[0] + off, false);
        p.meta[c] = (m_in & m_out & kFastBit) | (m_out & 255);
    }
    p.write_pads = 0;
    p.sub = ceil_div(p.L, p.S);
    const long long te = (long long)kBlock * (lean ? 1 : p.max_blocks > 0 ? kUCapped : kArU) * (16 / es);
    p.tiles_per_seg = p.sub > 0 ? ceil_div(p.sub, te) : 1;
    p.total_tiles = (long long)p.S * p.k * p.tiles_per_seg;
    return grid_for(p.total_tiles, p.max_blocks);
}

hipError_t launch_ar(const RsParams &p, int dt, int ep, hipStream_t st, bool lean)
{
    RsParams q = p;
    const long long grid = plan_ar(q, dt, lean);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return rs_dispatch<true>(q, dt, ep, grid, lean, st);
}

template <int DT, int EP>
hipError_t rsag_k(const RsParams &rp, const AgParams &ap, long long grid, hipStream_t st)
{
    // both halves over small shards (an empty half counts as small)
    const bool small = (rp.total_tiles == 0 || rp.tiles_per_seg < kCapSegTiles) &&
                       (ap.total_tiles == 0 || ap.tiles_per_seg < kCapSegTiles) && grid >= kCapMinTiles;
    const unsigned lds = small ? kCapLds4 : 0u;
    switch (rp.k) {
    case 2: hipLaunchKernelGGL((rsag_kernel<DT, EP, 2>), dim3((unsigned)grid), dim3(kBlock), lds, st, rp, ap); break;
    case 4: hipLaunchKernelGGL((rsag_kernel<DT, EP, 4>), dim3((unsigned)grid), dim3(kBlock), lds, st, rp, ap); break;
    case 8: hipLaunchKernelGGL((rsag_kernel<DT, EP, 8>), dim3((unsigned)grid), dim3(kBlock), lds, st, rp, ap); break;
    default: hipLaunchKernelGGL((rsag_kernel<DT, EP, 0>), dim3((unsigned)grid), dim3(kBlock), lds, st, rp, ap); break;
    }
    return hipGetLastError();
}

hipError_t launch_rsag(const RsParams &rp0, const AgParams &ap0, int dt, int ep, hipStream_t st)
{
    RsParams rp = rp0;
    AgParams ap = ap0;
    rp.max_blocks = 0;
    ap.max_blocks = 0;
    plan_rs(rp, dt);
    plan_ag(ap, dt);
    const long long grid = rp.total_tiles + ap.total_tiles;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dt == kF32) {
        switch (ep) {
        case kSum: return rsag_k<kF32, kSum>(rp, ap, grid, st);
        case kMul: return rsag_k<kF32, kMul>(rp, ap, grid, st);
        default: return rsag_k<kF32, kDiv>(rp, ap, grid, st);
        }
    }
    if (dt == kBF16) {
        switch (ep) {
        case kSum: return rsag_k<kBF16, kSum>(rp, ap, grid, st);
        case kMul: return rsag_k<kBF16, kMul>(rp, ap, grid, st);
        default: return rsag_k<kBF16, kDiv>(rp, ap, grid, st);
        }
    }
    return rsag_k<kI32, kSum>(rp, ap, grid, st);
}

hipError_t launch_ag(const AgParams &p, int dt, hipStream_t st)
{
    AgParams q = p;
    const long long grid = plan_ag(q, dt);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return elem_size(dt) == 2 ? ag_k<2>(q, grid, st) : ag_k<4>(q, grid, st);
}

}  // namespace dps
