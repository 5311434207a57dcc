// On-demand communication on one GPU: scatter-accumulate and settle.
//
// "Using ODC to Accelerate AMD SFT Training", section "From Collective
// Primitives to Two One-sided P2P Primitives" (Figure 2): after computing a
// gradient a rank pushes each shard of it to the shard's owner, which adds it
// into its gradient accumulator; section "From Per-iteration to Per-minibatch
// Synchronization": one settle per minibatch makes the accumulated gradients
// final. With K ranks emulated as K buffers, a push is the whole gradient added
// into the K owners' fp32 accumulators:
//   acc[c][j] = acc[c][j] + f32(g[c*L + j])
// One launch applies P pushes in their given order, each element of the
// accumulator read once and written once:
//   acc[c][j] = (...((acc[c][j] + f32(g_0[c*L+j])) + f32(g_1[c*L+j])) ...)
// which is bit-identical to P launches of one push (the same fp32 additions in
// the same order, no FMA). Per element: P*s bytes of gradient read, 4 bytes of
// accumulator read and 4 written: HBM-bound.
//
// Settle: out[c][j] = cast(acc[c][j] / divisor) (the multiply by an exact 1/2^m
// when the divisor is a power of two), pads zero, and optionally the
// accumulator reset to zero for the next minibatch.
#include "odc_internal.h"

#pragma clang fp contract(off)

namespace dps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Sizes measured best at layer size on MI355X
constexpr int kOdcBlock = 256;
constexpr long long kOdcTile = 4096;      // elements of one shard per workgroup tile
constexpr int kPushUnroll = 4;            // gradients whose loads are in flight together
// Residency: the bf16 push and settle launches of at least kOdcCapMinGrid
// workgroups reserve 52 KiB of LDS per workgroup (the kernels use none), so a
// CU holds 3 of them instead of 8. Measured on MI355X at layer size (K = 8,
// 27,262,976-value shards, 6,656 tiles each), interleaved processes on two
// boxes, same bits: push of 8 gradients 908-916 -> 896-905 us (2 per CU:
// 916-924, 4 per CU: 904-910), settle with reset 375-378 -> 358-361 us (2:
// 364-366, 4: 379-381). The fp32 forms run uncapped (not measured).
constexpr unsigned kOdcCapLds = 52u << 10;
constexpr long long kOdcCapMinGrid = 4096;

// Accumulators: ordinary loads, nontemporal stores (nontemporal loads as well
// measured slower); settled shards: nontemporal stores.
__device__ __forceinline__ f32x4 ld_acc(const float *p)
{
    return *reinterpret_cast<const f32x4 *>(p);
}

__device__ __forceinline__ void st_acc(float *p, f32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}

template <typename V>
__device__ __forceinline__ void st_out(V *p, V v)
{
    __builtin_nontemporal_store(v, p);
}

// G elements per thread group (the gradient load is G*s bytes, the
// accumulator G*4 bytes); U groups per thread per tile. With G = 4 every
// accumulator store instruction covers one contiguous 1 KiB per wave and the
// written bytes equal the accumulator bytes; bf16 with G = 8 (16-byte gradient
// loads, two 16-byte accumulator stores per group) writes about 12% more
// partial lines but runs faster on MI355X.
template <int DT> struct Grp {
    static constexpr int G = DT == kBF16 ? 8 : 4;
    static constexpr int U = (int)(kOdcTile / (kOdcBlock * G));
    static constexpr int W = G * (DT == kBF16 ? 2 : 4) / 4;     // 32-bit words per gradient load
};
template <int W> struct GradVec;
template <> struct GradVec<2> { typedef u32x2 T; };
template <> struct GradVec<4> { typedef u32x4 T; };

__device__ __forceinline__ float ld_elem(const char *g, long long i, int dt)
{
    if (dt == kBF16)
        return __uint_as_float((unsigned)(*reinterpret_cast<const unsigned short *>(g + 2 * i)) << 16);
    return *reinterpret_cast<const float *>(g + 4 * i);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN (sign kept).
__device__ __forceinline__ unsigned to_bf16_bits(float f)
{
    unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// add one gradient group (W words = G elements) into G accumulator values
template <int DT, int W, typename V>
__device__ __forceinline__ void add_group(float *a, const V v)
{
    if constexpr (DT == kBF16) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
            a[2 * w] = a[2 * w] + __uint_as_float(v[w] << 16);
            a[2 * w + 1] = a[2 * w + 1] + __uint_as_float(v[w] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int w = 0; w < W; ++w) a[w] = a[w] + __uint_as_float(v[w]);
    }
}

template <int DT>
__global__ __launch_bounds__(kOdcBlock) void scatter_accumulate_kernel(const SaParams p)
{
    constexpr int ES = DT == kBF16 ? 2 : 4;
    constexpr int G = Grp<DT>::G, U = Grp<DT>::U, W = Grp<DT>::W;
    typedef typename GradVec<W>::T V;
    const long long bid = blockIdx.x;
    const int c = (int)(bid / p.tiles_per_shard);
    const long long t = bid - (long long)c * p.tiles_per_shard;
    const long long base = (long long)c * p.L;
    const long long nc = max(0LL, min(p.L, p.n - base));
    const long long e0 = t * kOdcTile;
    const long long e1 = min(e0 + kOdcTile, nc);
    if (e0 >= e1) return;
    float *acc = p.acc[c];
    const long long ng = p.aligned[c] ? (e1 - e0) / G : 0;
    if (ng > 0) {
        // groups q = threadIdx.x + u*kOdcBlock; out-of-range lanes re-read the
        // last group and do not store
        long long q[U];
        float a[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            q[u] = min((long long)threadIdx.x + u * kOdcBlock, ng - 1);
            const float *ap = acc + e0 + q[u] * G;
#pragma unroll
            for (int h = 0; h < G / 4; ++h) {
                const f32x4 v = ld_acc(ap + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[u][4 * h + e] = v[e];
            }
        }
        const long long goff = (base + e0) * ES;
        for (int i0 = 0; i0 < p.np; i0 += kPushUnroll) {
            V v[kPushUnroll][U];
#pragma unroll
            for (int i = 0; i < kPushUnroll; ++i) {
                if (i0 + i < p.np) {
                    const char *g = p.g[i0 + i] + goff;
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[i][u] = __builtin_nontemporal_load(
                            reinterpret_cast<const V *>(g + q[u] * (G * ES)));
                }
            }
#pragma unroll
            for (int i = 0; i < kPushUnroll; ++i) {
                if (i0 + i < p.np) {
#pragma unroll
                    for (int u = 0; u < U; ++u) add_group<DT, W>(a[u], v[i][u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if ((long long)threadIdx.x + u * kOdcBlock < ng) {
                float *ap = acc + e0 + q[u] * G;
#pragma unroll
                for (int h = 0; h < G / 4; ++h)
                    st_acc(ap + 4 * h, f32x4{a[u][4 * h], a[u][4 * h + 1], a[u][4 * h + 2], a[u][4 * h + 3]});
            }
        }
    }
    for (long long j = e0 + ng * G + threadIdx.x; j < e1; j += kOdcBlock) {
        float s = acc[j];
        for (int i = 0; i < p.np; ++i) s = s + ld_elem(p.g[i], base + j, DT);
        acc[j] = s;
    }
}

template <bool MUL>
__device__ __forceinline__ float settle_val(const SettleParams &p, float a)
{
    return MUL ? a * p.scale : a / p.scale;
}

template <int DT>
__device__ __forceinline__ void store_out(char *out, long long j, float v)
{
    if constexpr (DT == kBF16) reinterpret_cast<unsigned short *>(out)[j] = (unsigned short)to_bf16_bits(v);
    else reinterpret_cast<float *>(out)[j] = v;
}

template <int DT, bool MUL>
__global__ __launch_bounds__(kOdcBlock) void settle_kernel(const SettleParams p)
{
    constexpr int U = (int)(kOdcTile / (kOdcBlock * 4));
    const long long bid = blockIdx.x;
    const int c = (int)(bid / p.tiles_per_shard);
    const long long t = bid - (long long)c * p.tiles_per_shard;
    const long long nc = max(0LL, min(p.L, p.n - (long long)c * p.L));
    const long long e0 = t * kOdcTile;
    const long long e1 = min(e0 + kOdcTile, p.L);
    float *acc = p.acc[c];
    char *out = p.out[c];
    // 4-element groups wholly inside the valid part
    const long long ng = p.aligned[c] ? max(0LL, min(e1, nc) - e0) / 4 : 0;
    if (ng > 0) {
        f32x4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long q = min((long long)threadIdx.x + u * kOdcBlock, ng - 1);
            a[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(acc + e0 + 4 * q));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long q = (long long)threadIdx.x + u * kOdcBlock;
            if (q < ng) {
                const long long j = e0 + 4 * q;
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = settle_val<MUL>(p, a[u][e]);
                if constexpr (DT == kBF16) {
                    const unsigned lo = to_bf16_bits(r[0]) | (to_bf16_bits(r[1]) << 16);
                    const unsigned hi = to_bf16_bits(r[2]) | (to_bf16_bits(r[3]) << 16);
                    st_out(reinterpret_cast<u32x2 *>(out + 2 * j), u32x2{lo, hi});
                } else {
                    st_out(reinterpret_cast<f32x4 *>(out + 4 * j), f32x4{r[0], r[1], r[2], r[3]});
                }
                if (p.reset) st_acc(acc + j, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            }
        }
    }
    for (long long j = e0 + 4 * ng + threadIdx.x; j < e1; j += kOdcBlock) {
        float v = 0.0f;
        if (j < nc) {
            v = settle_val<MUL>(p, acc[j]);
            if (p.reset) acc[j] = 0.0f;
        }
        store_out<DT>(out, j, v);
    }
}

long long ceil_div_ll(long long a, long long b) { return (a + b - 1) / b; }

}  // namespace

hipError_t launch_scatter_accumulate(const SaParams &p0, int dt, hipStream_t st)
{
    SaParams p = p0;
    const long long es = elem_size(dt);
    const int gbytes = dt == kBF16 ? Grp<kBF16>::G * 2 : Grp<kF32>::G * 4;
    for (int c = 0; c < p.k; ++c) {
        bool ok = (uintptr_t)p.acc[c] % 16 == 0;
        for (int i = 0; i < p.np && ok; ++i)
            ok = ((uintptr_t)p.g[i] + (uintptr_t)((long long)c * p.L * es)) % (uintptr_t)gbytes == 0;
        p.aligned[c] = ok ? 1 : 0;
    }
    p.tiles_per_shard = ceil_div_ll(p.L, kOdcTile);
    const long long grid = p.tiles_per_shard * p.k;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dt == kBF16)
        hipLaunchKernelGGL(scatter_accumulate_kernel<kBF16>, dim3((unsigned)grid), dim3(kOdcBlock),
                           grid >= kOdcCapMinGrid ? kOdcCapLds : 0u, st, p);
    else
        hipLaunchKernelGGL(scatter_accumulate_kernel<kF32>, dim3((unsigned)grid), dim3(kOdcBlock), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_settle(const SettleParams &p0, int dt, bool mul, hipStream_t st)
{
    SettleParams p = p0;
    const int es = elem_size(dt);
    for (int c = 0; c < p.k; ++c)
        p.aligned[c] =
            ((uintptr_t)p.acc[c] % 16 == 0 && (uintptr_t)p.out[c] % (uintptr_t)(4 * es) == 0) ? 1 : 0;
    p.tiles_per_shard = ceil_div_ll(p.L, kOdcTile);
    const long long grid = p.tiles_per_shard * p.k;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), b(kOdcBlock);
    if (dt == kBF16) {
        const unsigned lds = grid >= kOdcCapMinGrid ? kOdcCapLds : 0u;
        if (mul) hipLaunchKernelGGL((settle_kernel<kBF16, true>), g, b, lds, st, p);
        else hipLaunchKernelGGL((settle_kernel<kBF16, false>), g, b, lds, st, p);
    } else {
        if (mul) hipLaunchKernelGGL((settle_kernel<kF32, true>), g, b, 0, st, p);
        else hipLaunchKernelGGL((settle_kernel<kF32, false>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace dps
