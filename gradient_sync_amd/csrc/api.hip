// extern "C" entry points of libdpsync: argument validation, shard planning
// and kernel dispatch on the caller's stream. The contract of every call is
// stated in include/dpsync.h.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "dps_internal.h"
#include "odc_internal.h"
#include "dpsync.h"

static_assert(dps::kMaxK == DP_MAX_K, "kernel and ABI rank limits differ");

// Device memory of dp_fsdp_layer_static: the K gathered weights and the K
// per-rank weight gradients, for callers that cannot allocate. Each GPU the
// library runs on holds its own copy until the process ends. In host code the
// array's name is only a stand-in; its device address comes from
// hipGetSymbolAddress, once per device (scratch_base below).
static __device__ __align__(256) unsigned char scratch[DP_STATIC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

dp_status_t hip_status(hipError_t e)
{
    if (e == hipSuccess) return DP_OK;
    g_last_hip_error = (int)e;
    return DP_ERR_HIP;
}

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range span(const void *p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }

bool overlap(Range a, Range b) { return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi; }

bool valid_k(int k) { return k >= 1 && k <= DP_MAX_K; }

// launch options: NULL = defaults; a negative cap, unknown flags or non-zero
// reserved words are invalid
// DP_LAUNCH_SHARE_CU and DP_LAUNCH_LEAN pick the GEMM variants that leave room
// for a sync workgroup on each CU; neither: the fastest variant.
int gemm_variant(bool share_cu, bool lean)
{
    return share_cu ? dps::kGemmShareCU : lean ? dps::kGemmCoresident : dps::kGemmFast;
}

bool opts_ok(const dp_launch_opts_t *o, int &max_wg, bool *share_cu = nullptr,
             bool *two_phase = nullptr, bool *lean = nullptr, bool *b_nk = nullptr)
{
    max_wg = 0;
    if (share_cu) *share_cu = false;
    if (two_phase) *two_phase = false;
    if (lean) *lean = false;
    if (b_nk) *b_nk = false;
    if (!o) return true;
    if (o->max_workgroups < 0 ||
        (o->flags &
         ~(DP_LAUNCH_SHARE_CU | DP_LAUNCH_TWO_PHASE | DP_LAUNCH_LEAN | DP_LAUNCH_B_NK)) ||
        o->reserved[0] || o->reserved[1])
        return false;
    if (b_nk) *b_nk = (o->flags & DP_LAUNCH_B_NK) != 0;
    max_wg = o->max_workgroups;
    if (share_cu) *share_cu = (o->flags & DP_LAUNCH_SHARE_CU) != 0;
    if (two_phase) *two_phase = (o->flags & DP_LAUNCH_TWO_PHASE) != 0;
    if (lean) *lean = (o->flags & DP_LAUNCH_LEAN) != 0;
    return true;
}

bool valid_dtype(int dt) { return dt == DP_F32 || dt == DP_BF16 || dt == DP_I32; }

// every element non-null and element-aligned
bool ptrs_ok(const void *const *a, int k, int es)
{
    if (!a) return false;
    for (int i = 0; i < k; ++i)
        if (!a[i] || ((uintptr_t)a[i] % (uintptr_t)es) != 0) return false;
    return true;
}

// n elements of size es per rank must fit comfortably in a signed 64-bit byte count
bool size_ok(size_t n, int es) { return n <= ((size_t)1 << 58) / (size_t)es; }

bool pairwise_disjoint(void *const *a, int k, size_t bytes)
{
    for (int i = 0; i < k; ++i)
        for (int j = i + 1; j < k; ++j)
            if (overlap(span(a[i], bytes), span(a[j], bytes))) return false;
    return true;
}

int64_t shard_valid(int64_t n, int64_t L, int c)
{
    const int64_t lo = (int64_t)c * L;
    if (lo >= n) return 0;
    return n - lo < L ? n - lo : L;
}

// epilogue for DP_SUM / DP_AVG; AVG by a power-of-two K multiplies by the
// exact reciprocal, which rounds the same real number as the division
void pick_epilogue(int op, int k, int &ep, float &scale)
{
    if (op == DP_SUM) {
        ep = dps::kSum;
        scale = 1.0f;
    } else if ((k & (k - 1)) == 0) {
        ep = dps::kMul;
        scale = 1.0f / (float)k;
    } else {
        ep = dps::kDiv;
        scale = (float)k;
    }
}

dp_status_t validate_rs_ag_common(const void *const *send, void *const *recv, size_t n, int k,
                                  int dt, int s_chunks)
{
    if (!valid_k(k) || s_chunks < 1) return DP_ERR_INVALID_ARG;
    if (!valid_dtype(dt)) return DP_ERR_UNSUPPORTED;
    const int es = dps::elem_size(dt);
    if (!size_ok(n, es)) return DP_ERR_INVALID_ARG;
    if (n == 0) return (send && recv) ? DP_OK : DP_ERR_INVALID_ARG;
    if (!ptrs_ok(send, k, es) || !ptrs_ok((const void *const *)recv, k, es)) return DP_ERR_INVALID_ARG;
    return DP_OK;
}

// ReduceScatter launch shared by the RS and AR entry points.
// out[c] = element 0 of shard c's output region.
// keep_cached: an AllGather reads the shards next (two-phase AllReduce, bucket
// pipeline), so small shard sets are left in the caches.
dp_status_t run_rs(const void *const *send, char *const *out, int64_t n, int64_t L, int k, int dt,
                   int ep, float scale, const float *w, int write_pads, int s_chunks,
                   hipStream_t st, int max_wg = 0, bool lean = false, bool keep_cached = false)
{
    dps::RsParams p;
    memset(&p, 0, sizeof(p));
    for (int r = 0; r < k; ++r) {
        p.src[r] = (const char *)send[r];
        p.dst[r] = out[r];
        p.w[r] = w ? w[r] : 1.0f;
    }
    p.scale = scale;
    p.write_pads = write_pads;
    p.n = n;
    p.L = L;
    p.k = k;
    p.S = s_chunks;
    p.max_blocks = max_wg;
    p.cache_out = keep_cached ? 1 : 0;
    return hip_status(dps::launch_rs(p, dt, ep, st, lean));
}

dp_status_t run_ag(const void *const *shard, char *const *out, int64_t n, int64_t L, int k, int dt,
                   int skip_own, int s_chunks, hipStream_t st, int max_wg = 0)
{
    dps::AgParams p;
    memset(&p, 0, sizeof(p));
    for (int r = 0; r < k; ++r) {
        p.src[r] = (const char *)shard[r];
        p.dst[r] = out[r];
    }
    p.skip_own = skip_own;
    p.n = n;
    p.L = L;
    p.k = k;
    p.S = s_chunks;
    p.max_blocks = max_wg;
    return hip_status(dps::launch_ag(p, dt, st));
}

// AllReduce-shaped validation: for every r, recv[r] either equals send[r] or
// overlaps no send buffer; receive buffers are pairwise disjoint.
dp_status_t check_ar_alias(const void *const *send, void *const *recv, size_t n, int k, int es)
{
    const size_t bytes = n * (size_t)es;
    for (int r = 0; r < k; ++r) {
        if (recv[r] == send[r]) continue;
        for (int q = 0; q < k; ++q)
            if (overlap(span(recv[r], bytes), span(send[q], bytes))) return DP_ERR_ALIAS;
    }
    return pairwise_disjoint(recv, k, bytes) ? DP_OK : DP_ERR_ALIAS;
}

dp_status_t run_ar(const void *const *send, void *const *recv, size_t n, int k, int dt, int ep,
                   float scale, const float *w, int s_chunks, hipStream_t st, int max_wg = 0,
                   bool two_phase = false, bool lean = false)
{
    const int es = dps::elem_size(dt);
    const int64_t L = (int64_t)dp_shard_len(n, k);
    if (!two_phase) {
        // one pass: fold each shard and write it to every rank's output
        dps::RsParams p;
        memset(&p, 0, sizeof(p));
        for (int r = 0; r < k; ++r) {
            p.src[r] = (const char *)send[r];
            p.dst[r] = (char *)recv[r];
            p.w[r] = w ? w[r] : 1.0f;
        }
        p.scale = scale;
        p.n = (long long)n;
        p.L = L;
        p.k = k;
        p.S = s_chunks;
        p.max_blocks = max_wg;
        return hip_status(dps::launch_ar(p, dt, ep, st, lean));
    }
    char *rs_out[DP_MAX_K];
    for (int c = 0; c < k; ++c) rs_out[c] = (char *)recv[c] + (size_t)c * (size_t)L * (size_t)es;
    dp_status_t s = run_rs(send, rs_out, (int64_t)n, L, k, dt, ep, scale, w, 0, s_chunks, st,
                           max_wg, lean, true);
    if (s != DP_OK) return s;
    return run_ag((const void *const *)rs_out, (char *const *)recv, (int64_t)n, L, k, dt, 1,
                  s_chunks, st, max_wg);
}

// ReduceScatter argument checks (shared by the single and the fused call);
// in_place reports the documented in-place form.
dp_status_t check_rs(const void *const *send, void *const *recv, size_t n, int k, int dt, int op,
                     int s_chunks, bool &in_place)
{
    in_place = false;
    dp_status_t s = validate_rs_ag_common(send, recv, n, k, dt, s_chunks);
    if (s != DP_OK || n == 0) return s;
    if (op != DP_SUM && op != DP_AVG) return DP_ERR_UNSUPPORTED;
    if (dt == DP_I32 && op != DP_SUM) return DP_ERR_UNSUPPORTED;
    const int es = dps::elem_size(dt);
    const size_t L = dp_shard_len(n, k);
    in_place = n == L * (size_t)k;
    for (int c = 0; c < k && in_place; ++c)
        in_place = (const char *)recv[c] == (const char *)send[c] + (size_t)c * L * (size_t)es;
    if (!in_place) {
        for (int c = 0; c < k; ++c)
            for (int r = 0; r < k; ++r)
                if (overlap(span(recv[c], L * es), span(send[r], n * es))) return DP_ERR_ALIAS;
        if (!pairwise_disjoint(recv, k, L * es)) return DP_ERR_ALIAS;
    }
    return DP_OK;
}

// AllGather argument checks; in_place: shard c already sits in recv[c].
dp_status_t check_ag(const void *const *send, void *const *recv, size_t n, int k, int dt,
                     int s_chunks, bool &in_place)
{
    in_place = false;
    dp_status_t s = validate_rs_ag_common(send, recv, n, k, dt, s_chunks);
    if (s != DP_OK || n == 0) return s;
    const int es = dps::elem_size(dt);
    const size_t L = dp_shard_len(n, k);
    if (!pairwise_disjoint(recv, k, n * es)) return DP_ERR_ALIAS;
    in_place = true;
    for (int c = 0; c < k && in_place; ++c)
        in_place = (const char *)send[c] == (const char *)recv[c] + (size_t)c * L * (size_t)es;
    if (!in_place) {
        for (int c = 0; c < k; ++c) {
            const size_t nc = (size_t)shard_valid((int64_t)n, (int64_t)L, c);
            for (int r = 0; r < k; ++r)
                if (overlap(span(send[c], nc * es), span(recv[r], n * es))) return DP_ERR_ALIAS;
        }
    }
    return DP_OK;
}

// FSDP step argument checks. with_ws: the caller passes the w_full and dw_full
// workspaces (checked like outputs); without, they are the library's static
// scratch, which no caller buffer can overlap.
dp_status_t check_fsdp(int k, int64_t m_local, int64_t d, int64_t f, const float *const *x_local,
                       const float *const *w_shard, const float *const *dy_local,
                       float *const *w_full, float *const *y_local, float *const *dx_local,
                       float *const *dw_full, float *const *dw_shard, bool with_ws)
{
    if (!valid_k(k) || m_local < 1 || d < 1 || f < 1) return DP_ERR_INVALID_ARG;
    if (m_local > (1 << 24) || d > (1 << 24) || f > (1 << 24)) return DP_ERR_INVALID_ARG;
    if (!ptrs_ok((const void *const *)x_local, k, 4) || !ptrs_ok((const void *const *)w_shard, k, 4) ||
        (with_ws && !ptrs_ok((const void *const *)w_full, k, 4)) ||
        !ptrs_ok((const void *const *)y_local, k, 4))
        return DP_ERR_INVALID_ARG;
    const bool bwd = dy_local != nullptr;
    if (bwd && (!ptrs_ok((const void *const *)dy_local, k, 4) ||
                (with_ws && !ptrs_ok((const void *const *)dw_full, k, 4)) ||
                !ptrs_ok((const void *const *)dw_shard, k, 4)))
        return DP_ERR_INVALID_ARG;
    const bool want_dx = dx_local != nullptr;
    if (want_dx && (!bwd || !ptrs_ok((const void *const *)dx_local, k, 4))) return DP_ERR_INVALID_ARG;
    const int64_t R = (d + k - 1) / k;
    const size_t bx = (size_t)(m_local * d) * 4, bws = (size_t)(R * f) * 4, bdy = (size_t)(m_local * f) * 4;
    const size_t bwf = (size_t)(d * f) * 4, by = (size_t)(m_local * f) * 4;
    // outputs must be disjoint from every input and from each other
    Range ins[3 * DP_MAX_K], outs[5 * DP_MAX_K];
    int ni = 0, no = 0;
    for (int r = 0; r < k; ++r) {
        ins[ni++] = span(x_local[r], bx);
        ins[ni++] = span(w_shard[r], bws);
        if (bwd) ins[ni++] = span(dy_local[r], bdy);
        if (with_ws) outs[no++] = span(w_full[r], bwf);
        outs[no++] = span(y_local[r], by);
        if (bwd) {
            if (with_ws) outs[no++] = span(dw_full[r], bwf);
            outs[no++] = span(dw_shard[r], bws);
        }
        if (want_dx) outs[no++] = span(dx_local[r], bx);
    }
    for (int a = 0; a < no; ++a) {
        for (int b = 0; b < ni; ++b)
            if (overlap(outs[a], ins[b])) return DP_ERR_ALIAS;
        for (int b = a + 1; b < no; ++b)
            if (overlap(outs[a], outs[b])) return DP_ERR_ALIAS;
    }
    return DP_OK;
}

// The FSDP step on validated arguments (see dp_fsdp_layer_ex).
dp_status_t run_fsdp(int k, int64_t m_local, int64_t d, int64_t f, const float *const *x_local,
                     const float *const *w_shard, const float *const *dy_local,
                     float *const *w_full, float *const *y_local, float *const *dx_local,
                     float *const *dw_full, float *const *dw_shard, hipStream_t st)
{
    const bool bwd = dy_local != nullptr;
    const bool want_dx = dx_local != nullptr;
    const int64_t R = (d + k - 1) / k;
    dps::GemmF32Batch g;
    memset(&g, 0, sizeof(g));
    for (int r = 0; r < k; ++r) {
        g.a[r] = x_local[r];
        g.b[r] = w_full[r];
        g.c[r] = y_local[r];
        g.b_shard[r] = w_shard[r];
        g.b_copy[r] = w_full[r];
    }
    g.nb = k;
    g.M = m_local;
    g.N = f;
    g.Kd = d;
    g.trans_a = 0;
    g.b_rows = R;
    // dx_r = dy_r . W^T: [m_local, d], W^T's columns are W's rows (shards)
    dps::GemmF32Batch gx;
    memset(&gx, 0, sizeof(gx));
    for (int r = 0; r < k && want_dx; ++r) {
        gx.a[r] = dy_local[r];
        gx.b[r] = w_full[r];
        gx.c[r] = dx_local[r];
        gx.b_shard[r] = w_shard[r];
    }
    gx.nb = k;
    gx.M = m_local;
    gx.N = d;
    gx.Kd = f;
    gx.trans_b = 1;
    gx.b_rows = R;
    dp_status_t s;
    const bool fwd_fused = dps::gemm_f32_fusable_gather(g, k);
    const bool dx_fused = want_dx && dps::gemm_f32_fusable_gather(gx, k);
    // forward blocks of the one-launch step: 32x32 without dx, 64x64 tiles with it
    const int64_t n_fwd = want_dx ? (m_local / 64) * (f / 64) * k : (m_local / 32) * (f / 32) * k;
    const int64_t n_dx = want_dx ? (m_local / 64) * (d / 64) * k : 0;
    dps::FsdpFwd8 fw8;
    memset(&fw8, 0, sizeof(fw8));
    fw8.nb = k;
    fw8.M = m_local;
    fw8.N = f;
    fw8.Kd = d;
    fw8.b_rows = R;
    // without dx, where the shapes allow: the step as one wave of workgroups,
    // each wave running a forward and a backward chain side by side
    const bool step2 = bwd && !want_dx && k <= 8 && dps::fsdp_step2_ok(k, m_local, d, f);
    // the one-launch step: without dx its forward part is the 32x32 direct block,
    // with dx the 64x64 k-stage tile (beside the dx tiles)
    if (bwd && k <= 8 && dps::fsdp_bwd_fusable(k, m_local, d, f) &&
        (want_dx ? fwd_fused && dx_fused : step2 || dps::fsdp_fwd_direct_ok(fw8)) &&
        n_fwd + n_dx + (d / 32) * (f / 32) <= 0x7fffffffLL) {
        // the whole step in one launch: forward tiles (AllGather folded into
        // the dot) beside backward blocks (ReduceScatter folded into the dW
        // kernel); the two halves share no data
        dps::FsdpStepParams p;
        memset(&p, 0, sizeof(p));
        for (int r = 0; r < k; ++r) {
            p.fwd.a[r] = x_local[r];
            p.fwd.c[r] = y_local[r];
            p.fwd.b_shard[r] = w_shard[r];
            p.fwd.b_copy[r] = w_full[r];
            p.bwd.x[r] = x_local[r];
            p.bwd.dy[r] = dy_local[r];
            p.bwd.dw_full[r] = dw_full[r];
            p.bwd.dw_shard[r] = dw_shard[r];
        }
        p.fwd.nb = k;
        p.fwd.M = m_local;
        p.fwd.N = f;
        p.fwd.Kd = d;
        p.fwd.b_rows = R;
        p.bwd.k = k;
        p.bwd.m = m_local;
        p.bwd.d = d;
        p.bwd.f = f;
        p.bwd.R = R;
        p.tiles_x = (int)(want_dx ? f / 64 : f / 32);
        p.n_fwd = (int)n_fwd;
        if (want_dx) {
            for (int r = 0; r < k; ++r) {
                p.dx.a[r] = dy_local[r];
                p.dx.c[r] = dx_local[r];
                p.dx.b_shard[r] = w_shard[r];
            }
            p.dx.nb = k;
            p.dx.M = m_local;
            p.dx.N = d;
            p.dx.Kd = f;
            p.dx.b_rows = R;
            p.dx.trans_b = 1;
            p.tiles_x_dx = (int)(d / 64);
            p.n_dx = (int)n_dx;
        }
        if (step2) {
            p.n_fwd = (int)((k * m_local / 32) * (f / 64));
            return hip_status(dps::launch_fsdp_step2(p, st));
        }
        // with dx at the fixture sizes: the compile-time-sized step, each wave
        // running a backward, a forward and a dx chain
        if (want_dx && dps::fsdp_step2_ok(k, m_local, d, f) && dps::fsdp_step_k8_ok(p)) {
            p.n_fwd = (int)((k * m_local / 32) * (f / 64));
            return hip_status(dps::launch_fsdp_step2(p, st));
        }
        return hip_status(dps::launch_fsdp_step(p, st));
    }
    if (fwd_fused) {
        // 1+2 in one launch: the dot reads W's rows from the shards, and the
        // tiles of the first tile row write the gathered W into every w_full
        s = hip_status(dps::launch_gemm_f32(g, st));
    } else {
        // 1. forward: all-gather the weight row shards into every rank's W
        s = run_ag((const void *const *)w_shard, (char *const *)w_full, d * f, R * f, k, DP_F32, 0,
                   1, st);
        if (s != DP_OK) return s;
        // 2. local dot y_r = x_r . W
        g.b_rows = 0;
        s = hip_status(dps::launch_gemm_f32(g, st));
    }
    if (s != DP_OK || !bwd) return s;
    // dx = dy . W^T, from the shards where the shapes allow, else from the
    // gathered W (written above)
    if (want_dx) {
        if (!dx_fused) gx.b_rows = 0;
        s = hip_status(dps::launch_gemm_f32(gx, st));
        if (s != DP_OK) return s;
    }
    // 3+4 in one launch where the shapes allow: dW_r = x_r^T . dy_r for every
    // rank and the ReduceScatter of dW from the K blocks in LDS
    if (dps::fsdp_bwd_fusable(k, m_local, d, f)) {
        dps::FsdpBwdParams p;
        memset(&p, 0, sizeof(p));
        for (int r = 0; r < k; ++r) {
            p.x[r] = x_local[r];
            p.dy[r] = dy_local[r];
            p.dw_full[r] = dw_full[r];
            p.dw_shard[r] = dw_shard[r];
        }
        p.k = k;
        p.m = m_local;
        p.d = d;
        p.f = f;
        p.R = R;
        return hip_status(dps::launch_fsdp_bwd_fused(p, st));
    }
    // 3. backward: dW_r = x_r^T . dy_r
    for (int r = 0; r < k; ++r) {
        g.a[r] = x_local[r];
        g.b[r] = dy_local[r];
        g.c[r] = dw_full[r];
    }
    g.M = d;
    g.N = f;
    g.Kd = m_local;
    g.trans_a = 1;
    g.b_rows = 0;
    s = hip_status(dps::launch_gemm_f32(g, st));
    if (s != DP_OK) return s;
    // 4. reduce-scatter dW back to the row shards (sum, pad rows zero)
    return run_rs((const void *const *)dw_full, (char *const *)dw_shard, d * f, R * f, k, DP_F32,
                  dps::kSum, 1.0f, nullptr, 1, 1, st);
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept per device afterwards.
constexpr int kMaxDevices = 64;
std::atomic<char *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

dp_status_t scratch_base(char **base)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return DP_ERR_UNSUPPORTED;
    char *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *q = nullptr;
            e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e);
            p = (char *)q;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *base = p;
    return DP_OK;
}

}  // namespace

extern "C" {

size_t dp_shard_len(size_t n, int k)
{
    if (n == 0 || k < 1) return 0;
    return (n + (size_t)k - 1) / (size_t)k;
}

const char *dp_status_string(int status)
{
    switch (status) {
    case DP_OK: return "DP_OK: success";
    case DP_ERR_INVALID_ARG: return "DP_ERR_INVALID_ARG: invalid argument";
    case DP_ERR_UNSUPPORTED: return "DP_ERR_UNSUPPORTED: unsupported dtype or op";
    case DP_ERR_ALIAS: return "DP_ERR_ALIAS: buffers overlap outside the in-place forms";
    case DP_ERR_HIP: return "DP_ERR_HIP: HIP launch failed";
    case DP_ERR_SCRATCH:
        return "DP_ERR_SCRATCH: the workspaces exceed the library's static scratch buffer";
    default: return "unknown dpsync status";
    }
}

int dp_last_hip_error(void) { return g_last_hip_error; }

int dp_version(void) { return 100; }

dp_status_t dp_reduce_scatter_ex(const void *const *send, void *const *recv, size_t n, int k, int dt,
                                 int op, int s_chunks, const dp_launch_opts_t *opts, void *stream)
{
    int max_wg;
    bool lean, in_place;
    if (!opts_ok(opts, max_wg, nullptr, nullptr, &lean)) return DP_ERR_INVALID_ARG;
    dp_status_t s = check_rs(send, recv, n, k, dt, op, s_chunks, in_place);
    if (s != DP_OK || n == 0) return s;
    const size_t L = dp_shard_len(n, k);
    int ep;
    float scale;
    pick_epilogue(op, k, ep, scale);
    return run_rs(send, (char *const *)recv, (int64_t)n, (int64_t)L, k, dt, ep, scale, nullptr, 1,
                  s_chunks, (hipStream_t)stream, max_wg, lean);
}

dp_status_t dp_reduce_scatter(const void *const *send, void *const *recv, size_t n, int k, int dt,
                              int op, int s_chunks, void *stream)
{
    return dp_reduce_scatter_ex(send, recv, n, k, dt, op, s_chunks, nullptr, stream);
}

dp_status_t dp_all_gather_ex(const void *const *send, void *const *recv, size_t n, int k, int dt,
                             int s_chunks, const dp_launch_opts_t *opts, void *stream)
{
    int max_wg;
    bool in_place;
    if (!opts_ok(opts, max_wg)) return DP_ERR_INVALID_ARG;
    dp_status_t s = check_ag(send, recv, n, k, dt, s_chunks, in_place);
    if (s != DP_OK || n == 0) return s;
    const size_t L = dp_shard_len(n, k);
    return run_ag(send, (char *const *)recv, (int64_t)n, (int64_t)L, k, dt, in_place ? 1 : 0,
                  s_chunks, (hipStream_t)stream, max_wg);
}

dp_status_t dp_all_gather(const void *const *send, void *const *recv, size_t n, int k, int dt,
                          int s_chunks, void *stream)
{
    return dp_all_gather_ex(send, recv, n, k, dt, s_chunks, nullptr, stream);
}

dp_status_t dp_reduce_scatter_all_gather(const void *const *rs_send, void *const *rs_recv,
                                         size_t rs_n, const void *const *ag_send,
                                         void *const *ag_recv, size_t ag_n, int k, int dt, int op,
                                         int s_chunks, void *stream)
{
    bool rs_in_place, ag_in_place;
    dp_status_t s = check_rs(rs_send, rs_recv, rs_n, k, dt, op, s_chunks, rs_in_place);
    if (s != DP_OK) return s;
    s = check_ag(ag_send, ag_recv, ag_n, k, dt, s_chunks, ag_in_place);
    if (s != DP_OK) return s;
    if (rs_n == 0 && ag_n == 0) return DP_OK;
    const int es = dps::elem_size(dt);
    const size_t Lr = dp_shard_len(rs_n, k), La = dp_shard_len(ag_n, k);
    if (rs_n && ag_n) {
        // the two operations must not touch each other's buffers
        for (int i = 0; i < k; ++i) {
            const Range r_in = span(rs_send[i], rs_n * es), r_out = span(rs_recv[i], Lr * es);
            for (int j = 0; j < k; ++j) {
                const Range a_in = span(ag_send[j], La * es), a_out = span(ag_recv[j], ag_n * es);
                if (overlap(r_in, a_in) || overlap(r_in, a_out) || overlap(r_out, a_in) ||
                    overlap(r_out, a_out))
                    return DP_ERR_ALIAS;
            }
        }
    }
    int ep;
    float scale;
    pick_epilogue(op, k, ep, scale);
    hipStream_t st = (hipStream_t)stream;
    // a pipeline step: the shards written here are gathered by the next step,
    // and the shards gathered here were written by the previous one
    if (ag_n == 0)
        return run_rs(rs_send, (char *const *)rs_recv, (int64_t)rs_n, (int64_t)Lr, k, dt, ep, scale,
                      nullptr, 1, s_chunks, st, 0, false, true);
    if (rs_n == 0)
        return run_ag(ag_send, (char *const *)ag_recv, (int64_t)ag_n, (int64_t)La, k, dt,
                      ag_in_place ? 1 : 0, s_chunks, st, 0);
    dps::RsParams rp;
    dps::AgParams ap;
    memset(&rp, 0, sizeof(rp));
    memset(&ap, 0, sizeof(ap));
    for (int r = 0; r < k; ++r) {
        rp.src[r] = (const char *)rs_send[r];
        rp.dst[r] = (char *)rs_recv[r];
        rp.w[r] = 1.0f;
        ap.src[r] = (const char *)ag_send[r];
        ap.dst[r] = (char *)ag_recv[r];
    }
    rp.scale = scale;
    rp.write_pads = 1;
    rp.n = (long long)rs_n;
    rp.L = (long long)Lr;
    rp.k = k;
    rp.S = s_chunks;
    ap.skip_own = ag_in_place ? 1 : 0;
    ap.n = (long long)ag_n;
    ap.L = (long long)La;
    ap.k = k;
    ap.S = s_chunks;
    return hip_status(dps::launch_rsag(rp, ap, dt, ep, st));
}

dp_status_t dp_all_reduce_ex(const void *const *send, void *const *recv, size_t n, int k, int dt,
                             int op, int s_chunks, const dp_launch_opts_t *opts, void *stream)
{
    int max_wg;
    bool two_phase, lean;
    if (!opts_ok(opts, max_wg, nullptr, &two_phase, &lean)) return DP_ERR_INVALID_ARG;
    dp_status_t s = validate_rs_ag_common(send, recv, n, k, dt, s_chunks);
    if (s != DP_OK || n == 0) return s;
    if (op != DP_SUM && op != DP_AVG) return DP_ERR_UNSUPPORTED;
    if (dt == DP_I32 && op != DP_SUM) return DP_ERR_UNSUPPORTED;
    s = check_ar_alias(send, recv, n, k, dps::elem_size(dt));
    if (s != DP_OK) return s;
    int ep;
    float scale;
    pick_epilogue(op, k, ep, scale);
    return run_ar(send, recv, n, k, dt, ep, scale, nullptr, s_chunks, (hipStream_t)stream, max_wg,
                  two_phase, lean);
}

dp_status_t dp_all_reduce(const void *const *send, void *const *recv, size_t n, int k, int dt,
                          int op, int s_chunks, void *stream)
{
    return dp_all_reduce_ex(send, recv, n, k, dt, op, s_chunks, nullptr, stream);
}

dp_status_t dp_weighted_reduce(const void *const *send, void *const *recv, const int64_t *tokens,
                               size_t n, int k, int dt, int s_chunks, void *stream)
{
    return dp_weighted_reduce_ex(send, recv, tokens, n, k, dt, s_chunks, nullptr, stream);
}

dp_status_t dp_weighted_reduce_ex(const void *const *send, void *const *recv,
                                  const int64_t *tokens, size_t n, int k, int dt, int s_chunks,
                                  const dp_launch_opts_t *opts, void *stream)
{
    int max_wg;
    bool two_phase, lean;
    if (!opts_ok(opts, max_wg, nullptr, &two_phase, &lean)) return DP_ERR_INVALID_ARG;
    dp_status_t s = validate_rs_ag_common(send, recv, n, k, dt, s_chunks);
    if (s != DP_OK) return s;
    if (dt == DP_I32) return DP_ERR_UNSUPPORTED;
    if (!tokens) return DP_ERR_INVALID_ARG;
    float w[DP_MAX_K];
    int64_t total = 0;
    for (int r = 0; r < k; ++r) {
        if (tokens[r] < 0 || tokens[r] > ((int64_t)1 << 56)) return DP_ERR_INVALID_ARG;
        total += tokens[r];
        w[r] = (float)tokens[r];
    }
    if (total <= 0) return DP_ERR_INVALID_ARG;
    if (n == 0) return DP_OK;
    s = check_ar_alias(send, recv, n, k, dps::elem_size(dt));
    if (s != DP_OK) return s;
    return run_ar(send, recv, n, k, dt, dps::kWeighted, (float)total, w, s_chunks,
                  (hipStream_t)stream, max_wg, two_phase, lean);
}

dp_status_t dp_fsdp_layer(int k, int64_t m_local, int64_t d, int64_t f,
                          const float *const *x_local, const float *const *w_shard,
                          const float *const *dy_local, float *const *w_full,
                          float *const *y_local, float *const *dw_full, float *const *dw_shard,
                          void *stream)
{
    return dp_fsdp_layer_ex(k, m_local, d, f, x_local, w_shard, dy_local, w_full, y_local,
                            nullptr, dw_full, dw_shard, stream);
}

dp_status_t dp_fsdp_layer_ex(int k, int64_t m_local, int64_t d, int64_t f,
                             const float *const *x_local, const float *const *w_shard,
                             const float *const *dy_local, float *const *w_full,
                             float *const *y_local, float *const *dx_local,
                             float *const *dw_full, float *const *dw_shard, void *stream)
{
    dp_status_t s0 = check_fsdp(k, m_local, d, f, x_local, w_shard, dy_local, w_full, y_local,
                                dx_local, dw_full, dw_shard, true);
    if (s0 != DP_OK) return s0;
    return run_fsdp(k, m_local, d, f, x_local, w_shard, dy_local, w_full, y_local, dx_local,
                    dw_full, dw_shard, (hipStream_t)stream);
}

dp_status_t dp_fsdp_layer_static(int k, int64_t m_local, int64_t d, int64_t f,
                                 const float *const *x_local, const float *const *w_shard,
                                 const float *const *dy_local, float *const *y_local,
                                 float *const *dx_local, float *const *dw_shard, void *stream)
{
    dp_status_t s = check_fsdp(k, m_local, d, f, x_local, w_shard, dy_local, nullptr, y_local,
                               dx_local, nullptr, dw_shard, false);
    if (s != DP_OK) return s;
    // K gathered weights and K weight gradients, each [d, f] fp32, every one
    // starting on a 256-byte boundary (the alignment a caller's allocations
    // have, so the same kernels are chosen as with caller workspaces)
    const size_t region = ((size_t)(d * f) * 4 + 255) / 256 * 256;
    if ((size_t)(2 * k) * region > (size_t)DP_STATIC_SCRATCH_BYTES) return DP_ERR_SCRATCH;
    char *base = nullptr;
    s = scratch_base(&base);
    if (s != DP_OK) return s;
    float *w_full[DP_MAX_K], *dw_full[DP_MAX_K];
    for (int r = 0; r < k; ++r) {
        w_full[r] = (float *)(base + (size_t)r * region);
        dw_full[r] = (float *)(base + (size_t)(k + r) * region);
    }
    return run_fsdp(k, m_local, d, f, x_local, w_shard, dy_local, w_full, y_local, dx_local,
                    dw_full, dw_shard, (hipStream_t)stream);
}

dp_status_t dp_gemm_bf16_ex(const void *a, const void *b, void *c, int64_t m, int64_t n,
                            int64_t kk, const dp_launch_opts_t *opts, void *stream)
{
    int max_wg;
    bool share_cu, lean, b_nk;
    if (!opts_ok(opts, max_wg, &share_cu, nullptr, &lean, &b_nk)) return DP_ERR_INVALID_ARG;
    if (!a || !b || !c || m < 1 || n < 1 || kk < 1) return DP_ERR_INVALID_ARG;
    if (m > (1 << 24) || n > (1 << 24) || kk > (1 << 24)) return DP_ERR_INVALID_ARG;
    if (((uintptr_t)a & 1) || ((uintptr_t)b & 1) || ((uintptr_t)c & 1)) return DP_ERR_INVALID_ARG;
    const Range rc = span(c, (size_t)(m * n) * 2);
    if (overlap(rc, span(a, (size_t)(m * kk) * 2)) || overlap(rc, span(b, (size_t)(n * kk) * 2)))
        return DP_ERR_ALIAS;
    return hip_status(dps::launch_gemm_bf16(a, b, c, m, n, kk, gemm_variant(share_cu, lean),
                                            !b_nk, (hipStream_t)stream));
}

dp_status_t dp_backward_allreduce_overlap(int k, int n_pieces, const dp_grad_piece_t *pieces,
                                          int64_t t, const void *const *dy, const void *const *x,
                                          void *const *grad, void *const *out, int64_t total,
                                          int64_t bucket_elems, int op,
                                          const dp_launch_opts_t *opts, void *compute_stream,
                                          void *comm_stream, void *const *events, int n_events)
{
    int max_wg;
    bool share_cu, two_phase, lean;
    if (!opts_ok(opts, max_wg, &share_cu, &two_phase, &lean)) return DP_ERR_INVALID_ARG;
    if (!valid_k(k) || n_pieces < 1 || !pieces || t < 1 || t > (1 << 24) || total < 1 ||
        bucket_elems < 1 || !size_ok((size_t)total, 2))
        return DP_ERR_INVALID_ARG;
    if (op != DP_SUM && op != DP_AVG) return DP_ERR_UNSUPPORTED;
    if (t % 8 != 0) return DP_ERR_UNSUPPORTED;
    // the pieces tile [0, total) in order
    int64_t off = 0;
    for (int g = 0; g < n_pieces; ++g) {
        const dp_grad_piece_t &p = pieces[g];
        if (p.offset != off || p.m < 1 || p.n < 1 || p.m > (1 << 24) || p.n > (1 << 24))
            return DP_ERR_INVALID_ARG;
        off += p.m * p.n;
        if (off > total) return DP_ERR_INVALID_ARG;
    }
    if (off != total) return DP_ERR_INVALID_ARG;
    if (!dy || !x || !ptrs_ok((const void *const *)grad, k, 2) ||
        !ptrs_ok((const void *const *)out, k, 2))
        return DP_ERR_INVALID_ARG;
    for (int i = 0; i < n_pieces * k; ++i) {
        if (!dy[i] || !x[i]) return DP_ERR_INVALID_ARG;
        if (((uintptr_t)dy[i] & 15) || ((uintptr_t)x[i] & 15)) return DP_ERR_UNSUPPORTED;
    }
    const size_t bytes = (size_t)total * 2;
    if (!pairwise_disjoint(grad, k, bytes)) return DP_ERR_ALIAS;
    dp_status_t s = check_ar_alias((const void *const *)grad, out, (size_t)total, k, 2);
    if (s != DP_OK) return s;
    for (int g = 0; g < n_pieces; ++g)
        for (int r = 0; r < k; ++r) {
            const int i = g * k + r;
            const Range ra = span(dy[i], (size_t)(pieces[g].m * t) * 2);
            const Range rb = span(x[i], (size_t)(pieces[g].n * t) * 2);
            for (int q = 0; q < k; ++q) {
                const Range rg = span(grad[q], bytes), ro = span(out[q], bytes);
                if (overlap(ra, rg) || overlap(rb, rg) || overlap(ra, ro) || overlap(rb, ro))
                    return DP_ERR_ALIAS;
            }
        }
    const int64_t nb = (total + bucket_elems - 1) / bucket_elems;
    hipStream_t cs = (hipStream_t)compute_stream, ms = (hipStream_t)comm_stream;
    const bool two_streams = cs != ms;
    if (two_streams) {
        if (!events || n_events < nb) return DP_ERR_INVALID_ARG;
        for (int64_t b = 0; b < nb; ++b)
            if (!events[b]) return DP_ERR_INVALID_ARG;
    }
    int ep;
    float scale;
    pick_epilogue(op, k, ep, scale);

    // Backward order: piece g's gradient for every rank, then every bucket that
    // is now complete for all ranks goes to the comm stream, in bucket order.
    int64_t next = 0;
    for (int g = 0; g < n_pieces; ++g) {
        const dp_grad_piece_t &p = pieces[g];
        for (int r = 0; r < k; ++r) {
            char *c = (char *)grad[r] + (size_t)p.offset * 2;
            hipError_t e = dps::launch_gemm_bf16(dy[g * k + r], x[g * k + r], c, p.m, p.n, t,
                                                 gemm_variant(share_cu, lean), false, cs);
            if (e != hipSuccess) return hip_status(e);
        }
        const int64_t done = p.offset + p.m * p.n;
        for (; next < nb; ++next) {
            const int64_t b0 = next * bucket_elems;
            const int64_t bn = (total - b0 < bucket_elems) ? total - b0 : bucket_elems;
            if (b0 + bn > done) break;
            const void *src[DP_MAX_K];
            void *dst[DP_MAX_K];
            for (int r = 0; r < k; ++r) {
                src[r] = (const char *)grad[r] + (size_t)b0 * 2;
                dst[r] = (char *)out[r] + (size_t)b0 * 2;
            }
            hipStream_t st = cs;
            if (two_streams) {
                hipError_t e = hipEventRecord((hipEvent_t)events[next], cs);
                if (e == hipSuccess) e = hipStreamWaitEvent(ms, (hipEvent_t)events[next], 0);
                if (e != hipSuccess) return hip_status(e);
                st = ms;
            }
            s = run_ar(src, dst, (size_t)bn, k, DP_BF16, ep, scale, nullptr, 1, st, max_wg, two_phase,
                       lean);
            if (s != DP_OK) return s;
        }
    }
    return DP_OK;
}

dp_status_t dp_scatter_accumulate(const void *const *grads, int np, int dt, float *const *acc,
                                  size_t n, int k, void *stream)
{
    if (!valid_k(k) || np < 1 || np > DP_MAX_K) return DP_ERR_INVALID_ARG;
    if (dt != DP_F32 && dt != DP_BF16) return DP_ERR_UNSUPPORTED;
    const int es = dps::elem_size(dt);
    if (!size_ok(n, es)) return DP_ERR_INVALID_ARG;
    if (n == 0) return (grads && acc) ? DP_OK : DP_ERR_INVALID_ARG;
    if (!ptrs_ok(grads, np, es) || !ptrs_ok((const void *const *)acc, k, 4))
        return DP_ERR_INVALID_ARG;
    const size_t L = dp_shard_len(n, k);
    for (int c = 0; c < k; ++c)
        for (int i = 0; i < np; ++i)
            if (overlap(span(acc[c], L * 4), span(grads[i], n * es))) return DP_ERR_ALIAS;
    if (!pairwise_disjoint((void *const *)acc, k, L * 4)) return DP_ERR_ALIAS;
    dps::SaParams p;
    memset(&p, 0, sizeof(p));
    for (int i = 0; i < np; ++i) p.g[i] = (const char *)grads[i];
    for (int c = 0; c < k; ++c) p.acc[c] = acc[c];
    p.n = (long long)n;
    p.L = (long long)L;
    p.np = np;
    p.k = k;
    return hip_status(dps::launch_scatter_accumulate(p, dt, (hipStream_t)stream));
}

dp_status_t dp_settle(float *const *acc, void *const *out, size_t n, int k, int dt, float divisor,
                      int reset, void *stream)
{
    if (!valid_k(k)) return DP_ERR_INVALID_ARG;
    if (dt != DP_F32 && dt != DP_BF16) return DP_ERR_UNSUPPORTED;
    const int es = dps::elem_size(dt);
    if (!size_ok(n, 4)) return DP_ERR_INVALID_ARG;
    uint32_t bits;
    memcpy(&bits, &divisor, 4);
    const uint32_t ex = (bits >> 23) & 0xffu;
    if (ex == 0xffu || (bits & 0x7fffffffu) == 0) return DP_ERR_INVALID_ARG;
    if (n == 0) return (acc && out) ? DP_OK : DP_ERR_INVALID_ARG;
    if (!ptrs_ok((const void *const *)acc, k, 4) || !ptrs_ok((const void *const *)out, k, es))
        return DP_ERR_INVALID_ARG;
    const size_t L = dp_shard_len(n, k);
    const bool in_place_ok = dt == DP_F32 && !reset;
    for (int c = 0; c < k; ++c)
        for (int q = 0; q < k; ++q) {
            if (in_place_ok && c == q && out[c] == (void *)acc[c]) continue;
            if (overlap(span(out[c], L * es), span(acc[q], L * 4))) return DP_ERR_ALIAS;
        }
    if (!pairwise_disjoint((void *const *)acc, k, L * 4) || !pairwise_disjoint(out, k, L * es))
        return DP_ERR_ALIAS;
    dps::SettleParams p;
    memset(&p, 0, sizeof(p));
    for (int c = 0; c < k; ++c) {
        p.acc[c] = acc[c];
        p.out[c] = (char *)out[c];
    }
    // a normal power of two (zero fraction bits) has an exact reciprocal, and
    // multiplying by it rounds the same real number as dividing
    const bool mul = (bits & 0x7fffffu) == 0 && ex != 0;
    p.scale = mul ? 1.0f / divisor : divisor;
    p.reset = reset ? 1 : 0;
    p.n = (long long)n;
    p.L = (long long)L;
    p.k = k;
    return hip_status(dps::launch_settle(p, dt, mul, (hipStream_t)stream));
}

dp_status_t dp_gemm_bf16(const void *a, const void *b, void *c, int64_t m, int64_t n, int64_t kk,
                         void *stream)
{
    return dp_gemm_bf16_ex(a, b, c, m, n, kk, nullptr, stream);
}

}  // extern "C"
