/*
 * dp_oracle.c -- plain, slow CPU reference for data-parallel gradient and
 * parameter synchronisation.
 *
 * TEST INFRASTRUCTURE ONLY. This is the oracle the GPU library is checked
 * against. Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it; the product path never does. It shares no code,
 * header or constant with the GPU library.
 *
 * What it computes (K ranks, n elements per rank, L = ceil(n/K)):
 *
 *  - ReduceScatter (CMU 11-868 L14-L15 notes, section "Ring AllReduce:
 *    ReduceScatter, then AllGather", phase 1; "Sharding and Parallelism",
 *    section "The cost of the inserted collectives", the T_RS,ring equation):
 *    every rank starts with a reducible n-element buffer and rank c ends with
 *    shard c, the sum over ranks of elements [cL, min((c+1)L, n)).
 *    The sum is taken in the order a unidirectional ring r -> r+1 produces
 *    when rank c ends up owning chunk c: the partial for chunk c starts at
 *    rank c+1 and each hop adds the receiver's own value on the right, so the
 *    fold order is rho_c = (c+1, c+2, ..., c+K-1, c) mod K, as a left fold
 *    whose first operand is taken as it is. Rank order 0..K-1 is kept as an
 *    alternative reading (order = 1).
 *  - Averaging (same notes, "Intuition: data parallelism has only one thing
 *    to synchronize", step 3): one IEEE division of the fp32 sum by K.
 *  - Token weighting (uneven per-rank token counts, "Using ODC to Accelerate
 *    AMD SFT Training", section "Why FSDP is Slow ... Workload-imbalance
 *    Bubble"): out = sum_r t_r*g_r / sum_r t_r, with p_r = f32(t_r) * g_r
 *    folded in ring order and one division by f32(sum_r t_r) at the end.
 *  - Padding for n not divisible by K ("Sharding and Parallelism", section
 *    "Global arrays and device-local shards"): shards are L long; the last
 *    ones are short or empty and their pad elements are written as zero.
 *  - AllGather (CMU notes, phase 2; T_AG,ring equation): every rank receives
 *    all n valid elements; pads are dropped.
 *  - AllReduce = ReduceScatter then AllGather (CMU notes, section "NCCL's five
 *    building blocks"; T_AR,ring equation).
 *  - FSDP layer ("Sharding and Parallelism", sections "Real HLO before and
 *    after partitioning" (FSDP fixture) and "FSDP and ZeRO"): all-gather the
 *    row shards of w, local y = x_local * W, dW_r = x_local^T * dy_local,
 *    reduce-scatter dW back to row shards. GEMM references are in fp64.
 *
 * Arithmetic: every float operation below is one IEEE binary32 operation with
 * round-to-nearest-even (x86-64 SSE, built with -ffp-contract=off, no fast
 * math). bf16 values are widened exactly to fp32 and rounded back with
 * round-to-nearest-even. int32 sums wrap (done in uint32).
 *
 * Parallelism: an optional thread count splits the element loop across
 * OpenMP threads; each element is still computed by one thread in the same
 * order, so results do not depend on it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_SUM 0
#define ORC_AVG 1

/* ------------------------------------------------------------------ plan */

int64_t orc_shard_len(int64_t n, int k)
{
    if (n <= 0 || k <= 0) return 0;
    return (n + k - 1) / k;
}

/* number of valid (non-pad) elements of shard c */
int64_t orc_shard_valid(int64_t n, int64_t L, int c)
{
    int64_t lo = (int64_t)c * L;
    if (lo >= n) return 0;
    return (n - lo < L) ? n - lo : L;
}

/* rank whose value is the m-th operand of shard c's fold */
int orc_fold_rank(int c, int m, int k, int order)
{
    if (order == 1) return m;
    return (c + 1 + m) % k;
}

/* ------------------------------------------------------------------ bf16 */

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays NaN (quiet, sign
 * kept); +-Inf stays Inf; overflow rounds to Inf. */
uint16_t orc_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;          /* truncated result */
    uint32_t drop = u & 0xffffu;      /* discarded bits, in units of 2^-16 ulp */
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u;                   /* a carry into the exponent is correct */
    return (uint16_t)keep;
}

/* ------------------------------------------------------- per-element folds */

static float fold_f32(const float *const *x, int64_t i, int c, int k, int order)
{
    float acc = x[orc_fold_rank(c, 0, k, order)][i];
    for (int m = 1; m < k; ++m)
        acc = acc + x[orc_fold_rank(c, m, k, order)][i];
    return acc;
}

static float fold_bf16(const uint16_t *const *x, int64_t i, int c, int k, int order)
{
    float acc = orc_bf16_to_f32(x[orc_fold_rank(c, 0, k, order)][i]);
    for (int m = 1; m < k; ++m)
        acc = acc + orc_bf16_to_f32(x[orc_fold_rank(c, m, k, order)][i]);
    return acc;
}

static uint32_t fold_i32(const int32_t *const *x, int64_t i, int c, int k, int order)
{
    uint32_t acc = (uint32_t)x[orc_fold_rank(c, 0, k, order)][i];
    for (int m = 1; m < k; ++m)
        acc = acc + (uint32_t)x[orc_fold_rank(c, m, k, order)][i];
    return acc;
}

static float fold_weighted_f32(const float *const *g, const float *w, int64_t i,
                               int c, int k, int order)
{
    int r0 = orc_fold_rank(c, 0, k, order);
    float acc = w[r0] * g[r0][i];
    for (int m = 1; m < k; ++m) {
        int r = orc_fold_rank(c, m, k, order);
        float p = w[r] * g[r][i];
        acc = acc + p;
    }
    return acc;
}

static float fold_weighted_bf16(const uint16_t *const *g, const float *w, int64_t i,
                                int c, int k, int order)
{
    int r0 = orc_fold_rank(c, 0, k, order);
    float acc = w[r0] * orc_bf16_to_f32(g[r0][i]);
    for (int m = 1; m < k; ++m) {
        int r = orc_fold_rank(c, m, k, order);
        float p = w[r] * orc_bf16_to_f32(g[r][i]);
        acc = acc + p;
    }
    return acc;
}

/* f32(t_r) for each rank and f32 of the int64 total; -1 if invalid */
static int token_weights(const int64_t *t, int k, float *w, float *total)
{
    int64_t sum = 0;
    for (int r = 0; r < k; ++r) {
        if (t[r] < 0) return -1;
        sum += t[r];
        w[r] = (float)t[r];
    }
    if (sum <= 0) return -1;
    *total = (float)sum;
    return 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    omp_set_num_threads(nthreads > 0 ? nthreads : 1);
#else
    (void)nthreads;
#endif
}

/* ------------------------------------------------------------ ReduceScatter
 * out[c] points at shard c's output: L elements, of which the first
 * orc_shard_valid(n, L, c) are reduced values and the rest pads (zero),
 * written only when write_pads is set. L must be >= ceil(n/k).
 */

void orc_rs_f32(const float *const *x, float *const *out, int64_t n, int64_t L,
                int k, int op, int order, int write_pads, int nthreads)
{
    set_threads(nthreads);
    for (int c = 0; c < k; ++c) {
        int64_t nc = orc_shard_valid(n, L, c);
        int64_t base = (int64_t)c * L;
        float *o = out[c];
#pragma omp parallel for schedule(static) if (nthreads > 1)
        for (int64_t j = 0; j < nc; ++j) {
            float acc = fold_f32(x, base + j, c, k, order);
            if (op == ORC_AVG) acc = acc / (float)k;
            o[j] = acc;
        }
        if (write_pads)
            for (int64_t j = nc; j < L; ++j) o[j] = 0.0f;
    }
}

void orc_rs_bf16(const uint16_t *const *x, uint16_t *const *out, int64_t n, int64_t L,
                 int k, int op, int order, int write_pads, int nthreads)
{
    set_threads(nthreads);
    for (int c = 0; c < k; ++c) {
        int64_t nc = orc_shard_valid(n, L, c);
        int64_t base = (int64_t)c * L;
        uint16_t *o = out[c];
#pragma omp parallel for schedule(static) if (nthreads > 1)
        for (int64_t j = 0; j < nc; ++j) {
            float acc = fold_bf16(x, base + j, c, k, order);
            if (op == ORC_AVG) acc = acc / (float)k;
            o[j] = orc_bf16_from_f32(acc);
        }
        if (write_pads)
            for (int64_t j = nc; j < L; ++j) o[j] = 0;
    }
}

void orc_rs_i32(const int32_t *const *x, int32_t *const *out, int64_t n, int64_t L,
                int k, int order, int write_pads, int nthreads)
{
    set_threads(nthreads);
    for (int c = 0; c < k; ++c) {
        int64_t nc = orc_shard_valid(n, L, c);
        int64_t base = (int64_t)c * L;
        int32_t *o = out[c];
#pragma omp parallel for schedule(static) if (nthreads > 1)
        for (int64_t j = 0; j < nc; ++j)
            o[j] = (int32_t)fold_i32(x, base + j, c, k, order);
        if (write_pads)
            for (int64_t j = nc; j < L; ++j) o[j] = 0;
    }
}

/* returns 0, or -1 when a token count is negative or the total is not positive */
int orc_rs_weighted_f32(const float *const *g, float *const *out, const int64_t *tokens,
                        int64_t n, int64_t L, int k, int order, int write_pads, int nthreads)
{
    float w[256], total;
    if (k > 256 || token_weights(tokens, k, w, &total) != 0) return -1;
    set_threads(nthreads);
    for (int c = 0; c < k; ++c) {
        int64_t nc = orc_shard_valid(n, L, c);
        int64_t base = (int64_t)c * L;
        float *o = out[c];
#pragma omp parallel for schedule(static) if (nthreads > 1)
        for (int64_t j = 0; j < nc; ++j)
            o[j] = fold_weighted_f32(g, w, base + j, c, k, order) / total;
        if (write_pads)
            for (int64_t j = nc; j < L; ++j) o[j] = 0.0f;
    }
    return 0;
}

int orc_rs_weighted_bf16(const uint16_t *const *g, uint16_t *const *out,
                         const int64_t *tokens, int64_t n, int64_t L, int k, int order,
                         int write_pads, int nthreads)
{
    float w[256], total;
    if (k > 256 || token_weights(tokens, k, w, &total) != 0) return -1;
    set_threads(nthreads);
    for (int c = 0; c < k; ++c) {
        int64_t nc = orc_shard_valid(n, L, c);
        int64_t base = (int64_t)c * L;
        uint16_t *o = out[c];
#pragma omp parallel for schedule(static) if (nthreads > 1)
        for (int64_t j = 0; j < nc; ++j)
            o[j] = orc_bf16_from_f32(fold_weighted_bf16(g, w, base + j, c, k, order) / total);
        if (write_pads)
            for (int64_t j = nc; j < L; ++j) o[j] = 0;
    }
    return 0;
}

/* ------------------------------------------------- sampled ReduceScatter
 * Value of the reduced element at global indices idx[0..count) (each < n),
 * i.e. shard c = idx / L, element idx - c*L. Same folds as above. */

void orc_rs_f32_at(const float *const *x, const int64_t *idx, int64_t count, int64_t L,
                   int k, int op, int order, float *vals)
{
    for (int64_t s = 0; s < count; ++s) {
        int c = (int)(idx[s] / L);
        float acc = fold_f32(x, idx[s], c, k, order);
        if (op == ORC_AVG) acc = acc / (float)k;
        vals[s] = acc;
    }
}

void orc_rs_bf16_at(const uint16_t *const *x, const int64_t *idx, int64_t count, int64_t L,
                    int k, int op, int order, uint16_t *vals)
{
    for (int64_t s = 0; s < count; ++s) {
        int c = (int)(idx[s] / L);
        float acc = fold_bf16(x, idx[s], c, k, order);
        if (op == ORC_AVG) acc = acc / (float)k;
        vals[s] = orc_bf16_from_f32(acc);
    }
}

/* Folds of compact samples: sample s has the K rank values x[r][s] and
 * belongs to shard shard_id[s], whose ring order it is folded in. */
void orc_fold_f32_at(const float *const *x, const int32_t *shard_id, int64_t count, int k,
                     int op, int order, float *vals)
{
    for (int64_t s = 0; s < count; ++s) {
        float acc = fold_f32(x, s, shard_id[s], k, order);
        if (op == ORC_AVG) acc = acc / (float)k;
        vals[s] = acc;
    }
}

void orc_fold_bf16_at(const uint16_t *const *x, const int32_t *shard_id, int64_t count, int k,
                      int op, int order, uint16_t *vals)
{
    for (int64_t s = 0; s < count; ++s) {
        float acc = fold_bf16(x, s, shard_id[s], k, order);
        if (op == ORC_AVG) acc = acc / (float)k;
        vals[s] = orc_bf16_from_f32(acc);
    }
}

/* ------------------------------------------------- scatter-accumulate, settle
 * On-demand communication ("Using ODC to Accelerate AMD SFT Training", section
 * "From Collective Primitives to Two One-sided P2P Primitives", Figure 2): a
 * rank that has computed a gradient pushes each shard of it to the shard's
 * owner, which adds it into its gradient accumulator Acc; after the minibatch
 * one settle makes the accumulated shards final (section "From Per-iteration
 * to Per-minibatch Synchronization").
 *
 * Push of one gradient g (n elements, shard length L, k owners):
 *   acc[c][j] = acc[c][j] + f32(g[c*L + j])   for every c and j < n_c,
 * one fp32 addition per element, in the order the pushes are made.
 * Settle: out[c][j] = cast(acc[c][j] / divisor) for j < n_c, pads zero. */

/* dtype of g: 0 = f32, 1 = bf16 */
void orc_scatter_accumulate(int dtype, const void *g, float *const *acc, int64_t n, int64_t L,
                            int k)
{
    for (int c = 0; c < k; ++c) {
        int64_t nc = orc_shard_valid(n, L, c);
        for (int64_t j = 0; j < nc; ++j) {
            int64_t i = (int64_t)c * L + j;
            float v = dtype == 1 ? orc_bf16_to_f32(((const uint16_t *)g)[i]) : ((const float *)g)[i];
            acc[c][j] = acc[c][j] + v;
        }
    }
}

/* dtype of out: 0 = f32, 1 = bf16 */
void orc_settle(int dtype, const float *const *acc, void *const *out, int64_t n, int64_t L, int k,
                float divisor)
{
    for (int c = 0; c < k; ++c) {
        int64_t nc = orc_shard_valid(n, L, c);
        for (int64_t j = 0; j < L; ++j) {
            float v = j < nc ? acc[c][j] / divisor : 0.0f;
            if (dtype == 1) ((uint16_t *)out[c])[j] = j < nc ? orc_bf16_from_f32(v) : 0;
            else ((float *)out[c])[j] = v;
        }
    }
}

/* -------------------------------------------------------------- AllGather
 * out[r][i] = shard[i / L][i mod L] for every rank r and 0 <= i < n. */

void orc_ag(int esize, const void *const *shard, void *const *out, int64_t n, int64_t L,
            int k, int nthreads)
{
    set_threads(nthreads);
    for (int r = 0; r < k; ++r) {
        char *o = (char *)out[r];
#pragma omp parallel for schedule(static) if (nthreads > 1)
        for (int64_t i = 0; i < n; ++i) {
            int64_t c = i / L;
            const char *src = (const char *)shard[c] + (i - c * L) * esize;
            memcpy(o + i * esize, src, (size_t)esize);
        }
    }
}

/* -------------------------------------------------------------- AllReduce
 * AllGather of the ReduceScatter result. out[r] may equal x[r]. */

static void **alloc_shards(int k, int64_t L, int esize)
{
    void **sh = (void **)calloc((size_t)k, sizeof(void *));
    if (!sh) return NULL;
    for (int c = 0; c < k; ++c) {
        sh[c] = calloc((size_t)(L > 0 ? L : 1), (size_t)esize);
        if (!sh[c]) {
            for (int q = 0; q < c; ++q) free(sh[q]);
            free(sh);
            return NULL;
        }
    }
    return sh;
}

static void free_shards(void **sh, int k)
{
    for (int c = 0; c < k; ++c) free(sh[c]);
    free(sh);
}

/* dtype: 0 = f32, 1 = bf16, 2 = i32; op: 0 sum, 1 avg; returns 0 or -1 */
int orc_ar(int dtype, const void *const *x, void *const *out, int64_t n, int k, int op,
           int order, int nthreads)
{
    int esize = dtype == 1 ? 2 : 4;
    int64_t L = orc_shard_len(n, k);
    void **sh = alloc_shards(k, L, esize);
    if (!sh) return -1;
    if (dtype == 0)
        orc_rs_f32((const float *const *)x, (float *const *)sh, n, L, k, op, order, 1, nthreads);
    else if (dtype == 1)
        orc_rs_bf16((const uint16_t *const *)x, (uint16_t *const *)sh, n, L, k, op, order, 1,
                    nthreads);
    else
        orc_rs_i32((const int32_t *const *)x, (int32_t *const *)sh, n, L, k, order, 1, nthreads);
    orc_ag(esize, (const void *const *)sh, out, n, L, k, nthreads);
    free_shards(sh, k);
    return 0;
}

/* dtype: 0 = f32, 1 = bf16 */
int orc_ar_weighted(int dtype, const void *const *g, void *const *out, const int64_t *tokens,
                    int64_t n, int k, int order, int nthreads)
{
    int esize = dtype == 1 ? 2 : 4;
    int64_t L = orc_shard_len(n, k);
    void **sh = alloc_shards(k, L, esize);
    int rc;
    if (!sh) return -1;
    if (dtype == 0)
        rc = orc_rs_weighted_f32((const float *const *)g, (float *const *)sh, tokens, n, L, k,
                                 order, 1, nthreads);
    else
        rc = orc_rs_weighted_bf16((const uint16_t *const *)g, (uint16_t *const *)sh, tokens, n,
                                  L, k, order, 1, nthreads);
    if (rc == 0) orc_ag(esize, (const void *const *)sh, out, n, L, k, nthreads);
    free_shards(sh, k);
    return rc;
}

/* ------------------------------------------------------------------ GEMMs
 * C[m,n] = op(A)[m,kk] * B[kk,n], all row-major. op(A) = A stored [m,kk], or,
 * with trans_a, A^T where A is stored [kk,m]. */

static double a_at(const float *a, int64_t i, int64_t p, int64_t m, int64_t kk, int trans_a)
{
    return trans_a ? (double)a[p * m + i] : (double)a[i * kk + p];
}

/* fp64 reference; abs_c (optional) receives sum_p |A(i,p)|*|B(p,j)| */
void orc_gemm_f64(const float *a, const float *b, double *c, double *abs_c, int64_t m,
                  int64_t n, int64_t kk, int trans_a, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(static) if (nthreads > 1)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0, sa = 0.0;
            for (int64_t p = 0; p < kk; ++p) {
                double av = a_at(a, i, p, m, kk, trans_a);
                double bv = (double)b[p * n + j];
                s += av * bv;
                sa += fabs(av) * fabs(bv);
            }
            c[i * n + j] = s;
            if (abs_c) abs_c[i * n + j] = sa;
        }
    }
}

/* bf16 inputs, fp64 result at sampled (rows[s], cols[s]) of C = A B with A
 * [m, kk]; B stored [kk, n] (b_nk = 0) or [n, kk] (b_nk = 1, so C = A B^T);
 * abs_c as above */
void orc_gemm_bf16_at(const uint16_t *a, const uint16_t *b, int64_t n, int64_t kk, int b_nk,
                      const int64_t *rows, const int64_t *cols, int64_t count, double *vals,
                      double *abs_vals, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(static) if (nthreads > 1)
    for (int64_t s = 0; s < count; ++s) {
        double acc = 0.0, sa = 0.0;
        for (int64_t p = 0; p < kk; ++p) {
            double av = (double)orc_bf16_to_f32(a[rows[s] * kk + p]);
            double bv = (double)orc_bf16_to_f32(b_nk ? b[cols[s] * kk + p] : b[p * n + cols[s]]);
            acc += av * bv;
            sa += fabs(av) * fabs(bv);
        }
        vals[s] = acc;
        if (abs_vals) abs_vals[s] = sa;
    }
}

/* -------------------------------------------------------------- FSDP layer
 * k ranks; x_local[r]: [m_local, d]; w_shard[c]: [R, f] with R = ceil(d/k)
 * (rows cR .. min((c+1)R, d) of w, then zero pad rows); dy_local[r]:
 * [m_local, f] or NULL.
 * Outputs: w_full[r] [d, f] (fp32, exact gather); y_local[r] [m_local, f]
 * (fp64); when dy_local is given, dw_full[r] [d, f] (fp64) and dw_shard[c]
 * [R, f] (fp64 sum over ranks of the rows of shard c; pad rows zero). */
void orc_fsdp_layer(int k, int64_t m_local, int64_t d, int64_t f,
                    const float *const *x_local, const float *const *w_shard,
                    const float *const *dy_local, float *const *w_full,
                    double *const *y_local, double *const *dw_full, double *const *dw_shard,
                    int nthreads)
{
    int64_t R = orc_shard_len(d, k);
    orc_ag(4, (const void *const *)w_shard, (void *const *)w_full, d * f, R * f, k, nthreads);
    for (int r = 0; r < k; ++r)
        orc_gemm_f64(x_local[r], w_full[r], y_local[r], NULL, m_local, f, d, 0, nthreads);
    if (!dy_local) return;
    for (int r = 0; r < k; ++r)
        orc_gemm_f64(x_local[r], dy_local[r], dw_full[r], NULL, d, f, m_local, 1, nthreads);
    for (int c = 0; c < k; ++c) {
        for (int64_t e = 0; e < R * f; ++e) {
            int64_t g = (int64_t)c * R * f + e;
            double s = 0.0;
            if (g < d * f)
                for (int r = 0; r < k; ++r) s += dw_full[r][g];
            dw_shard[c][e] = s;
        }
    }
}
