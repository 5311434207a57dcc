/* Runs the oracle's routines on small inputs in exactly sized heap buffers, for
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer: any read or
 * write outside a buffer, or undefined arithmetic, stops the run. The values
 * are small integers, so the reductions are exact and are also checked here.
 * Exit status 0 when every check passes. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_shard_len(int64_t n, int k);
int64_t orc_shard_valid(int64_t n, int64_t L, int c);
uint16_t orc_bf16_from_f32(float f);
float orc_bf16_to_f32(uint16_t b);
void orc_rs_f32(const float *const *x, float *const *out, int64_t n, int64_t L, int k, int op,
                int order, int write_pads, int nthreads);
void orc_rs_bf16(const uint16_t *const *x, uint16_t *const *out, int64_t n, int64_t L, int k,
                 int op, int order, int write_pads, int nthreads);
void orc_rs_i32(const int32_t *const *x, int32_t *const *out, int64_t n, int64_t L, int k,
                int order, int write_pads, int nthreads);
int orc_rs_weighted_f32(const float *const *g, float *const *out, const int64_t *tokens,
                        int64_t n, int64_t L, int k, int order, int write_pads, int nthreads);
void orc_ag(int esize, const void *const *shard, void *const *out, int64_t n, int64_t L, int k,
            int nthreads);
int orc_ar(int dtype, const void *const *x, void *const *out, int64_t n, int k, int op, int order,
           int nthreads);
int orc_ar_weighted(int dtype, const void *const *g, void *const *out, const int64_t *tokens,
                    int64_t n, int k, int order, int nthreads);
void orc_scatter_accumulate(int dtype, const void *g, float *const *acc, int64_t n, int64_t L,
                            int k);
void orc_settle(int dtype, const float *const *acc, void *const *out, int64_t n, int64_t L, int k,
                float divisor);
void orc_gemm_f64(const float *a, const float *b, double *c, double *abs_c, int64_t m, int64_t n,
                  int64_t kk, int trans_a, int nthreads);

static int failures = 0;
static uint64_t state = 12345;

static int small_int(void)
{
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (int)((state >> 33) % 21) - 10;     /* -10 .. 10 */
}

static void *xmalloc(size_t bytes) { return malloc(bytes ? bytes : 1); }

static void check(int ok, const char *what, int k, int64_t n)
{
    if (!ok) {
        fprintf(stderr, "FAIL %s k=%d n=%lld\n", what, k, (long long)n);
        ++failures;
    }
}

static void run_case(int k, int64_t n)
{
    const int64_t L = orc_shard_len(n, k);
    float *xf[64], *sf[64], *of[64], *acc[64];
    uint16_t *xb[64], *sb[64];
    int32_t *xi[64], *si[64];
    void *ov[64];
    int64_t tokens[64];
    for (int r = 0; r < k; ++r) {
        xf[r] = xmalloc((size_t)n * 4);
        xb[r] = xmalloc((size_t)n * 2);
        xi[r] = xmalloc((size_t)n * 4);
        for (int64_t i = 0; i < n; ++i) {
            int v = small_int();
            xf[r][i] = (float)v;
            xb[r][i] = orc_bf16_from_f32((float)v);
            xi[r][i] = v;
        }
        sf[r] = xmalloc((size_t)L * 4);
        sb[r] = xmalloc((size_t)L * 2);
        si[r] = xmalloc((size_t)L * 4);
        of[r] = xmalloc((size_t)n * 4);
        acc[r] = xmalloc((size_t)L * 4);
        memset(acc[r], 0, (size_t)L * 4);
        ov[r] = of[r];
        tokens[r] = 1 + r;
    }
    for (int order = 0; order < 2; ++order) {
        orc_rs_f32((const float *const *)xf, sf, n, L, k, 0, order, 1, 1);
        orc_rs_bf16((const uint16_t *const *)xb, sb, n, L, k, 0, order, 1, 1);
        orc_rs_i32((const int32_t *const *)xi, si, n, L, k, order, 1, 1);
        for (int c = 0; c < k; ++c) {
            const int64_t nc = orc_shard_valid(n, L, c);
            for (int64_t j = 0; j < L; ++j) {
                int64_t want = 0;
                if (j < nc)
                    for (int r = 0; r < k; ++r) want += xi[r][c * L + j];
                check(sf[c][j] == (float)want, "rs_f32", k, n);
                check(si[c][j] == (int32_t)want, "rs_i32", k, n);
                check(orc_bf16_to_f32(sb[c][j]) == orc_bf16_to_f32(orc_bf16_from_f32((float)want)),
                      "rs_bf16", k, n);
            }
        }
    }
    orc_ag(4, (const void *const *)sf, ov, n, L, k, 1);
    for (int r = 0; r < k; ++r)
        for (int64_t i = 0; i < n; ++i) {
            float want = 0.0f;
            for (int q = 0; q < k; ++q) want += xf[q][i];
            check(of[r][i] == want, "ag", k, n);
        }
    check(orc_ar(0, (const void *const *)xf, ov, n, k, 1, 0, 1) == 0, "ar", k, n);
    check(orc_ar_weighted(0, (const void *const *)xf, ov, tokens, n, k, 0, 1) == 0, "ar_w", k, n);
    check(orc_rs_weighted_f32((const float *const *)xf, sf, tokens, n, L, k, 0, 1, 1) == 0,
          "rs_w", k, n);
    for (int r = 0; r < k; ++r) {
        orc_scatter_accumulate(0, xf[r], acc, n, L, k);
        orc_scatter_accumulate(1, xb[r], acc, n, L, k);
    }
    orc_settle(0, (const float *const *)acc, ov, n, L, k, 2.0f);
    for (int c = 0; c < k; ++c) {
        const int64_t nc = orc_shard_valid(n, L, c);
        for (int64_t j = 0; j < nc; ++j) {
            float want = 0.0f;
            for (int r = 0; r < k; ++r) want += xf[r][c * L + j];
            check(of[c][j] == want, "settle", k, n);     /* (2 sums) / 2 */
        }
    }
    orc_settle(1, (const float *const *)acc, (void *const *)sb, n, L, k, 3.0f);
    for (int r = 0; r < k; ++r) {
        free(xf[r]); free(xb[r]); free(xi[r]); free(sf[r]); free(sb[r]); free(si[r]);
        free(of[r]); free(acc[r]);
    }
}

static void run_gemm(int64_t m, int64_t n, int64_t kk)
{
    float *a = xmalloc((size_t)(m * kk) * 4), *b = xmalloc((size_t)(kk * n) * 4);
    double *c64 = xmalloc((size_t)(m * n) * 8), *abs64 = xmalloc((size_t)(m * n) * 8);
    for (int64_t i = 0; i < m * kk; ++i) a[i] = (float)small_int();
    for (int64_t i = 0; i < kk * n; ++i) b[i] = (float)small_int();
    for (int trans = 0; trans < 2; ++trans) {
        orc_gemm_f64(a, b, c64, abs64, m, n, kk, trans, 1);
        /* small-integer operands: every product and partial sum is exact */
        for (int64_t i = 0; i < m * n; ++i) check(c64[i] == rint(c64[i]), "gemm", (int)m, n);
    }
    free(a); free(b); free(c64); free(abs64);
}

int main(void)
{
    for (int k = 1; k <= 9; ++k)
        for (int64_t n = 0; n <= 3 * k + 2; ++n) run_case(k, n);
    run_case(8, 1001);
    run_case(64, 200);
    run_gemm(1, 1, 1);
    run_gemm(7, 5, 3);
    run_gemm(33, 17, 65);
    printf("oracle driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
