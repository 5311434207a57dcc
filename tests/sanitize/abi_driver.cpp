// Calls every entry point of libdpsync with invalid arguments and with n = 0,
// for a build whose host code has AddressSanitizer and
// UndefinedBehaviorSanitizer: validation runs before any HIP call, so this
// needs no GPU, and any out-of-range access or undefined arithmetic in the
// argument checks stops the run. The device pointers are fake addresses that
// are never dereferenced. Exit status 0 when every call returns the expected
// status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "dpsync.h"

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

static void fake(void **p, int k, uintptr_t base, uintptr_t stride = 1u << 20)
{
    for (int i = 0; i < k; ++i) p[i] = (void *)(base + (uintptr_t)i * stride);
}

int main()
{
    void *a[DP_MAX_K], *b[DP_MAX_K], *c[DP_MAX_K], *d[DP_MAX_K];
    fake(a, DP_MAX_K, (uintptr_t)1 << 40);
    fake(b, DP_MAX_K, (uintptr_t)1 << 41);
    fake(c, DP_MAX_K, (uintptr_t)1 << 42);
    fake(d, DP_MAX_K, (uintptr_t)1 << 43);
    const void *const *ca = (const void *const *)a;

    for (int s = -1; s < 8; ++s)
        if (!dp_status_string(s) || !strlen(dp_status_string(s))) ++failures;
    expect((int)dp_shard_len(10, 4), 3, "shard_len");
    expect((int)dp_shard_len(0, 4), 0, "shard_len 0");
    expect((int)dp_shard_len(10, 0), 0, "shard_len k 0");
    expect(dp_version(), 100, "version");

    for (int k : {0, -3, DP_MAX_K + 1}) {
        expect(dp_reduce_scatter(ca, b, 100, k, DP_F32, DP_SUM, 1, nullptr), DP_ERR_INVALID_ARG, "rs k");
        expect(dp_all_gather(ca, b, 100, k, DP_F32, 1, nullptr), DP_ERR_INVALID_ARG, "ag k");
        expect(dp_all_reduce(ca, b, 100, k, DP_F32, DP_SUM, 1, nullptr), DP_ERR_INVALID_ARG, "ar k");
    }
    expect(dp_reduce_scatter(ca, b, 100, 4, 9, DP_SUM, 1, nullptr), DP_ERR_UNSUPPORTED, "rs dtype");
    expect(dp_reduce_scatter(ca, b, 100, 4, DP_I32, DP_AVG, 1, nullptr), DP_ERR_UNSUPPORTED, "rs i32 avg");
    expect(dp_reduce_scatter(ca, b, 100, 4, DP_F32, DP_SUM, 0, nullptr), DP_ERR_INVALID_ARG, "rs S");
    expect(dp_reduce_scatter(nullptr, b, 100, 4, DP_F32, DP_SUM, 1, nullptr), DP_ERR_INVALID_ARG, "rs null");
    expect(dp_reduce_scatter(ca, b, (size_t)1 << 62, 4, DP_F32, DP_SUM, 1, nullptr), DP_ERR_INVALID_ARG, "rs size");
    void *ov[4] = {(char *)a[1] + 64, b[1], b[2], b[3]};
    expect(dp_reduce_scatter(ca, ov, 1000, 4, DP_F32, DP_SUM, 1, nullptr), DP_ERR_ALIAS, "rs alias");
    void *mis[4] = {(char *)b[0] + 2, b[1], b[2], b[3]};
    expect(dp_all_gather(ca, mis, 1000, 4, DP_F32, 1, nullptr), DP_ERR_INVALID_ARG, "ag misaligned");
    expect(dp_reduce_scatter(ca, b, 0, 4, DP_F32, DP_AVG, 1, nullptr), DP_OK, "rs n 0");
    expect(dp_all_gather(ca, b, 0, 4, DP_BF16, 1, nullptr), DP_OK, "ag n 0");
    expect(dp_all_reduce(ca, b, 0, 4, DP_I32, DP_SUM, 1, nullptr), DP_OK, "ar n 0");

    int64_t tok[4] = {1, -2, 3, 4}, tok0[4] = {0, 0, 0, 0};
    expect(dp_weighted_reduce(ca, b, tok, 100, 4, DP_F32, 1, nullptr), DP_ERR_INVALID_ARG, "wr neg");
    expect(dp_weighted_reduce(ca, b, tok0, 100, 4, DP_F32, 1, nullptr), DP_ERR_INVALID_ARG, "wr zero");
    expect(dp_weighted_reduce(ca, b, nullptr, 100, 4, DP_F32, 1, nullptr), DP_ERR_INVALID_ARG, "wr null");
    expect(dp_weighted_reduce(ca, b, tok, 100, 4, DP_I32, 1, nullptr), DP_ERR_UNSUPPORTED, "wr i32");

    dp_launch_opts_t bad = {-1, 0, {0, 0}}, badf = {0, 64, {0, 0}}, badr = {0, 0, {1, 0}};
    for (const dp_launch_opts_t *o : {&bad, &badf, &badr}) {
        expect(dp_reduce_scatter_ex(ca, b, 100, 4, DP_F32, DP_SUM, 1, o, nullptr), DP_ERR_INVALID_ARG, "rs opts");
        expect(dp_all_gather_ex(ca, b, 100, 4, DP_F32, 1, o, nullptr), DP_ERR_INVALID_ARG, "ag opts");
        expect(dp_all_reduce_ex(ca, b, 100, 4, DP_F32, DP_SUM, 1, o, nullptr), DP_ERR_INVALID_ARG, "ar opts");
        expect(dp_gemm_bf16_ex(a[0], b[0], c[0], 8, 8, 8, o, nullptr), DP_ERR_INVALID_ARG, "gemm opts");
        expect(dp_weighted_reduce_ex(ca, b, tok, 100, 4, DP_F32, 1, o, nullptr), DP_ERR_INVALID_ARG, "wr opts");
    }

    expect(dp_fsdp_layer(0, 8, 8, 8, (const float *const *)a, (const float *const *)b,
                         (const float *const *)c, (float *const *)d, (float *const *)d,
                         (float *const *)d, (float *const *)d, nullptr), DP_ERR_INVALID_ARG, "fsdp k");
    expect(dp_fsdp_layer_ex(2, 8, 8, 8, (const float *const *)a, (const float *const *)b, nullptr,
                            (float *const *)c, (float *const *)d, (float *const *)d,
                            (float *const *)d, (float *const *)d, nullptr),
           DP_ERR_INVALID_ARG, "fsdp_ex dx without dy");
    void *e[DP_MAX_K];
    fake(e, DP_MAX_K, (uintptr_t)1 << 44);
    expect(dp_fsdp_layer_static(0, 8, 8, 8, (const float *const *)a, (const float *const *)b,
                                (const float *const *)c, (float *const *)d, nullptr,
                                (float *const *)e, nullptr), DP_ERR_INVALID_ARG, "fsdp static k");
    expect(dp_fsdp_layer_static(8, 8, 1024, 1024, (const float *const *)a, (const float *const *)b,
                                (const float *const *)c, (float *const *)d, nullptr,
                                (float *const *)e, nullptr), DP_ERR_SCRATCH, "fsdp static size");
    expect(dp_gemm_bf16(a[0], b[0], c[0], 0, 8, 8, nullptr), DP_ERR_INVALID_ARG, "gemm m");
    expect(dp_gemm_bf16(a[0], (char *)b[0] + 1, c[0], 8, 8, 12, nullptr), DP_ERR_INVALID_ARG,
           "gemm b alignment");
    expect(dp_gemm_bf16(a[0], b[0], (char *)a[0] + 16, 8, 8, 8, nullptr), DP_ERR_ALIAS, "gemm alias");

    float *acc[4];
    for (int i = 0; i < 4; ++i) acc[i] = (float *)c[i];
    expect(dp_scatter_accumulate(ca, 0, DP_F32, acc, 100, 4, nullptr), DP_ERR_INVALID_ARG, "sa np");
    expect(dp_scatter_accumulate(ca, 2, DP_I32, acc, 100, 4, nullptr), DP_ERR_UNSUPPORTED, "sa dtype");
    expect(dp_scatter_accumulate(ca, 2, DP_BF16, acc, 0, 4, nullptr), DP_OK, "sa n 0");
    expect(dp_settle(acc, b, 100, 4, DP_F32, 0.0f, 0, nullptr), DP_ERR_INVALID_ARG, "settle 0");
    expect(dp_settle(acc, b, 0, 4, DP_BF16, 2.0f, 1, nullptr), DP_OK, "settle n 0");

    dp_grad_piece_t pieces[2] = {{0, 32, 32}, {1024, 16, 8}};
    expect(dp_backward_allreduce_overlap(2, 2, pieces, 16, ca, (const void *const *)b, c, d,
                                         1024 + 128 + 1, 500, DP_AVG, nullptr, nullptr,
                                         (void *)1, nullptr, 0), DP_ERR_INVALID_ARG, "overlap tile");
    expect(dp_backward_allreduce_overlap(2, 2, pieces, 12, ca, (const void *const *)b, c, d,
                                         1024 + 128, 500, DP_AVG, nullptr, nullptr, (void *)1,
                                         nullptr, 0), DP_ERR_UNSUPPORTED, "overlap t");
    expect(dp_backward_allreduce_overlap(2, 2, pieces, 16, ca, (const void *const *)b, c, d,
                                         1024 + 128, 500, DP_AVG, nullptr, nullptr, (void *)1,
                                         nullptr, 0), DP_ERR_INVALID_ARG, "overlap events");

    expect(dp_reduce_scatter_all_gather(ca, b, 100, (const void *const *)c, d, 100, 4, DP_F32,
                                        DP_AVG, 0, nullptr), DP_ERR_INVALID_ARG, "rsag S");
    void *cross[4] = {a[0], c[1], c[2], c[3]};
    expect(dp_reduce_scatter_all_gather(ca, b, 100, (const void *const *)cross, d, 100, 4, DP_F32,
                                        DP_SUM, 1, nullptr), DP_ERR_ALIAS, "rsag alias");
    expect(dp_reduce_scatter_all_gather(ca, b, 0, (const void *const *)c, d, 0, 4, DP_BF16, DP_SUM, 1,
                                        nullptr), DP_OK, "rsag n 0");

    printf("abi driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
