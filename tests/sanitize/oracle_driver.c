/*
 * oracle_driver.c -- runs every entry point of oracle/attn_oracle.c on small
 * inputs (and on rejected arguments) so that a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer sees each code path.  Test infrastructure:
 * built and run by tests/test_host_sanitizers.py on the CPU.  Exit status 0
 * means every call returned the expected status; the sanitizers abort on
 * any memory or undefined-behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn_rows(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                     int64_t, int64_t, int64_t, int64_t, int64_t, int, double, const int64_t*,
                     int64_t, double*, double*, int);
int oracle_attn_rows_elem(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                          int64_t, int64_t, int64_t, int64_t, int64_t, int, double, int64_t,
                          int64_t, const int64_t*, int64_t, double*, double*, int, int);
int oracle_merge_states(const double*, const double*, int64_t, int64_t, int64_t, double*,
                        double*);
int oracle_online_rows(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                       int64_t, int64_t, int64_t, int64_t, int64_t, int, double, int64_t, int,
                       double, int64_t, const int64_t*, int64_t, double*, double*, double*,
                       int64_t*, int);
int oracle_attn_varlen(const uint16_t*, const uint16_t*, const uint16_t*, const int64_t*,
                       const int64_t*, int64_t, int64_t, int64_t, int64_t, int64_t, int, double,
                       const int64_t*, int64_t, double*, double*, int, int);
int oracle_attn_bwd(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, int64_t,
                    int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, double, int,
                    double*, double*, double*, double*, int);

static int failures = 0;
#define EXPECT(call, want)                                                            \
    do {                                                                              \
        int rc_ = (call);                                                             \
        if (rc_ != (want)) {                                                          \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__,   \
                    #call, rc_, (want));                                              \
            ++failures;                                                               \
        }                                                                             \
    } while (0)

/* bf16 patterns of small values: a fixed linear congruential sequence
 * mapped to [-2, 2), rounded down to bf16 by dropping the low half */
static uint16_t* bf16_array(size_t n, uint32_t seed)
{
    uint16_t* a = malloc(n * sizeof *a);
    uint32_t s = seed;
    for (size_t i = 0; i < n; ++i) {
        s = s * 1664525u + 1013904223u;
        float f = ((float)(s >> 8) / 16777216.0f) * 4.0f - 2.0f;
        uint32_t w;
        memcpy(&w, &f, sizeof w);
        a[i] = (uint16_t)(w >> 16);
    }
    return a;
}

int main(void)
{
    const int64_t B = 2, Hq = 4, Hkv = 2, Lq = 9, Lk = 13, d = 8;
    uint16_t* q = bf16_array((size_t)(B * Hq * Lq * d), 1);
    uint16_t* k = bf16_array((size_t)(B * Hkv * Lk * d), 2);
    uint16_t* v = bf16_array((size_t)(B * Hkv * Lk * d), 3);
    uint16_t* g = bf16_array((size_t)(B * Hq * Lq * d), 4);
    const int64_t rows = B * Hq * Lq;
    double* o = calloc((size_t)(rows * d), sizeof(double));
    double* lse = calloc((size_t)rows, sizeof(double));
    double* st = calloc((size_t)(rows * 2), sizeof(double));
    int64_t events = 0;

    for (int causal = 0; causal < 2; ++causal) {
        EXPECT(oracle_attn_rows(q, k, v, B, Hq, Hkv, Lq, Lk, d, d, causal, 0.35, NULL, rows, o,
                                lse, 2), 0);
        int64_t some[3] = {0, 17, rows - 1};
        EXPECT(oracle_attn_rows(q, k, v, B, Hq, Hkv, Lq, Lk, d, d, causal, 0.35, some, 3, o, lse,
                                1), 0);
        for (int elem = 0; elem < 2; ++elem)
            EXPECT(oracle_attn_rows_elem(q, k, v, B, Hq, Hkv, Lq, Lk, d, d, causal, 0.35, 3, 11,
                                         NULL, rows, o, lse, 2, elem), 0);
        for (int mode = 0; mode < 3; ++mode)
            EXPECT(oracle_online_rows(q, k, v, B, Hq, Hkv, Lq, Lk, d, d, causal, 0.35, 5, mode,
                                      8.0, 2, NULL, rows, o, lse, st, &events, 2), 0);
    }
    /* Lq > Lk under the causal mask: rows without keys */
    EXPECT(oracle_attn_rows(q, k, v, 1, 2, 1, 13, 5, d, d, 1, 0.35, NULL, 26, o, lse, 1), 0);

    /* rejected arguments */
    EXPECT(oracle_attn_rows(q, k, v, B, 3, 2, Lq, Lk, d, d, 0, 0.35, NULL, 3 * B * Lq, o, lse, 1),
           2);
    EXPECT(oracle_attn_rows(q, k, v, B, Hq, Hkv, Lq, Lk, d, d, 0, -1.0, NULL, rows, o, lse, 1), 3);
    EXPECT(oracle_attn_rows(NULL, k, v, B, Hq, Hkv, Lq, Lk, d, d, 0, 0.35, NULL, rows, o, lse, 1),
           4);
    int64_t bad[1] = {rows};
    EXPECT(oracle_attn_rows(q, k, v, B, Hq, Hkv, Lq, Lk, d, d, 0, 0.35, bad, 1, o, lse, 1), 6);

    /* merge of segment states, one of them empty */
    double op[3 * 4 * 8], lp[3 * 4], om[4 * 8], lm[4];
    for (int i = 0; i < 3 * 4 * 8; ++i) op[i] = (double)(i % 7) - 3.0;
    for (int i = 0; i < 12; ++i) lp[i] = (i % 5 == 0) ? -INFINITY : 0.1 * i;
    EXPECT(oracle_merge_states(op, lp, 3, 4, 8, om, lm), 0);
    EXPECT(oracle_merge_states(op, lp, 0, 4, 8, om, lm), 1);

    /* packed variable-length batch with empty sequences */
    const int64_t cu_q[5] = {0, 3, 3, 9, 10}, cu_k[5] = {0, 5, 7, 7, 13};
    uint16_t* vq = bf16_array(10 * 4 * 8, 5);
    uint16_t* vk = bf16_array(13 * 2 * 8, 6);
    uint16_t* vv = bf16_array(13 * 2 * 8, 7);
    double* vo = calloc(40 * 8, sizeof(double));
    double* vl = calloc(40, sizeof(double));
    for (int causal = 0; causal < 2; ++causal)
        EXPECT(oracle_attn_varlen(vq, vk, vv, cu_q, cu_k, 4, 4, 2, 8, 8, causal, 0.35, NULL, 40,
                                  vo, vl, 2, 0), 0);
    const int64_t bad_cu[5] = {0, 3, 2, 9, 10};
    EXPECT(oracle_attn_varlen(vq, vk, vv, bad_cu, cu_k, 4, 4, 2, 8, 8, 0, 0.35, NULL, 40, vo, vl,
                              1, 0), 9);

    /* backward by the definition */
    double* dq = calloc((size_t)(B * Hq * Lq * d), sizeof(double));
    double* dk = calloc((size_t)(B * Hkv * Lk * d), sizeof(double));
    double* dv = calloc((size_t)(B * Hkv * Lk * d), sizeof(double));
    double* dl = calloc((size_t)rows, sizeof(double));
    for (int causal = 0; causal < 2; ++causal)
        EXPECT(oracle_attn_bwd(q, k, v, g, B, Hq, Hkv, Lq, Lk, d, d, causal, 0.35, 0, dq, dk, dv,
                               dl, 2), 0);

    free(q); free(k); free(v); free(g); free(o); free(lse); free(st);
    free(vq); free(vk); free(vv); free(vo); free(vl);
    free(dq); free(dk); free(dv); free(dl);
    if (failures) {
        fprintf(stderr, "%d unexpected status codes\n", failures);
        return 1;
    }
    printf("oracle driver: all calls returned the expected status\n");
    return 0;
}
