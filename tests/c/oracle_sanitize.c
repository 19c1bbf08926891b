/*
 * Drives every entry point of oracle/oracle.c on small and edge-case inputs
 * so that a build with -fsanitize=address,undefined (tests/test_oracle.py)
 * sees each of its loops, allocations and conversions: all bf16, E4M3 and
 * E2M1 patterns, infinities and NaN, K not a multiple of 32, row subsets,
 * optional outputs left out, one and several threads.  Prints
 * "oracle_sanitize ok" when every call returned what its contract says.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_double(uint16_t bits);
int oracle_bf16_array_to_double(const uint16_t *src, int64_t n, double *dst);
double oracle_e4m3_to_double(uint8_t code);
uint8_t oracle_e4m3_from_float(float v);
int oracle_quantize_e4m3_columns(const uint16_t *w, int64_t K, int64_t N, uint8_t *codes,
                                 float *scales);
double oracle_e2m1_to_double(uint8_t code);
uint8_t oracle_e2m1_from_double(double v);
int oracle_mx_shared_exponent(double amax);
int oracle_quantize_mxfp4_columns(const uint16_t *w, int64_t K, int64_t N, uint8_t *codes,
                                  uint8_t *scales);
int oracle_dequantize_mxfp4_columns(const uint8_t *codes, const uint8_t *scales, int64_t K,
                                    int64_t N, double *out);
int oracle_dequantize_e4m3_columns(const uint8_t *codes, const float *scales, int64_t K,
                                   int64_t N, double *out);
double oracle_sigmoid(double z);
double oracle_silu(double z);
int oracle_swiglu_rows(int dtype, const void *x, const void *wg, const void *wu, int64_t M,
                       int64_t d, int64_t dff, const int64_t *rows, int64_t nrows, double *g,
                       double *u, double *h, int nthreads);
int oracle_mlp_rows(int dtype, const void *x, const void *wg, const void *wu, const void *wd,
                    int64_t M, int64_t d, int64_t dff, const int64_t *rows, int64_t nrows,
                    double *h_out, double *y, int nthreads);
int oracle_rmsnorm_rows(int dtype, const void *r, const void *gamma, double eps, int64_t M,
                        int64_t d, double *out);
int oracle_default_threads(void);

static int failures = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                            \
        }                                                          \
    } while (0)

static uint32_t lcg = 12345u;
static uint16_t rnd_bf16(void)
{
    /* small normal-ish values: sign, exponent in [120, 129], random mantissa */
    lcg = lcg * 1664525u + 1013904223u;
    uint16_t sign = (uint16_t)((lcg >> 31) << 15);
    uint16_t exp = (uint16_t)(120 + (lcg >> 8) % 10);
    uint16_t man = (uint16_t)((lcg >> 16) & 0x7F);
    return (uint16_t)(sign | (exp << 7) | man);
}

int main(void)
{
    /* every bf16 pattern, one by one and as an array */
    uint16_t *all = (uint16_t *)malloc(65536 * sizeof(uint16_t));
    double *alld = (double *)malloc(65536 * sizeof(double));
    for (int i = 0; i < 65536; ++i)
        all[i] = (uint16_t)i;
    CHECK(oracle_bf16_array_to_double(all, 65536, alld) == 0);
    for (int i = 0; i < 65536; ++i) {
        double v = oracle_bf16_to_double((uint16_t)i);
        CHECK(memcmp(&v, &alld[i], sizeof v) == 0 || (isnan(v) && isnan(alld[i])));
    }
    /* E4M3 and E2M1: every code, and encodes of edge values */
    for (int c = 0; c < 256; ++c)
        (void)oracle_e4m3_to_double((uint8_t)c);
    const float fv[] = {0.0f, -0.0f, 1e-10f, 1.0f, -448.0f, 448.0f, 1e6f, -1e6f,
                        INFINITY, -INFINITY, NAN, 0.001953125f};
    for (size_t i = 0; i < sizeof fv / sizeof fv[0]; ++i)
        (void)oracle_e4m3_from_float(fv[i]);
    for (int c = 0; c < 16; ++c)
        (void)oracle_e2m1_to_double((uint8_t)c);
    const double dv[] = {0.0, -0.0, 0.25, 0.75, 5.0, 6.0, 7.0, 1e300, -1e300,
                         INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof dv / sizeof dv[0]; ++i)
        (void)oracle_e2m1_from_double(dv[i]);
    const double av[] = {0.0, 1e-300, 1.0, 6.0, 1e38, 1e300, INFINITY};
    for (size_t i = 0; i < sizeof av / sizeof av[0]; ++i) {
        int s = oracle_mx_shared_exponent(av[i]);
        CHECK(s >= -126 && s <= 127);
    }
    const double zv[] = {0.0, 1.0, -1.0, 40.0, -40.0, 800.0, -800.0, INFINITY, -INFINITY};
    for (size_t i = 0; i < sizeof zv / sizeof zv[0]; ++i) {
        double s = oracle_sigmoid(zv[i]);
        CHECK(s >= 0.0 && s <= 1.0);
        (void)oracle_silu(zv[i]);
    }

    /* quantisers on K = 37 (one full and one partial MXFP4 block), N = 5,
     * with an all-zero column */
    enum { K = 37, N = 5 };
    uint16_t w[K * N];
    for (int i = 0; i < K * N; ++i)
        w[i] = (i % N == 2) ? 0 : rnd_bf16();
    uint8_t codes[K * N], mcodes[K * N], mscales[2 * N];
    float scales[N];
    double deq[K * N];
    CHECK(oracle_quantize_e4m3_columns(w, K, N, codes, scales) == 0);
    CHECK(scales[2] == 0.0f);
    CHECK(oracle_dequantize_e4m3_columns(codes, scales, K, N, deq) == 0);
    CHECK(oracle_quantize_mxfp4_columns(w, K, N, mcodes, mscales) == 0);
    CHECK(oracle_dequantize_mxfp4_columns(mcodes, mscales, K, N, deq) == 0);
    /* non-finite weights: column 4 holds NaN in its first block and -inf in
     * its second; both saturate with their sign, the NaN does not count
     * toward its block's exponent, the infinity puts it at the top (127) */
    w[0 * N + 4] = 0x7FC0;
    w[33 * N + 4] = 0xFF80;
    CHECK(oracle_quantize_mxfp4_columns(w, K, N, mcodes, mscales) == 0);
    CHECK(mcodes[0 * N + 4] == 0x7 && mcodes[33 * N + 4] == 0xF);
    CHECK(mscales[0 * N + 4] < 254 && mscales[1 * N + 4] == 254);
    CHECK(oracle_dequantize_mxfp4_columns(mcodes, mscales, K, N, deq) == 0);
    CHECK(oracle_quantize_e4m3_columns(w, K, N, codes, scales) == 0);
    CHECK(isinf(scales[4]) && codes[0 * N + 4] == 0x7F);
    CHECK(oracle_dequantize_e4m3_columns(codes, scales, K, N, deq) == 0);
    CHECK(oracle_quantize_e4m3_columns(w, 0, N, codes, scales) == -1);
    CHECK(oracle_dequantize_mxfp4_columns(mcodes, mscales, K, N, NULL) == -1);

    /* swiglu and MLP in every storage type, row subsets, optional outputs */
    enum { M = 3, D = 24, F = 40 };
    uint16_t xb[M * D], wgb[D * F], wub[D * F], wdb[F * D];
    float xf[M * D], wgf[D * F], wuf[D * F], wdf[F * D];
    double xd[M * D], wgd[D * F], wud[D * F], wdd[F * D];
    for (int i = 0; i < M * D; ++i) {
        xb[i] = rnd_bf16();
        xf[i] = (float)oracle_bf16_to_double(xb[i]);
        xd[i] = xf[i];
    }
    for (int i = 0; i < D * F; ++i) {
        wgb[i] = rnd_bf16();
        wub[i] = rnd_bf16();
        wdb[i] = rnd_bf16();
        wgf[i] = (float)oracle_bf16_to_double(wgb[i]);
        wuf[i] = (float)oracle_bf16_to_double(wub[i]);
        wdf[i] = (float)oracle_bf16_to_double(wdb[i]);
        wgd[i] = wgf[i];
        wud[i] = wuf[i];
        wdd[i] = wdf[i];
    }
    const void *xs[3] = {xf, xb, xd}, *wgs[3] = {wgf, wgb, wgd}, *wus[3] = {wuf, wub, wud},
               *wds[3] = {wdf, wdb, wdd};
    double g[M * F], u[M * F], h[M * F], h2[M * F], y[M * D], y2[M * D], n[M * D];
    const int64_t rows[2] = {2, 0};
    for (int dt = 0; dt < 3; ++dt) {
        for (int threads = 1; threads <= 2; ++threads) {
            CHECK(oracle_swiglu_rows(dt, xs[dt], wgs[dt], wus[dt], M, D, F, NULL, M, g, u, h,
                                     threads) == 0);
            CHECK(oracle_swiglu_rows(dt, xs[dt], wgs[dt], wus[dt], M, D, F, rows, 2, NULL, NULL,
                                     h2, threads) == 0);
            CHECK(memcmp(h2, h + 2 * F, F * sizeof(double)) == 0);   /* row 2 first */
            CHECK(oracle_mlp_rows(dt, xs[dt], wgs[dt], wus[dt], wds[dt], M, D, F, NULL, M, NULL, y,
                                  threads) == 0);
            CHECK(oracle_mlp_rows(dt, xs[dt], wgs[dt], wus[dt], wds[dt], M, D, F, rows, 2, h2, y2,
                                  threads) == 0);
            CHECK(memcmp(y2 + D, y, D * sizeof(double)) == 0);       /* row 0 second */
        }
        CHECK(oracle_rmsnorm_rows(dt, xs[dt], wgs[dt], 1e-6, M, D, n) == 0);
    }
    CHECK(oracle_swiglu_rows(7, xf, wgf, wuf, M, D, F, NULL, M, NULL, NULL, h, 1) != 0);
    const int64_t bad_rows[1] = {M};
    CHECK(oracle_swiglu_rows(0, xf, wgf, wuf, M, D, F, bad_rows, 1, NULL, NULL, h, 1) != 0);
    CHECK(oracle_rmsnorm_rows(0, xf, wgf, -1.0, M, D, n) != 0);
    CHECK(oracle_default_threads() >= 1);

    free(all);
    free(alld);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle_sanitize ok\n");
    return 0;
}
