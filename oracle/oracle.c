/*
 * oracle.c -- plain CPU reference for the fused SwiGLU MLP.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code with the GPU
 * library and is never used to produce a product result.
 *
 * What it computes (fp64 throughout, no blocking of the sums):
 *   g = x . Wgate,  u = x . Wup                  (two independent products;
 *       Tile-Level Activation Overlap for Efficient LLM Inference, problem
 *       statement: Y = SiLU(A x W1) (.) (A x W2))
 *   h = silu(g) * u,  silu(z) = z * sigmoid(z)   (same passage; SiLU is the
 *       Swish activation with beta = 1)
 *   y = h . Wdown                                (optional down projection;
 *       "Anatomie d'un transformeur sur GPU" §1.1 layer skeleton, and the
 *       §1.2 projection table: Wgate and Wup are d x d_ff, Wdown is d_ff x d)
 *
 * Inputs are the exact bits handed to the GPU: fp32 arrays, or bf16 stored
 * as raw uint16 patterns, which are widened exactly (bits << 16 -> float ->
 * double); or fp64 arrays (the dequantised FP8 weights below, with x
 * widened from bf16).  Every element of g, u and y is a sum taken in ascending order of
 * the contraction index.  Threads only split independent output elements,
 * so results do not depend on the thread count.  h is never rounded before
 * the down projection.
 *
 * Layouts: x is M x d, Wgate and Wup are d x dff, Wdown is dff x d, all
 * row-major.  Parity pins: tests/test_oracle.py (closed forms, integer-exact
 * products, one-hot rows, brute force on tiny shapes).
 *
 * FP8 weights.  "Tile-Level Activation Overlap for Efficient LLM
 * Inference" (section on the problem) notes that quantised weights make the
 * memory-bound part of the MLP weigh more; the pages fix no scheme.  The
 * one used here: OCP 8-bit E4M3 codes (the variant with no infinities), one
 * fp32 scale per output column equal to the column's largest magnitude over
 * 448 (the largest E4M3 value), codes rounded to nearest with ties to the
 * even code and saturated at +-448.  The scale and w / scale are fp32
 * divisions, as on the GPU, so both sides take the same rounding decisions;
 * everything after that is exact in fp64.  Pins: tests/test_oracle.py
 * (format constants, brute-force nearest search, exact grids, error
 * bounds).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

/* bf16 is the top 16 bits of an IEEE binary32; widening is exact. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static inline double elem(const void *p, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)p)[i];
    if (dtype == ORACLE_F64)
        return ((const double *)p)[i];
    return oracle_bf16_to_double(((const uint16_t *)p)[i]);
}

/* Exact widening of n bf16 patterns. */
int oracle_bf16_array_to_double(const uint16_t *src, int64_t n, double *dst)
{
    if (n < 0 || (n > 0 && (!src || !dst)))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_bf16_to_double(src[i]);
    return 0;
}

/*
 * E4M3 value of a code: sign bit, 4-bit exponent field e with bias 7, 3-bit
 * mantissa m.  e = 0 holds the subnormals m * 2^-9; otherwise the value is
 * (1 + m/8) * 2^(e-7).  Exponent 15 with mantissa 7 is NaN; there is no
 * infinity, so 0x7E = 1.75 * 2^8 = 448 is the largest finite value.
 */
double oracle_e4m3_to_double(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return s ? -v : v;
}

/*
 * Nearest E4M3 code to v; ties go to the even code; magnitudes of 448 and
 * above saturate to +-448.  Works on |v| in fp64 (exact for any fp32 v):
 * within a binade [2^b, 2^(b+1)) the E4M3 values are spaced 2^(b-3), and
 * below 2^-6 they are spaced 2^-9, so rounding |v| / spacing to the nearest
 * even integer (the default rounding mode) picks the code; the integer is
 * 8 + mantissa in a binade and the mantissa itself below 2^-6, so an even
 * integer is an even code.
 */
uint8_t oracle_e4m3_from_float(float v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    int e;
    frexp(a, &e);                   /* a = f * 2^e with f in [0.5, 1) */
    int b = e - 1;                  /* binade of a: 2^b <= a < 2^(b+1) */
    double spacing = (a == 0.0 || b < -6) ? ldexp(1.0, -9) : ldexp(1.0, b - 3);
    double r = nearbyint(a / spacing) * spacing;
    if (r < ldexp(1.0, -6))
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    frexp(r, &e);
    b = e - 1;
    int m = (int)(r / ldexp(1.0, b - 3)) - 8;
    return sign | (uint8_t)(((b + 7) << 3) | m);
}

/*
 * Quantises the K x N row-major bf16 matrix w column by column: scale[n] =
 * max_k |w[k][n]| / 448 and code[k][n] = e4m3(w[k][n] / scale[n]), both
 * divisions in fp32; a column of zeros gets scale 0 and code 0 throughout.
 */
int oracle_quantize_e4m3_columns(const uint16_t *w, int64_t K, int64_t N, uint8_t *codes,
                                 float *scales)
{
    if (K <= 0 || N <= 0 || !w || !codes || !scales)
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf((float)oracle_bf16_to_double(w[k * N + n]));
            if (a > amax)
                amax = a;
        }
        float s = amax / 448.0f;
        scales[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            float x = (float)oracle_bf16_to_double(w[k * N + n]);
            codes[k * N + n] = s == 0.0f ? 0 : oracle_e4m3_from_float(x / s);
        }
    }
    return 0;
}

/*
 * MXFP4 weights (OCP Microscaling v1.0, MXFP4): blocks of 32 consecutive K
 * values of one column share a power-of-two scale X = 2^s (an E8M0 code
 * s + 127); each value is stored as an E2M1 code of w / X.  The shared
 * exponent is s = floor(log2(amax)) - 2, amax the block's largest
 * magnitude and 2 the exponent of E2M1's largest power of two (4), so
 * amax / X lies in [4, 8); s is clamped to [-126, 127] so that every scale
 * is a normal fp32 number, and an all-zero block takes s = 0.  w / X is
 * exact; the element code is the nearest E2M1 value, ties to the even code,
 * saturating at +-6.
 *
 * Non-finite weights (the format defines no code for them; this is the
 * reading taken here): E2M1 has neither infinity nor NaN, so both saturate
 * to +-6 with their sign bit; a NaN does not count toward amax (it compares
 * false), and an infinite amax takes the clamp's top, s = 127, since
 * floor(log2(inf)) is infinite.  The MX block-NaN scale code 0xFF is not
 * used: a NaN weight does not make its block NaN.
 *
 * E2M1: sign bit 3, exponent bits 2-1 with bias 1, mantissa bit 0; exponent
 * 0 holds the subnormal 0.5 * m, otherwise (1 + m/2) * 2^(e-1): the values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
double oracle_e2m1_to_double(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* Nearest E2M1 code (ties to the even code, saturating at 6); within a
 * binade [2^b, 2^(b+1)) the values are spaced 2^(b-1), below 1 by 0.5. */
uint8_t oracle_e2m1_from_double(double v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs(v);
    if (!(a < 6.0))                 /* 6 and beyond, infinities, NaN */
        return sign | 0x7;
    int e;
    frexp(a, &e);
    int b = e - 1;
    double step = (a == 0.0 || b < 0) ? 0.5 : ldexp(1.0, b - 1);
    double r = nearbyint(a / step) * step;
    if (r < 1.0)
        return sign | (uint8_t)(r / 0.5);
    frexp(r, &e);
    b = e - 1;
    int m = (int)(r / ldexp(1.0, b - 1)) - 2;
    return sign | (uint8_t)(((b + 1) << 1) | m);
}

/* Shared exponent of a block with largest magnitude amax (see above). */
int oracle_mx_shared_exponent(double amax)
{
    if (amax == 0.0 || isnan(amax))
        return 0;
    if (isinf(amax))
        return 127;
    int e;
    frexp(amax, &e);
    int s = (e - 1) - 2;
    return s < -126 ? -126 : (s > 127 ? 127 : s);
}

/*
 * Quantises the K x N row-major bf16 matrix w to MXFP4 along K: codes
 * (K x N, one E2M1 code per byte) and E8M0 scale codes (ceil(K/32) x N,
 * block b covering rows 32b .. 32b+31).
 */
int oracle_quantize_mxfp4_columns(const uint16_t *w, int64_t K, int64_t N, uint8_t *codes,
                                  uint8_t *scales)
{
    if (K <= 0 || N <= 0 || !w || !codes || !scales)
        return -1;
    int64_t nb = (K + 31) / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t k1 = 32 * b + 32 < K ? 32 * b + 32 : K;
            double amax = 0.0;
            for (int64_t k = 32 * b; k < k1; ++k) {
                double a = fabs(oracle_bf16_to_double(w[k * N + n]));
                if (a > amax)
                    amax = a;
            }
            int s = oracle_mx_shared_exponent(amax);
            scales[b * N + n] = (uint8_t)(s + 127);
            for (int64_t k = 32 * b; k < k1; ++k)
                codes[k * N + n] = oracle_e2m1_from_double(ldexp(oracle_bf16_to_double(w[k * N + n]), -s));
        }
    }
    return 0;
}

/* out[k][n] = 2^(scale[k/32][n] - 127) * e2m1(code[k][n]), exact in fp64. */
int oracle_dequantize_mxfp4_columns(const uint8_t *codes, const uint8_t *scales, int64_t K,
                                    int64_t N, double *out)
{
    if (K <= 0 || N <= 0 || !codes || !scales || !out)
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            out[k * N + n] = ldexp(oracle_e2m1_to_double(codes[k * N + n]),
                                   (int)scales[(k / 32) * N + n] - 127);
    return 0;
}

/* out[k][n] = scale[n] * e4m3(code[k][n]), exact in fp64. */
int oracle_dequantize_e4m3_columns(const uint8_t *codes, const float *scales, int64_t K,
                                   int64_t N, double *out)
{
    if (K <= 0 || N <= 0 || !codes || !scales || !out)
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            out[k * N + n] = (double)scales[n] * oracle_e4m3_to_double(codes[k * N + n]);
    return 0;
}

/* Logistic function 1/(1+e^-z), written so that exp never overflows. */
double oracle_sigmoid(double z)
{
    if (z >= 0.0)
        return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

/* SiLU (Swish with beta = 1): z * sigmoid(z). */
double oracle_silu(double z)
{
    return z * oracle_sigmoid(z);
}

static int bad_dims(int dtype, int64_t M, int64_t d, int64_t dff)
{
    return (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) || M < 0 ||
           d <= 0 || dff <= 0;
}

static int threads_or_default(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Columns handled by one task: independent output elements only. */
#define COL_BLOCK 512

/*
 * Gate and up products for the selected rows of x.
 *   rows: indices into x (nrows of them), or NULL for rows 0..nrows-1.
 *   g, u, h: nrows x dff outputs (each may be NULL if not wanted).
 * h[r][n] = silu(g[r][n]) * u[r][n].  Returns 0, or -1 on bad arguments.
 */
int oracle_swiglu_rows(int dtype, const void *x, const void *wg, const void *wu,
                       int64_t M, int64_t d, int64_t dff,
                       const int64_t *rows, int64_t nrows,
                       double *g, double *u, double *h, int nthreads)
{
    if (bad_dims(dtype, M, d, dff) || nrows < 0 || !x || !wg || !wu)
        return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        if (m < 0 || m >= M)
            return -1;
    }
    int64_t nblocks = (dff + COL_BLOCK - 1) / COL_BLOCK;
    int nt = threads_or_default(nthreads);
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) collapse(2)
    for (int64_t r = 0; r < nrows; ++r) {
        for (int64_t b = 0; b < nblocks; ++b) {
            int64_t m = rows ? rows[r] : r;
            int64_t n0 = b * COL_BLOCK;
            int64_t n1 = n0 + COL_BLOCK < dff ? n0 + COL_BLOCK : dff;
            double *gs = (double *)calloc((size_t)(n1 - n0), sizeof(double));
            double *us = (double *)calloc((size_t)(n1 - n0), sizeof(double));
            if (!gs || !us) {
                free(gs);
                free(us);
#pragma omp atomic write
                err = 1;
                continue;
            }
            /* g[n] = sum_k x[m][k] * Wg[k][n], k ascending; likewise u. */
            for (int64_t k = 0; k < d; ++k) {
                double xv = elem(x, dtype, m * d + k);
                for (int64_t n = n0; n < n1; ++n) {
                    gs[n - n0] += xv * elem(wg, dtype, k * dff + n);
                    us[n - n0] += xv * elem(wu, dtype, k * dff + n);
                }
            }
            for (int64_t n = n0; n < n1; ++n) {
                double gv = gs[n - n0], uv = us[n - n0];
                if (g)
                    g[r * dff + n] = gv;
                if (u)
                    u[r * dff + n] = uv;
                if (h)
                    h[r * dff + n] = oracle_silu(gv) * uv;
            }
            free(gs);
            free(us);
        }
    }
    return err ? -1 : 0;
}

/*
 * Full MLP for the selected rows: y[r][j] = sum_n h[r][n] * Wd[n][j], with h
 * from oracle_swiglu_rows, unrounded, and n ascending.
 *   h_out (nrows x dff) may be NULL; y (nrows x d) is required.
 */
int oracle_mlp_rows(int dtype, const void *x, const void *wg, const void *wu,
                    const void *wd, int64_t M, int64_t d, int64_t dff,
                    const int64_t *rows, int64_t nrows,
                    double *h_out, double *y, int nthreads)
{
    if (bad_dims(dtype, M, d, dff) || nrows < 0 || !wd || !y)
        return -1;
    double *h = h_out;
    if (!h) {
        h = (double *)malloc((size_t)(nrows > 0 ? nrows : 1) * (size_t)dff * sizeof(double));
        if (!h)
            return -1;
    }
    int rc = oracle_swiglu_rows(dtype, x, wg, wu, M, d, dff, rows, nrows,
                                NULL, NULL, h, nthreads);
    if (rc == 0) {
        int64_t nblocks = (d + COL_BLOCK - 1) / COL_BLOCK;
        int nt = threads_or_default(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) collapse(2)
        for (int64_t r = 0; r < nrows; ++r) {
            for (int64_t b = 0; b < nblocks; ++b) {
                int64_t j0 = b * COL_BLOCK;
                int64_t j1 = j0 + COL_BLOCK < d ? j0 + COL_BLOCK : d;
                for (int64_t j = j0; j < j1; ++j)
                    y[r * d + j] = 0.0;
                for (int64_t n = 0; n < dff; ++n) {
                    double hv = h[r * dff + n];
                    for (int64_t j = j0; j < j1; ++j)
                        y[r * d + j] += hv * elem(wd, dtype, n * d + j);
                }
            }
        }
    }
    if (!h_out)
        free(h);
    return rc;
}

/*
 * RMSNorm of the rows of r (M x d): n[m][i] = r[m][i] / sqrt(ms + eps) *
 * gamma[i], with ms = (1/d) sum_i r[m][i]^2 taken in ascending i.  The
 * pre-normalisation of the MLP half of a layer ("Anatomie d'un
 * transformeur sur GPU" §1.1 skeleton; §1.6 kernel 7); the pages do not
 * write the formula out, this is the usual root-mean-square normalisation
 * with a learned per-feature gain and a caller-given eps.  fp64 throughout.
 */
int oracle_rmsnorm_rows(int dtype, const void *r, const void *gamma, double eps, int64_t M,
                        int64_t d, double *out)
{
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) || M < 0 ||
        d <= 0 || !r || !gamma || !out || !(eps >= 0.0))
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            double v = elem(r, dtype, m * d + i);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)d + eps);
        for (int64_t i = 0; i < d; ++i)
            out[m * d + i] = elem(r, dtype, m * d + i) * inv * elem(gamma, dtype, i);
    }
    return 0;
}

/* Number of threads an nthreads=0 call would use (for reporting). */
int oracle_default_threads(void)
{
    return threads_or_default(0);
}
