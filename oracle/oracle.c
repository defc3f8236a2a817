/*
 * oracle.c -- plain, slow CPU reference for the group-wise 4-bit (W4A16),
 * ternary 2-bit, 16-bit (W16A16) and MXFP4 small-M linear layer.  TEST INFRASTRUCTURE ONLY: nothing in
 * the product library links, includes or calls this file; only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark use it.
 *
 * What it computes, and where the pages define it:
 *   - The layer is y[M,N] = x[M,K] . W[K,N], M = 1 for one decode token and a
 *     few rows when draft tokens are verified together (Z100 vLLM port
 *     article, forum.sourcefind.cn, section 五 "单请求快了以后..."; Ninfer V100
 *     article, haowenji.com, section 三).
 *   - W is stored as 4-bit integers restored group by group: the integer is
 *     multiplied back by its group's scale after the zero point is taken off,
 *     w = (q - z) * s (Ninfer V100 article, section 十一, "groupwise-int"; Z100
 *     article, section 四, scale = size of one tick, zero point = where the
 *     ticks start).
 *   - Ternary weights take values -1, 0, +1 with one scale per group
 *     ("NINFER 三元引擎性能调优", markdownregistry page, sections 五/六).
 * The pages leave the storage layout open; the readings used here:
 *   qweight int32 [N][K/8]: nibble i (bits 4i..4i+3) of word (n, j) is
 *                           q[k = 8j + i][n];
 *   scales  fp16  [K/g][N]; zeros int32 [K/g][N/8], nibble i of word (gi, j)
 *                           is z[gi][8j + i];
 *   codes   int32 [N][K/16]: 2-bit field i (bits 2i..2i+1) of word (n, j) is
 *                           c[k = 16j + i][n], weight = c - 1, c = 3 invalid.
 *
 * Arithmetic: everything in IEEE binary64.  Decoding x and s is exact, the
 * dequantized weight is exact (|q - z| <= 15 times an 11-bit significand), each
 * product x*w is exact (<= 26 significant bits), and the sum over k runs in
 * ascending k with one rounding per addition.  No blocking, no reordering.
 * Parallelism is over output columns only (each column's sum is sequential).
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_EBADCODE (-2)

/* Threads OpenMP will use for the column loops. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 (8 exponent bits, bias 127,
 * 7 fraction bits). */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/128) * 2^(e-127) */
    return sign ? -v : v;
}

static double decode_x(const uint16_t* x, int x_is_bf16, size_t i)
{
    return x_is_bf16 ? oracle_bf16_to_f64(x[i]) : oracle_f16_to_f64(x[i]);
}

/* q[k][n] from qweight [N][K/8]. */
static int w4_q(const int32_t* qweight, int K, int k, int n)
{
    uint32_t word = (uint32_t)qweight[(size_t)n * (K / 8) + k / 8];
    return (int)((word >> (4 * (k % 8))) & 0xFu);
}

/* z[gi][n] from zeros [G][N/8]. */
static int w4_z(const int32_t* zeros, int N, int gi, int n)
{
    uint32_t word = (uint32_t)zeros[(size_t)gi * (N / 8) + n / 8];
    return (int)((word >> (4 * (n % 8))) & 0xFu);
}

/* c[k][n] from codes [N][K/16]. */
static int w2_c(const int32_t* codes, int K, int k, int n)
{
    uint32_t word = (uint32_t)codes[(size_t)n * (K / 16) + k / 16];
    return (int)((word >> (2 * (k % 16))) & 0x3u);
}

static int w4_shape_ok(int N, int K, int group)
{
    return N > 0 && K > 0 && group > 0 && K % group == 0 && K % 8 == 0 && N % 8 == 0;
}

static int w2_shape_ok(int N, int K, int group)
{
    return N > 0 && K > 0 && group > 0 && K % group == 0 && K % 16 == 0;
}

/* One dequantized 4-bit weight, w = (q - z) * s, in binary64. */
static double w4_weight(const int32_t* qweight, const uint16_t* scales, const int32_t* zeros,
                        int N, int K, int group, int k, int n)
{
    int gi = k / group;
    int q = w4_q(qweight, K, k, n);
    int z = w4_z(zeros, N, gi, n);
    double s = oracle_f16_to_f64(scales[(size_t)gi * N + n]);
    return (double)(q - z) * s;
}

/* Dequantize the whole matrix into W[K][N] (row k, column n). */
int oracle_w4_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* zeros,
                      int N, int K, int group, double* W)
{
    if (!w4_shape_ok(N, K, group)) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            W[(size_t)k * N + n] = w4_weight(qweight, scales, zeros, N, K, group, k, n);
    return ORACLE_OK;
}

/* y[m][c] = sum_k x[m][k] * W[k][cols[c]] for the listed columns, k ascending. */
int oracle_w4_gemv_cols(const uint16_t* x, int x_is_bf16, const int32_t* qweight,
                        const uint16_t* scales, const int32_t* zeros, int M, int N, int K,
                        int group, const int64_t* cols, int ncols, double* y)
{
    if (!w4_shape_ok(N, K, group) || M <= 0 || ncols < 0) return ORACLE_EINVAL;
    for (int c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int c = 0; c < ncols; ++c) {
        int n = (int)cols[c];
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double w = w4_weight(qweight, scales, zeros, N, K, group, k, n);
                acc += decode_x(x, x_is_bf16, (size_t)m * K + k) * w;
            }
            y[(size_t)m * ncols + c] = acc;
        }
    }
    return ORACLE_OK;
}

/* Full product y[M][N]. */
int oracle_w4_gemv(const uint16_t* x, int x_is_bf16, const int32_t* qweight,
                   const uint16_t* scales, const int32_t* zeros, int M, int N, int K, int group,
                   double* y)
{
    if (!w4_shape_ok(N, K, group) || M <= 0) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double w = w4_weight(qweight, scales, zeros, N, K, group, k, n);
                acc += decode_x(x, x_is_bf16, (size_t)m * K + k) * w;
            }
            y[(size_t)m * N + n] = acc;
        }
    }
    return ORACLE_OK;
}

/* Ternary: weight = (c - 1) * s; returns ORACLE_EBADCODE if any code is 3. */
static int w2_all_codes_valid(const int32_t* codes, int N, int K)
{
    size_t words = (size_t)N * (K / 16);
    for (size_t i = 0; i < words; ++i) {
        uint32_t w = (uint32_t)codes[i];
        for (int f = 0; f < 16; ++f)
            if (((w >> (2 * f)) & 3u) == 3u) return 0;
    }
    return 1;
}

static double w2_weight(const int32_t* codes, const uint16_t* scales, int N, int K, int group,
                        int k, int n)
{
    int c = w2_c(codes, K, k, n);
    double s = oracle_f16_to_f64(scales[(size_t)(k / group) * N + n]);
    return (double)(c - 1) * s;
}

int oracle_w2t_dequant(const int32_t* codes, const uint16_t* scales, int N, int K, int group,
                       double* W)
{
    if (!w2_shape_ok(N, K, group)) return ORACLE_EINVAL;
    if (!w2_all_codes_valid(codes, N, K)) return ORACLE_EBADCODE;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            W[(size_t)k * N + n] = w2_weight(codes, scales, N, K, group, k, n);
    return ORACLE_OK;
}

int oracle_w2t_gemv_cols(const uint16_t* x, int x_is_bf16, const int32_t* codes,
                         const uint16_t* scales, int M, int N, int K, int group,
                         const int64_t* cols, int ncols, double* y)
{
    if (!w2_shape_ok(N, K, group) || M <= 0 || ncols < 0) return ORACLE_EINVAL;
    for (int c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return ORACLE_EINVAL;
    /* Only the listed columns' codes are checked here, so a sample stays cheap. */
    for (int c = 0; c < ncols; ++c)
        for (int k = 0; k < K; ++k)
            if (w2_c(codes, K, k, (int)cols[c]) == 3) return ORACLE_EBADCODE;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int c = 0; c < ncols; ++c) {
        int n = (int)cols[c];
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += decode_x(x, x_is_bf16, (size_t)m * K + k) *
                       w2_weight(codes, scales, N, K, group, k, n);
            y[(size_t)m * ncols + c] = acc;
        }
    }
    return ORACLE_OK;
}

int oracle_w2t_gemv(const uint16_t* x, int x_is_bf16, const int32_t* codes,
                    const uint16_t* scales, int M, int N, int K, int group, double* y)
{
    if (!w2_shape_ok(N, K, group) || M <= 0) return ORACLE_EINVAL;
    if (!w2_all_codes_valid(codes, N, K)) return ORACLE_EBADCODE;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += decode_x(x, x_is_bf16, (size_t)m * K + k) *
                       w2_weight(codes, scales, N, K, group, k, n);
            y[(size_t)m * N + n] = acc;
        }
    }
    return ORACLE_OK;
}

/* ---- 16-bit weights (W16A16) --------------------------------------------
 * The Z100 article, section 六, measures the same small-M linear layer with
 * FP16/BF16 weights (no quantization): y[m][n] = sum_k x[m][k] * w[n][k],
 * with w stored as the layer's own [N][K] matrix of 16-bit values of the
 * same type as x.  Both factors decode exactly and their product (at most 22
 * significant bits) is exact in binary64; the sum runs in ascending k. */
static int w16_shape_ok(int M, int N, int K) { return M > 0 && N > 0 && K > 0; }

int oracle_w16_gemv(const uint16_t* x, int is_bf16, const uint16_t* w, int M, int N, int K,
                    double* y)
{
    if (!w16_shape_ok(M, N, K)) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += decode_x(x, is_bf16, (size_t)m * K + k) *
                       decode_x(w, is_bf16, (size_t)n * K + k);
            y[(size_t)m * N + n] = acc;
        }
    }
    return ORACLE_OK;
}

int oracle_w16_gemv_cols(const uint16_t* x, int is_bf16, const uint16_t* w, int M, int N, int K,
                         const int64_t* cols, int ncols, double* y)
{
    if (!w16_shape_ok(M, N, K) || ncols < 0) return ORACLE_EINVAL;
    for (int c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int c = 0; c < ncols; ++c) {
        int n = (int)cols[c];
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += decode_x(x, is_bf16, (size_t)m * K + k) *
                       decode_x(w, is_bf16, (size_t)n * K + k);
            y[(size_t)m * ncols + c] = acc;
        }
    }
    return ORACLE_OK;
}

/* ---- MXFP4 weights --------------------------------------------------------
 * The Z100 article's closing section names FP4/MXFP4 as the next weight
 * format: 4-bit floating-point elements sharing one block-level scale
 * (microscaling), defined publicly by the Open Compute Project's MX
 * specification, which that section cites.  Readings of that definition
 * (MX v1.0, MXFP4):
 *   - blocks of 32 consecutive elements along K share one scale;
 *   - element: FP4 E2M1 -- bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 *     mantissa; exponent field 0 is subnormal (0 or 0.5), no inf or NaN;
 *   - scale: E8M0 -- an unsigned 8-bit exponent, value 2^(E - 127), and the
 *     code 255 is NaN;
 *   - the weight is element * scale.
 * Storage (the pages leave it open): qweight uint8 [N][K/2], element k of
 * row n in byte k/2, low nibble for even k; scales uint8 [N][K/32].  K must
 * be a multiple of 32.  Every weight and every product with a 16-bit x is
 * exact in binary64 (at most 2 + 11 significant bits, exponents within
 * range); the sum runs in ascending k. */
double oracle_e2m1_to_f64(int code)
{
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

double oracle_e8m0_to_f64(int code)
{
    code &= 0xff;
    return code == 255 ? NAN : ldexp(1.0, code - 127);
}

static int mx_shape_ok(int N, int K) { return N > 0 && K > 0 && K % 32 == 0; }

static double mx_weight(const uint8_t* qweight, const uint8_t* scales, int K, int n, int k)
{
    const uint8_t b = qweight[(size_t)n * (K / 2) + k / 2];
    const int code = (k & 1) ? (b >> 4) : (b & 15);
    return oracle_e2m1_to_f64(code) * oracle_e8m0_to_f64(scales[(size_t)n * (K / 32) + k / 32]);
}

/* w[n][k] in binary64, [N][K]. */
int oracle_mx_dequant(const uint8_t* qweight, const uint8_t* scales, int N, int K, double* w)
{
    if (!mx_shape_ok(N, K)) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            w[(size_t)n * K + k] = mx_weight(qweight, scales, K, n, k);
    return ORACLE_OK;
}

/* y[m][c] = sum_k x[m][k] w[cols[c]][k] for the listed output columns. */
int oracle_mx_gemv_cols(const uint16_t* x, int x_is_bf16, const uint8_t* qweight,
                        const uint8_t* scales, int M, int N, int K, const int64_t* cols, int ncols,
                        double* y)
{
    if (!mx_shape_ok(N, K) || M <= 0 || ncols < 0) return ORACLE_EINVAL;
    for (int c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int c = 0; c < ncols; ++c) {
        const int n = (int)cols[c];
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += decode_x(x, x_is_bf16, (size_t)m * K + k) * mx_weight(qweight, scales, K, n, k);
            y[(size_t)m * ncols + c] = acc;
        }
    }
    return ORACLE_OK;
}

/* y[M][N] = x[M][K] . w^T. */
int oracle_mx_gemv(const uint16_t* x, int x_is_bf16, const uint8_t* qweight, const uint8_t* scales,
                   int M, int N, int K, double* y)
{
    if (!mx_shape_ok(N, K) || M <= 0) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += decode_x(x, x_is_bf16, (size_t)m * K + k) * mx_weight(qweight, scales, K, n, k);
            y[(size_t)m * N + n] = acc;
        }
    return ORACLE_OK;
}
