/*
 * oracle.c -- plain, slow CPU reference for the group-quantized weight-only GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (fp64 throughout):
 *
 *   w_hat[k,n] = s[g,n] * (q[k,n] - z[g,n]),        g = k / G
 *   ref[m,n]   = sum_{k=0..K-1} a[m,k] * w_hat[k,n]  (k ascending)
 *   bound[m,n] = sum_{k=0..K-1} |a[m,k] * w_hat[k,n]|
 *
 * This is the check the page "quantization-and-fused-kernels"
 * (arganzheng.life) prescribes in section 八 (numerical validation, second
 * principle): dequantize the packed weights by definition to
 * W_hat = s * (q - z) and multiply the activations by it, so that a kernel
 * differs from the reference only by its summation order and rounding.
 * Summed over the groups, it is the blockwise definition on the page
 * "04 · 分组量化 GEMM 内核" (developer.aliyun.com), section 二:
 * out = sum_g a_scale[m][g] * b_scale[n][g] * sum_{k in g} Aq[m][k] * Wq[n][k].
 *
 * Storage it reads (canonical layouts):
 *   int4 weights  uint32 [K/8][N]: code of k = 8r + j in bits 4j..4j+3
 *                 (packing rule: arganzheng.life page, section 二.4)
 *   int8 weights  int8 [K][N], codes in [-127, 127], zero-point 0
 *                 (Q8_0, developer.aliyun.com page, section 二)
 *   scales        [K/G][N], float32 or bf16 bits
 *   zero-points   uint32 [K/G][ceil(N/8)], column n = 8c + j in bits 4j..4j+3;
 *                 without them int4 codes use zero-point 8 (the symmetric
 *                 convention of the teaching GEMV, arganzheng.life section 九.4)
 *   activations   [M][K] float32, bf16 bits, or int8 codes with float32
 *                 scales a_scale[M][K/G] (a = a_scale * code)
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC oracle.c
 * OpenMP splits the work over output columns only; the per-element
 * summation order does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_W4 = 0, OR_W8 = 1 };
enum { OR_A_F32 = 0, OR_A_BF16 = 1, OR_A_I8 = 2 };
enum { OR_S_F32 = 0, OR_S_BF16 = 1 };

/* bf16 is the upper half of a float32 pattern: widening is a 16-bit shift. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double f32_to_double(const float *p) { return (double)*p; }

/* Weight code q[k,n] as an integer. */
static int weight_code(const void *W, int wfmt, int N, int k, int n)
{
    if (wfmt == OR_W4) {
        const uint32_t *w = (const uint32_t *)W;
        uint32_t word = w[(size_t)(k / 8) * N + n];
        return (int)((word >> (4 * (k % 8))) & 0xFu);
    }
    return (int)((const int8_t *)W)[(size_t)k * N + n];
}

/* Zero-point z[g,n]. */
static int zero_point(const uint32_t *Z, int wfmt, int has_zp, int N, int g, int n)
{
    if (wfmt == OR_W8)
        return 0;
    if (!has_zp)
        return 8;
    int words_per_row = (N + 7) / 8;
    uint32_t word = Z[(size_t)g * words_per_row + n / 8];
    return (int)((word >> (4 * (n % 8))) & 0xFu);
}

static double scale_value(const void *S, int sfmt, int N, int g, int n)
{
    size_t i = (size_t)g * N + n;
    if (sfmt == OR_S_BF16)
        return bf16_to_double(((const uint16_t *)S)[i]);
    return f32_to_double(&((const float *)S)[i]);
}

static double activation(const void *A, const float *a_scale, int afmt, int K, int G, int m, int k)
{
    size_t i = (size_t)m * K + k;
    if (afmt == OR_A_F32)
        return f32_to_double(&((const float *)A)[i]);
    if (afmt == OR_A_BF16)
        return bf16_to_double(((const uint16_t *)A)[i]);
    return (double)a_scale[(size_t)m * (K / G) + k / G] * (double)((const int8_t *)A)[i];
}

/* Structural checks: the shapes the definition needs. Returns 0 or -1. */
int oracle_check(int M, int N, int K, int G, int wfmt, int afmt, int sfmt, int has_zp)
{
    if (M < 0 || N <= 0 || K <= 0 || G <= 0)
        return -1;
    if (K % G != 0)
        return -1;
    if (wfmt != OR_W4 && wfmt != OR_W8)
        return -1;
    if (afmt < OR_A_F32 || afmt > OR_A_I8 || sfmt < OR_S_F32 || sfmt > OR_S_BF16)
        return -1;
    if (wfmt == OR_W4 && G % 8 != 0)  /* a packed word must not straddle two groups */
        return -1;
    if (has_zp && wfmt != OR_W4)
        return -1;
    return 0;
}

/* The column-index list: NULL means all N columns. */
static int col_index(const int64_t *cols, int j) { return cols ? (int)cols[j] : j; }
static int row_index(const int64_t *rows, int i) { return rows ? (int)rows[i] : i; }

static int check_indices(const int64_t *idx, int count, int limit)
{
    if (!idx)
        return 0;
    for (int i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= limit)
            return -1;
    return 0;
}

/* Dequantized weight column n: w_hat[k] = s[k/G, n] * (q[k, n] - z[k/G, n]). */
static void dequant_column(const void *W, const void *S, const uint32_t *Z, int N, int K, int G,
                           int wfmt, int sfmt, int has_zp, int n, double *w_hat)
{
    for (int k = 0; k < K; ++k) {
        int g = k / G;
        int q = weight_code(W, wfmt, N, k, n);
        int z = zero_point(Z, wfmt, has_zp, N, g, n);
        w_hat[k] = scale_value(S, sfmt, N, g, n) * (double)(q - z);
    }
}

/* w_hat for the selected columns: out[k * ncols + j]. */
int oracle_dequant(int N, int K, int G, int wfmt, int sfmt, int has_zp, const void *W,
                   const void *S, const uint32_t *Z, const int64_t *cols, int ncols, double *out)
{
    if (oracle_check(0, N, K, G, wfmt, OR_A_F32, sfmt, has_zp) != 0)
        return -1;
    if (!cols)
        ncols = N;
    if (check_indices(cols, ncols, N) != 0 || !W || !S || (has_zp && !Z) || !out)
        return -1;
    double *col = (double *)malloc(sizeof(double) * (size_t)K);
    if (!col)
        return -2;
    for (int j = 0; j < ncols; ++j) {
        dequant_column(W, S, Z, N, K, G, wfmt, sfmt, has_zp, col_index(cols, j), col);
        for (int k = 0; k < K; ++k)
            out[(size_t)k * ncols + j] = col[k];
    }
    free(col);
    return 0;
}

/*
 * ref and bound for the selected rows x columns: ref[i * ncols + j] is output
 * (rows[i], cols[j]). rows/cols NULL selects all M rows / N columns.
 */
int oracle_qgemm(int M, int N, int K, int G, int wfmt, int afmt, int sfmt, int has_zp,
                 const void *A, const float *a_scale, const void *W, const void *S,
                 const uint32_t *Z, const int64_t *rows, int nrows, const int64_t *cols,
                 int ncols, double *ref, double *bound)
{
    if (oracle_check(M, N, K, G, wfmt, afmt, sfmt, has_zp) != 0)
        return -1;
    if (!rows)
        nrows = M;
    if (!cols)
        ncols = N;
    if (check_indices(rows, nrows, M) != 0 || check_indices(cols, ncols, N) != 0)
        return -1;
    if (nrows == 0 || ncols == 0)
        return 0;
    if (!A || !W || !S || (has_zp && !Z) || (afmt == OR_A_I8 && !a_scale) || !ref || !bound)
        return -1;

    int failed = 0;
#pragma omp parallel
    {
        double *w_hat = (double *)malloc(sizeof(double) * (size_t)K);
        if (!w_hat) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int j = 0; j < ncols; ++j) {
            if (!w_hat)
                continue;
            int n = col_index(cols, j);
            dequant_column(W, S, Z, N, K, G, wfmt, sfmt, has_zp, n, w_hat);
            for (int i = 0; i < nrows; ++i) {
                int m = row_index(rows, i);
                double sum = 0.0, mag = 0.0;
                for (int k = 0; k < K; ++k) {
                    double term = activation(A, a_scale, afmt, K, G, m, k) * w_hat[k];
                    sum += term;
                    mag += fabs(term);
                }
                ref[(size_t)i * ncols + j] = sum;
                bound[(size_t)i * ncols + j] = mag;
            }
        }
        free(w_hat);
    }
    return failed ? -2 : 0;
}

/*
 * Integer per-group partial sums for int8 activation codes:
 * P[(i * (K/G) + g) * ncols + j] = sum_{k in g} Aq[m,k] * (q[k,n] - z[g,n]).
 * The integer dot over a whole group is the exact quantity the blockwise
 * definition scales (developer.aliyun.com page, section 二).
 */
int oracle_int_partials(int M, int N, int K, int G, int wfmt, int has_zp, const int8_t *Aq,
                        const void *W, const uint32_t *Z, const int64_t *rows, int nrows,
                        const int64_t *cols, int ncols, int64_t *P)
{
    if (oracle_check(M, N, K, G, wfmt, OR_A_I8, OR_S_F32, has_zp) != 0)
        return -1;
    if (!rows)
        nrows = M;
    if (!cols)
        ncols = N;
    if (check_indices(rows, nrows, M) != 0 || check_indices(cols, ncols, N) != 0)
        return -1;
    if (nrows == 0 || ncols == 0)
        return 0;
    if (!Aq || !W || (has_zp && !Z) || !P)
        return -1;
    int ngroups = K / G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int j = 0; j < ncols; ++j) {
        int n = col_index(cols, j);
        for (int i = 0; i < nrows; ++i) {
            int m = row_index(rows, i);
            for (int g = 0; g < ngroups; ++g) {
                int64_t acc = 0;
                int z = zero_point(Z, wfmt, has_zp, N, g, n);
                for (int k = g * G; k < (g + 1) * G; ++k)
                    acc += (int64_t)Aq[(size_t)m * K + k] * (int64_t)(weight_code(W, wfmt, N, k, n) - z);
                P[((size_t)i * ngroups + g) * ncols + j] = acc;
            }
        }
    }
    return 0;
}

/*
 * Dynamic per-group int8 quantization of float32 activations: the absmax ->
 * scale -> round -> clamp kernel of the page "quantization-and-fused-kernels"
 * (arganzheng.life), section 四.5 (there for fp8 per token; here with int8
 * codes per (row, group of G), the activation format that the blockwise
 * product of the page "04 · 分组量化 GEMM 内核" (developer.aliyun.com),
 * section 二, consumes). Read as, for every row m and group g, in float32
 * (the precision the codes are decided in):
 *     amax        = max_k |a[m,k]|                     (exact)
 *     a_scale[m,g] = amax / 127, or 1 if amax == 0     (one rounding)
 *     Aq[m,k]     = clamp(rint(a[m,k] / a_scale[m,g]), -127, 127)
 * with rint rounding halves to even. A group of zeros gets scale 1 and
 * codes 0 (the section's guard against dividing by zero).
 * Returns 0, or -1 on bad shapes.
 */
int oracle_quantize_act(int M, int K, int G, const float *A, int8_t *Aq, float *a_scale)
{
    if (M < 0 || K <= 0 || G <= 0 || K % G != 0)
        return -1;
    const int ng = K / G;
    for (int m = 0; m < M; ++m) {
        for (int g = 0; g < ng; ++g) {
            const float *a = A + (size_t)m * K + (size_t)g * G;
            float amax = 0.0f;
            for (int j = 0; j < G; ++j) {
                float v = fabsf(a[j]);
                if (v > amax)
                    amax = v;
            }
            const float sc = amax > 0.0f ? amax / 127.0f : 1.0f;
            a_scale[(size_t)m * ng + g] = sc;
            for (int j = 0; j < G; ++j) {
                float q = rintf(a[j] / sc);
                if (q > 127.0f)
                    q = 127.0f;
                if (q < -127.0f)
                    q = -127.0f;
                Aq[(size_t)m * K + (size_t)g * G + j] = (int8_t)q;
            }
        }
    }
    return 0;
}

/*
 * ---------------------------------------------------------------------------
 * FP8 W8A8 (E4M3, "fn" variant), the variant the page
 * "quantization-and-fused-kernels" (arganzheng.life) contrasts with W4A16 in
 * section 四: both operands in FP8, products accumulated in float32, scales
 * either outside the K sum (section 四.2) or per 128-wide K block inside it
 * (section 四.3).
 * ---------------------------------------------------------------------------
 *
 * Value of an 8-bit E4M3 code, from the format's definition (same page,
 * section 二.1: 1 sign bit, 4 exponent bits, 3 mantissa bits, largest finite
 * value 448, no infinities, and the pattern with exponent and mantissa all
 * ones is NaN). Exponent bias 7; exponent field 0 holds the subnormals:
 *   e == 0:  (-1)^s * (f / 8) * 2^(1 - 7)
 *   e  > 0:  (-1)^s * (1 + f / 8) * 2^(e - 7)
 * Returns NaN for 0x7F and 0xFF.
 */
double oracle_fp8_value(int code)
{
    const int s = (code >> 7) & 1, e = (code >> 3) & 0xF, f = code & 7;
    if (e == 0xF && f == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)f / 8.0, 1 - 7) : ldexp(1.0 + (double)f / 8.0, e - 7);
    return s ? -v : v;
}

/*
 * A float32 value x with |x| <= 448 rounded to the nearest E4M3 code, ties to
 * the code whose mantissa (lowest bit) is even; the sign is kept, so values
 * that round to zero from below give negative zero (0x80). Found by comparing
 * x with every finite non-negative code.
 */
static int fp8_round(float x)
{
    const int neg = signbit(x) != 0;
    const double ax = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double d = fabs(oracle_fp8_value(c) - ax);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return best | (neg << 7);
}

/*
 * Dynamic FP8 quantization of bf16 activations A[M][K], after the per-token
 * kernel of the same page, section 四.5 (absmax reduction, scale = max / 448,
 * divide, saturate to +-448, round to FP8): with block == 0 one scale per row
 * (per token, a_scale[M]); with block == 128 one scale per 128 consecutive
 * elements of a row (the 1 x 128 activation blocks of section 四.3,
 * a_scale[M][K/128]). In float32 (the precision the codes are decided in):
 *   amax    = max |a| over the row or block         (exact)
 *   a_scale = amax / 448, or 1 when amax == 0       (one rounding)
 *   x       = a / a_scale                           (one rounding)
 *   code    = fp8_round(clamp(x, -448, 448))
 * The section's optional upper bound on the scale is not used, and its
 * minimum scale (whose value the page does not give) is read as the guard of
 * an all-zero row or block. Returns 0, or -1 on bad shapes.
 */
int oracle_fp8_quantize(int M, int K, int block, const uint16_t *A, uint8_t *Aq, float *a_scale)
{
    if (M < 0 || K <= 0 || !(block == 0 || block == 128) || (block && K % block != 0))
        return -1;
    const int len = block ? block : K;
    const int nb = K / len;
    for (int m = 0; m < M; ++m) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t *a = A + (size_t)m * K + (size_t)b * len;
            float amax = 0.0f;
            for (int j = 0; j < len; ++j) {
                const float v = fabsf((float)bf16_to_double(a[j]));
                if (v > amax)
                    amax = v;
            }
            const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
            a_scale[(size_t)m * nb + b] = sc;
            for (int j = 0; j < len; ++j) {
                float x = (float)bf16_to_double(a[j]) / sc;
                if (x > 448.0f)
                    x = 448.0f;
                if (x < -448.0f)
                    x = -448.0f;
                Aq[(size_t)m * K + (size_t)b * len + j] = (uint8_t)fp8_round(x);
            }
        }
    }
    return 0;
}

/*
 * FP8 GEMM reference, fp64. Aq: E4M3 codes [M][K]; Wq: E4M3 codes [N][K]
 * (each output channel's K codes contiguous). With v() = oracle_fp8_value:
 *   scaling 0 (per-token x per-channel, section 四.2; a_scale[M], w_scale[N]):
 *     ref[m,n] = a_scale[m] * w_scale[n] * sum_k v(Aq[m,k]) * v(Wq[n,k])
 *   scaling 1 (per-block, section 四.3; a_scale[M][K/128], w_scale[N/128][K/128]):
 *     ref[m,n] = sum_b a_scale[m,b] * w_scale[n/128,b] * sum_{k in b} v(Aq[m,k]) * v(Wq[n,k])
 * bound[m,n] = the same sums of absolute values of the terms. k ascending;
 * rows / cols select outputs (NULL: all). Returns 0, or -1 on bad arguments.
 */
int oracle_fp8_gemm(int M, int N, int K, int scaling, const uint8_t *Aq, const float *a_scale,
                    const uint8_t *Wq, const float *w_scale, const int64_t *rows, int nrows,
                    const int64_t *cols, int ncols, double *ref, double *bound)
{
    if (M < 0 || N <= 0 || K <= 0 || !(scaling == 0 || scaling == 1))
        return -1;
    if (scaling == 1 && (K % 128 != 0 || N % 128 != 0))
        return -1;
    if (check_indices(rows, nrows, M) || check_indices(cols, ncols, N))
        return -1;
    const int nb = K / 128;
#pragma omp parallel for schedule(dynamic, 1)
    for (int j = 0; j < ncols; ++j) {
        const int n = col_index(cols, j);
        for (int i = 0; i < nrows; ++i) {
            const int m = row_index(rows, i);
            double total = 0.0, total_abs = 0.0;
            for (int k = 0; k < K; ++k) {
                double sc;
                if (scaling == 0)
                    sc = (double)a_scale[m] * (double)w_scale[n];
                else
                    sc = (double)a_scale[(size_t)m * nb + k / 128] * (double)w_scale[(size_t)(n / 128) * nb + k / 128];
                const double prod = sc * oracle_fp8_value(Aq[(size_t)m * K + k]) * oracle_fp8_value(Wq[(size_t)n * K + k]);
                total += prod;
                total_abs += fabs(prod);
            }
            ref[(size_t)i * ncols + j] = total;
            bound[(size_t)i * ncols + j] = total_abs;
        }
    }
    return 0;
}

/* Threads the OpenMP loops use from now on (n >= 1); returns the previous
 * count. The per-element summation order does not depend on it. */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    const int prev = omp_get_max_threads();
    if (n >= 1)
        omp_set_num_threads(n);
    return prev;
#else
    (void)n;
    return 1;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
