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

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
