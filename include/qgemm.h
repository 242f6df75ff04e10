/*
 * qgemm.h -- C ABI of the group-quantized weight-only GEMM for MI355X (gfx950).
 *
 * It computes, for m < M and n < N,
 *
 *     out[m,n] = sum_g  s[g,n] * sum_{k in group g}  a[m,k] * (q[k,n] - z[g,n])
 *
 * with groups of G consecutive k (G = 32 or 128). This is the quantity of the
 * page "04 · 分组量化 GEMM 内核" (developer.aliyun.com), section 二
 * (out[m][n] = sum_g a_scale[m][g] * b_scale[n][g] * sum_{k in g} Aq*Wq), and
 * of the W4A16 GEMM of the page "quantization-and-fused-kernels"
 * (arganzheng.life), section 三.1 (int4 weights with per-group scales
 * [K/g, N] and optional int4-packed zero-points [K/g, N/8], real value
 * s * (q - z), fp32 accumulation).
 *
 * Conventions (all arrays row-major, caller-owned):
 *   - int4 weights (canonical): uint32 [K/8][N]; the code of k = 8r + j sits
 *     in bits 4j..4j+3 of word (r, n) (arganzheng.life section 二.4).
 *     Without zero-points the zero-point is 8, so code c means c - 8
 *     (section 九.4); a signed int4 value v in [-8, 7] is stored as v + 8.
 *   - int8 weights (canonical): int8 [K][N], codes in [-127, 127], zero-point 0
 *     (Q8_0, developer.aliyun.com section 二).
 *   - scales: [K/G][N], bf16 or float32 by precision (below).
 *   - zero-points: uint32 [K/G][N/8], column n = 8c + j in bits 4j..4j+3 of
 *     word (g, c); int4 weights only; requires N % 8 == 0.
 *   - activations: [M][K], bf16, float32, or int8 codes with float32 per-group
 *     scales a_scales [M][K/G] (a = a_scale * code).
 *   - out: [M][N], bf16 (rounded to nearest even once, at the end) or float32.
 *   Accumulation is float32 throughout (arganzheng.life section 二.2).
 *
 * Memory and streams: every pointer passed to qgemm_pack / qgemm_run is a
 * device pointer owned by the caller. The library allocates no device memory.
 * All work is enqueued on `stream` (a hipStream_t; NULL is the null stream);
 * no call synchronizes the host or copies between host and device.
 *
 * Errors: arguments are validated before anything is enqueued; on error
 * nothing is launched and nothing is written. QG_EHIP reports an error of the
 * library's own launches only: an error that an earlier runtime call of the
 * caller's left pending on the thread (the runtime keeps the last one until
 * it is read) is read and dropped right before the first launch. A fault of
 * the device persists and is still reported.
 *
 * The library and the caller must share one HIP runtime (the one that made
 * the caller's streams and memory): in a process that also loads PyTorch,
 * load PyTorch first, since it ships its own runtime under the same name.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    QG_OK = 0,
    QG_EINVAL = -1,        /* null pointer, negative/zero size, K % G != 0          */
    QG_EUNSUPPORTED = -2,  /* G not 32/128, unknown prec, zero-points not allowed  */
    QG_EWORKSPACE = -3,    /* workspace smaller than qgemm_workspace_bytes()        */
    QG_EALIGN = -4,        /* a pointer is not 16-byte aligned                      */
    QG_EHIP = -5           /* the HIP runtime reported an error                     */
};

/* Precisions: weight codes | activations | scales | out. */
enum {
    QG_W4_A_BF16 = 1,      /* int4  | bf16                  | bf16    | bf16    */
    QG_W4_A_F32 = 2,       /* int4  | float32               | float32 | float32 */
    QG_W8_A_F32 = 3,       /* int8  | float32               | float32 | float32 */
    QG_W4_A_I8 = 4,        /* int4  | int8 + a_scales f32   | float32 | float32 */
    QG_W8_A_I8 = 5,        /* int8  | int8 + a_scales f32   | float32 | float32 */
    QG_W4_A_BF16_OF32 = 6, /* int4  | bf16                  | bf16    | float32 */
    QG_W4_A_F32_DQ8 = 7,   /* int4  | float32, quantized    | float32 | float32 */
    QG_W8_A_F32_DQ8 = 8    /* int8  | float32, quantized    | float32 | float32 */
};
/* Precisions 7 and 8 take float32 activations and quantize them inside the
 * call, exactly as qgemm_quantize_activations does: for M <= 4 inside the
 * product kernel (the codes and scales stay on chip), above that with a
 * pre-pass into the workspace. The product is then that of precision 4 / 5
 * on those codes and scales, bit for bit. */

/* Paths (for qgemm_plan / qgemm_run_ex). */
enum {
    QG_PATH_AUTO = -1,
    QG_PATH_GEMV = 0,      /* vector-ALU path: weight streaming, any M               */
    QG_PATH_GEMM = 1,      /* MFMA path: bf16 activations (prec 1 and 6), G == 128,
                              N % 8 == 0, M <= 65535                                   */
    QG_PATH_SMALL = 2      /* small-M MFMA path: weights streamed once, M <= 64,
                              bf16 activations, G == 128, N % 8 == 0                  */
};

/*
 * Version of the packed weight layout written by qgemm_pack. A packed buffer
 * saved by one version must be re-packed if the version differs.
 *
 * Layout version 2. Np = N rounded up to a multiple of 256 (columns >= N are
 * zero); R = K/8 (int4) or K/4 (int8) word-rows. The words are stored in
 * tiles of 64 columns, each tile's rows one after another:
 *     word (r, n) is at index ((n / 64) * R + r) * 64 + (n % 64)
 *   int4: word (r, n) holds the 8 codes of k = 8r .. 8r+7 of column n with the
 *         even k in the low half-word and the odd k in the high half-word:
 *         bits 4p..4p+3 hold k = 8r + {0,2,4,6,1,3,5,7}[p].
 *   int8: byte j of word (r, n) is the code of k = 4r + j.
 */
int qgemm_layout_version(void);

/* Bytes of the packed weight buffer for a K x N weight of precision prec
 * (0 if the arguments are invalid). */
size_t qgemm_packed_bytes(int K, int N, int prec);

/*
 * Repack canonical weights (device pointer, layout above) into the kernel
 * layout (device pointer of qgemm_packed_bytes(K, N, prec) bytes). Requires
 * K % 8 == 0 (int4) or K % 4 == 0 (int8). Enqueued on `stream`.
 */
int qgemm_pack(const void *w_canonical, void *w_packed, int K, int N, int prec, void *stream);

/*
 * Device workspace bytes qgemm_run needs for this problem (0: none, and the
 * workspace pointer may be NULL). The workspace holds the int8 codes and
 * float32 scales of in-call activation quantization (precisions 7 and 8,
 * M > 4), on the tiled MFMA path the pre-pass's fp16 activations, row
 * exponents and float32 scales, and the float32 partial sums of a K-split;
 * its contents before a call do not matter. Calls that share a workspace
 * must not run concurrently.
 */
size_t qgemm_workspace_bytes(int M, int N, int K, int group, int prec);

/*
 * The plan qgemm_run_ex would use: path (QG_PATH_GEMV, QG_PATH_GEMM or QG_PATH_SMALL),
 * nsplit (number of K-slices of whole groups whose float32 partial sums are
 * added in the fixed order z = 0, 1, ..., nsplit-1) and workspace bytes.
 * force_path: QG_PATH_AUTO or a path; force_nsplit: <= 0 for automatic, else
 * the requested split (clamped to [1, K/G]). The plan is a pure function of
 * the arguments and the device's compute-unit count.
 */
int qgemm_plan(int M, int N, int K, int group, int prec, int force_path, int force_nsplit,
               int *path, int *nsplit, size_t *workspace_bytes);

/*
 * out = the group-quantized product described at the top of this file.
 * Enqueues one kernel, or two when K is split (nsplit > 1: the partial sums
 * of the K-slices, then their fixed-order reduction); the tiled MFMA path
 * first enqueues a pre-pass that writes the activations as fp16 scaled by a
 * power of two per row, the row exponents, and the scales as float32, into
 * the workspace.
 *   M >= 0 (M == 0 is a no-op), N >= 1, K >= 1, K % group == 0, group in {32, 128}.
 *   A:         activations [M][K] (bf16 / float32 / int8 by prec)
 *   a_scales:  float32 [M][K/G] for *_A_I8, else NULL (unused)
 *   w_packed:  output of qgemm_pack
 *   scales:    [K/G][N] (bf16 for prec 1 and 6, else float32)
 *   zeros:     uint32 [K/G][N/8] when has_zp (int4 only, N % 8 == 0), else NULL
 *   out:       [M][N] (bf16 for prec 1, else float32)
 *   workspace: device memory of at least qgemm_workspace_bytes() (see there)
 * All pointers must be 16-byte aligned. Results are bitwise reproducible for
 * a given plan (fixed partition and fixed summation orders, no floating-point
 * atomics).
 */
int qgemm_run(int M, int N, int K, int group, int prec, int has_zp, const void *A,
              const void *a_scales, const void *w_packed, const void *scales, const void *zeros,
              void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Fused gate_up product with SwiGLU's gate step, for a Llama-style FFN
 * (page "quantization-and-fused-kernels" (arganzheng.life), section 五.2:
 * the gate_up GEMM writes [M][2d], gate columns first, and
 * out = silu(gate) * up with silu(x) = x * sigmoid(x) = x / (1 + e^-x); the
 * MoE pipeline of section 六.1 has the same step between its two GEMMs).
 * Here the step runs in the product's epilogue: out [M][d] is written once
 * and the [M][2d] product never reaches memory.
 *
 * The weight is one canonical int4 matrix of N = 2d columns (gate columns
 * 0..d-1, up columns d..2d-1), scales [K/G][2d] bf16 and zero-points
 * [K/G][2d/8] in that canonical column order, as for qgemm_run.
 *   d: output columns, d % 32 == 0; prec: QG_W4_A_BF16 (bf16 out) or
 *   QG_W4_A_BF16_OF32 (float32 out); A: bf16 [M][K].
 * qgemm_pack_gate_up packs it in gate-up order: packed tile t (64 columns)
 * holds gate columns 32t..32t+31 and then up columns d+32t..d+32t+31, so
 * that one workgroup makes both inputs of each of its outputs; the buffer
 * has qgemm_packed_bytes(K, 2d, prec) bytes. The product runs on the GEMV or
 * small-M path (the plan of qgemm_plan for N = 2d); a problem that would take
 * the tiled GEMM (M > 64 with group 128) returns QG_EUNSUPPORTED.
 * out[m][j] = silu(y[m][j]) * y[m][d + j] with y the float32 product of
 * qgemm_run (the same sums in the same order), the step in float32 (expf),
 * then one rounding to the output type. With a K-split the reduce kernel
 * applies the step after its fixed-order sum. Workspace, errors, streams and
 * reproducibility are those of qgemm_run.
 */
int qgemm_pack_gate_up(const void *w_canonical, void *w_packed, int K, int d, int prec, void *stream);
int qgemm_gate_up_plan(int M, int d, int K, int group, int prec, int force_path, int force_nsplit, int *path,
                       int *nsplit, size_t *workspace_bytes);
size_t qgemm_gate_up_workspace_bytes(int M, int d, int K, int group, int prec);
int qgemm_run_gate_up_silu(int M, int d, int K, int group, int prec, int has_zp, const void *A,
                           const void *w_packed, const void *scales, const void *zeros, void *out,
                           void *workspace, size_t workspace_bytes, void *stream);
/* qgemm_run_gate_up_silu with an explicit plan; for tests and tuning. */
int qgemm_run_gate_up_silu_ex(int M, int d, int K, int group, int prec, int has_zp, const void *A,
                              const void *w_packed, const void *scales, const void *zeros, void *out,
                              void *workspace, size_t workspace_bytes, void *stream, int force_path,
                              int force_nsplit);

/* Bytes of the workspace that qgemm_run_noalloc owns on each GPU. */
#define QG_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * qgemm_run for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It
 * allocates nothing (no hipMalloc, hipFree or allocating library routine)
 * and takes no workspace: it uses a library-owned array of
 * QG_NOALLOC_SCRATCH_BYTES on the current device, which is placed when the
 * library's code is loaded on that device and held until the process ends.
 * Arguments, results and the plan are those of qgemm_run (same kernels, same
 * bits). Returns QG_EWORKSPACE when the problem needs more than
 * QG_NOALLOC_SCRATCH_BYTES (qgemm_workspace_bytes), before anything is
 * enqueued; QG_EHIP when the array's address cannot be had.
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents (no call depends on them). Calls that may overlap on
 * one GPU (concurrent streams, or host threads without an order between
 * them) race on the array and must not be made; calls ordered on one stream
 * are safe.
 */
int qgemm_run_noalloc(int M, int N, int K, int group, int prec, int has_zp, const void *A,
                      const void *a_scales, const void *w_packed, const void *scales,
                      const void *zeros, void *out, void *stream);

/* qgemm_run with an explicit plan (see qgemm_plan); for tests and tuning. */
int qgemm_run_ex(int M, int N, int K, int group, int prec, int has_zp, const void *A,
                 const void *a_scales, const void *w_packed, const void *scales,
                 const void *zeros, void *out, void *workspace, size_t workspace_bytes,
                 void *stream, int force_path, int force_nsplit);

/*
 * Dynamic per-group int8 quantization of float32 activations: the absmax ->
 * scale -> round -> saturate step that precedes an int8-activation product,
 * as in the per-token dynamic quantization kernel of the page
 * "quantization-and-fused-kernels" (arganzheng.life), section 四.5, here per
 * (row, group of G consecutive k) with int8 codes, the activation format of
 * the page "04 · 分组量化 GEMM 内核" (developer.aliyun.com), section 二.
 * For every row m < M and group g < K/G, in float32:
 *     a_scales[m][g] = max_{k in g} |A[m][k]| / 127, or 1 when that max is 0
 *     Aq[m][k]       = clamp(rint(A[m][k] / a_scales[m][g]), -127, 127)
 * with the division correctly rounded and rint rounding halves to even.
 *   A:        float32 [M][K] (device, read)
 *   Aq:       int8 [M][K] (device, written)
 *   a_scales: float32 [M][K/G] (device, written)
 * Its outputs are the A and a_scales of a QG_W4_A_I8 / QG_W8_A_I8 call.
 * M >= 0 (0 is a no-op), K >= 1, K % group == 0, group in {32, 128}; all three
 * pointers 16-byte aligned; non-finite inputs give unspecified codes. One
 * kernel, enqueued on `stream`; nothing is allocated.
 */
int qgemm_quantize_activations(const void *A, int M, int K, int group, void *Aq, void *a_scales,
                               void *stream);

/* Whole-matrix dequantization of packed int4 weights to bf16, for comparing
 * the fused kernels with dequantization followed by a dense bf16 GEMM (the
 * prefill alternative of the page "quantization-and-fused-kernels"
 * (arganzheng.life), section 三.2):
 *     out[k][n] = bf16(s[k/G][n] * (q[k][n] - z[k/G][n]))
 * with z = 8 without zero-points. s * (q - z) is exact in float32, so out is
 * the correctly rounded (nearest even) bf16 of the exact value.
 *   w_packed: qgemm_pack's output for K, N and prec (device, read)
 *   scales:   bf16 [K/G][N]; zeros: [K/G][N/8] packed int4 when has_zp, else
 *             NULL (device, read)
 *   out:      bf16 [K][N], row-major (device, written)
 * prec is QG_W4_A_BF16 or QG_W4_A_BF16_OF32 (int4 weights, bf16 scales);
 * group in {32, 128}, K % group == 0, K / 8 <= 65535, has_zp requires
 * N % 8 == 0; pointers 16-byte aligned. One kernel, enqueued on `stream`;
 * nothing is allocated. Errors as for qgemm_run.
 */
int qgemm_dequantize(const void *w_packed, const void *scales, const void *zeros, int K, int N, int group,
                     int prec, int has_zp, void *out, void *stream);

/*
 * Grouped (MoE) W4A16 GEMV -- grouped GEMM #1 of the fused MoE pipeline on
 * the page "quantization-and-fused-kernels" (arganzheng.life), section 六:
 * each of T tokens is routed to topk experts (slot i = t * topk + j holds
 * expert topk_ids[i]); every slot's output row is its token's activations
 * times its expert's weights,
 *     out[i][n] = sum_g s_e[g,n] * sum_{k in g} A[i / topk][k] * (q_e[k,n] - z_e[g,n]),
 * e = topk_ids[i]. Rows of one expert are gathered into blocks of `block`
 * rows by the align step (section 六.3), so each block reads its expert's
 * weights once: blocks of 1, 2, 4 or 8 rows run on the vector-ALU GEMV,
 * blocks of 16, 32 or 64 rows on the small-M MFMA path (groups of 128,
 * N % 8 == 0). qgemm_moe_default_block gives the block this library
 * recommends for a shape (1 for a single token, whose experts each get one
 * row; 16 up to 16 tokens, which puts every expert's rows in one block).
 *
 * qgemm_moe_max_tiles: row blocks the align step may produce for numel
 * routed slots (0 if the arguments are invalid); sorted_ids holds
 * max_tiles * block ints and tile_experts max_tiles ints.
 */
int qgemm_moe_max_tiles(int numel, int E, int block);
int qgemm_moe_default_block(int T, int topk, int E, int group, int N);

/*
 * Align (section 六.3), one kernel on `stream`: from topk_ids (int32
 * [numel], experts in [0, E); slots with other values are skipped) write
 * sorted_ids (the slots grouped by
 * expert, each expert's segment padded to a multiple of `block` with the
 * value numel), tile_experts (each block's expert, -1 past the padded rows)
 * and num_post_pad (one int: the padded row count); the output rows of
 * skipped slots are unspecified. The order of slots
 * within an expert follows atomic arrival, as on the page; the grouped GEMV's
 * output does not depend on it. 1 <= E <= 1024; device pointers, 16-byte
 * aligned.
 */
int qgemm_moe_align(const int *topk_ids, int numel, int E, int block, int *sorted_ids, int *tile_experts,
                    int *num_post_pad, void *stream);

/* Workspace bytes of qgemm_moe_run (float32 K-split partials; 0: none). */
size_t qgemm_moe_workspace_bytes(int T, int topk, int N, int K, int group, int prec, int E, int block);

/*
 * The grouped GEMV on the align step's metadata (device pointers, 16-byte
 * aligned; enqueued on `stream` after the align step):
 *   prec:      QG_W4_A_BF16 (bf16 out) or QG_W4_A_BF16_OF32 (float32 out)
 *   A:         bf16 [T][K] token activations
 *   w_packed:  E packed weights one after another, each qgemm_packed_bytes(K, N, prec)
 *   scales:    bf16 [E][K/G][N]; zeros: uint32 [E][K/G][N/8] when has_zp (N % 8 == 0)
 *   out:       [T * topk][N], row i for slot i
 *   workspace: qgemm_moe_workspace_bytes() bytes (float32 partials of a K-split)
 * T >= 0 (0 is a no-op), topk >= 1, group 32 or 128, K % group == 0.
 * Bitwise reproducible (each row is computed on its own, in a fixed order).
 */
int qgemm_moe_run(int T, int topk, int N, int K, int group, int prec, int has_zp, int E, int block,
                  const void *A, const void *w_packed, const void *scales, const void *zeros,
                  const int *sorted_ids, const int *tile_experts, const int *num_post_pad, void *out,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * The grouped product with SwiGLU's gate step in its epilogue: GEMM #1 of
 * the MoE pipeline and the SiLU-and-mul after it (page
 * "quantization-and-fused-kernels", sections 五.2 and 六.1), fused. Each of
 * the E experts' weights is a [K][2d] gate_up matrix (gate columns first)
 * packed with qgemm_pack_gate_up, the experts' packed buffers
 * qgemm_packed_bytes(K, 2d, prec) bytes apart; scales [E][K/G][2d] and
 * zero-points [E][K/G][2d/8] in canonical column order. Row i of out
 * [T * topk][d] is silu(y_i[:d]) * y_i[d:] with y_i the row qgemm_moe_run
 * would give for N = 2d. d % 32 == 0; every other argument, the workspace
 * (qgemm_moe_workspace_bytes with N = 2d) and the errors are those of
 * qgemm_moe_run.
 */
int qgemm_moe_run_gate_up_silu(int T, int topk, int d, int K, int group, int prec, int has_zp, int E, int block,
                               const void *A, const void *w_packed, const void *scales, const void *zeros,
                               const int *sorted_ids, const int *tile_experts, const int *num_post_pad,
                               void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * FP8 (E4M3) W8A8 -- the variant the page "quantization-and-fused-kernels"
 * (arganzheng.life) contrasts with W4A16 in section 四: weights and
 * activations both in FP8, products accumulated in float32 on the matrix
 * cores. E4M3 is the OCP "fn" variant of section 二.1 (1 sign, 4 exponent,
 * 3 mantissa bits, bias 7, largest finite 448, no infinities; 0x7F and 0xFF
 * are NaN). Codes are stored one per byte.
 */
enum {
    QG_FP8_PER_TOKEN = 0,  /* scales outside the K sum: a_scales [M], w_scales [N]   */
    QG_FP8_BLOCKWISE = 1   /* per 128-wide K block: a_scales [M][K/128] (1 x 128 of
                              the activations), w_scales [N/128][K/128] (128 x 128
                              of the weights)                                         */
};

/*
 * Dynamic FP8 quantization of bf16 activations (section 四.5): for every row
 * (block == QG_FP8_PER_TOKEN, a_scales float32 [M]) or every 128 consecutive
 * elements of a row (block == 128, a_scales float32 [M][K/128]), in float32:
 *     a_scale = max |a| / 448, or 1 when that max is 0
 *     code    = E4M3(clamp(a / a_scale, -448, 448)), rounded to nearest even
 * with the division correctly rounded (the codes are those of the correctly
 * rounded quotient; the kernel may reach them through a reciprocal and a
 * correction step). The page's optional upper bound on the scale is not
 * applied.
 *   A:  bf16 [M][K] (device, read); Aq: E4M3 codes [M][K] (device, written).
 * M >= 0 (0 is a no-op), K >= 1 with K % 8 == 0 (K % 128 == 0 for block 128);
 * all pointers 16-byte aligned. One kernel on `stream`; nothing allocated.
 */
int qgemm_fp8_quantize(const void *A, int M, int K, int block, void *Aq, void *a_scales, void *stream);

/*
 * FP8 GEMM, out (bf16 [M][N], rounded once to nearest even) from
 *   Aq: E4M3 codes [M][K]; Wq: E4M3 codes [N][K] (each output channel's K
 *   codes contiguous); float32 scales as `scaling` says:
 *   QG_FP8_PER_TOKEN (section 四.2): out[m][n] = a_scales[m] * (w_scales[n] * acc),
 *       acc = sum_k a[m][k] w[n][k] accumulated in float32;
 *   QG_FP8_BLOCKWISE (section 四.3): out[m][n] = sum_b (a_scales[m][b] *
 *       w_scales[n/128][b]) * P_b with P_b the float32 sum over K block b,
 *       promoted into a float32 accumulator once per block.
 * M >= 0 (0 is a no-op), N >= 1, K % 128 == 0; N % 128 == 0 for
 * QG_FP8_BLOCKWISE; all pointers device pointers, 16-byte aligned. One
 * kernel on `stream` (never split along K); nothing allocated; bitwise
 * reproducible.
 */
int qgemm_fp8_gemm(int M, int N, int K, int scaling, const void *Aq, const void *a_scales, const void *Wq,
                   const void *w_scales, void *out, void *stream);

/*
 * The same product with the K steps split into slices when the 128 x 128
 * output tiles alone leave compute units idle (the z-split of the page
 * "04 · 分组量化 GEMM 内核" (developer.aliyun.com), section 3.3): each slice
 * writes its scaled float32 partial to `workspace` ([nsplit][M][Np] float32,
 * Np = N rounded up to 128), and a second kernel adds the slices in the
 * fixed order z = 0..nsplit-1, then rounds once to bf16. The split count is a
 * pure function of (M, N, K) and the device's compute-unit count; results
 * are bitwise reproducible, and differ from the unsplit sum by float32
 * rounding order only.
 *   workspace: device, 16-byte aligned, at least
 *              qgemm_fp8_workspace_bytes(M, N, K, scaling) bytes (NULL when
 *              that is 0); contents on entry do not matter.
 *   force_nsplit: 0 for the automatic split, or a slice count to use (for
 *              tests and benchmarks; clamped to the K / 128 steps).
 * QG_EWORKSPACE when the split needs more workspace than given; otherwise
 * errors as qgemm_fp8_gemm. Two kernels on `stream` when split; nothing
 * allocated.
 */
size_t qgemm_fp8_workspace_bytes(int M, int N, int K, int scaling);
int qgemm_fp8_gemm_ex(int M, int N, int K, int scaling, const void *Aq, const void *a_scales, const void *Wq,
                      const void *w_scales, void *out, void *workspace, size_t workspace_bytes, int force_nsplit,
                      void *stream);

/* Measurement aid (not part of the product): a plain streaming read of
 * `bytes` bytes at `src`, the reference point for the HBM rate the GEMV path
 * reaches on the same byte count (the pages measure kernels against the
 * memory roofline: "quantization-and-fused-kernels", section 三.2 and 十).
 * Each of `blocks` workgroups reads a balanced contiguous range of 16-byte
 * pieces with 8 loads in flight per lane.
 *   src: device, 16-byte aligned; bytes: a multiple of 16, 0 < bytes < 2^31.
 *   out: device, at least 4 * blocks uint32_t, written (an XOR of the data
 *        each wave read, so the reads are not optimised away).
 *   blocks: 1 .. 65535 (2 per compute unit is a good choice).
 * QG_EINVAL for a null pointer or a size outside those limits, QG_EALIGN
 * for a misaligned pointer, QG_EHIP if the launch fails. One kernel on
 * `stream`, nothing allocated. */
int qgemm_stream_read(const void *src, size_t bytes, void *out, int blocks, void *stream);

/* Human-readable text of a status code. */
const char *qgemm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
