// Internal definitions shared by the HIP kernels and the C-ABI dispatcher.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KiB LDS per compute unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

// Storage formats.
enum WFmt { W4 = 0, W8 = 1 };                // int4 packed 8 per word | int8 packed 4 per word
enum AFmt { A_F32 = 0, A_BF16 = 1, A_I8 = 2 };
enum SFmt { S_F32 = 0, S_BF16 = 1 };
enum OFmt { O_F32 = 0, O_BF16 = 1 };

constexpr int kWave = 64;
constexpr int kColAlign = 256;               // packed weights: N padded to this
constexpr int kTileCols = 64;                // packed layout: columns per tile

// GEMV path: one workgroup = 4 waves over one 64-column tile; lane l owns the
// 4 adjacent columns 4 (l % 16) .. +3 of the tile and every 4th word-row
// (l / 16) of its wave's K range. (Eight or sixteen waves per workgroup
// measured slower on MI355X, for single-row decode and the other shapes.)
__host__ __device__ constexpr int gemv_waves(int) { return 4; }

// GEMM path: one workgroup = 8 waves (two per SIMD, sharing 128 rows x 32
// columns and splitting each chunk's k-steps), tile 128 x 128, K chunks of
// 128 (one group).
constexpr int kGemmThreads = 512;
constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmKC = 128;

struct GemvArgs {
  const void *A;           // [M][K] activations
  const float *a_scale;    // [M][K/G] (int8 activations)
  const uint32_t *W;       // packed weights (layout version 2)
  const void *S;           // [K/G][N]
  const uint32_t *Z;       // [K/G][N/8] or null
  void *out;               // [M][N] (nsplit == 1)
  float *partial;          // [nsplit][M][Np] (nsplit > 1)
  int M, N, K, G, Np;
  int ngroups, nsplit;
  int gu_d;                // > 0: gate-up packed product of N = 2 gu_d columns, out [M][gu_d] = silu(g) * u
  // grouped (MoE) launches only: routed rows per row block, each block's
  // expert, the padded routed-row count, and each expert's weight stride
  const int *sorted_ids;   // [row blocks * MB] slot ids (>= M: padding)
  const int *tile_experts; // [row blocks] expert of the block, or -1
  const int *num_post_pad; // padded routed rows (device scalar)
  int topk;                // activation row = slot / topk
  size_t w_expert_words, s_expert_bytes, z_expert_words;
};

struct GemmArgs {
  const uint16_t *A;       // [M][K] bf16 (read by the pre-pass only)
  const uint32_t *W;       // packed int4, layout version 2
  const uint16_t *S;       // [K/128][N] bf16 (read by the pre-pass only)
  const uint32_t *Z;       // [K/128][N/8] or null
  void *out;               // [M][N] bf16 or float32 (nsplit == 1)
  float *partial;          // [nsplit][M][Np] (nsplit > 1)
  // written by the pre-pass into the workspace:
  uint16_t *A16;           // [M][K] fp16: a * 2^e(m), exact for |a| within 2^-14 .. 2^15 after scaling
  int *rexp;               // [M] the row's exponent e(m)
  float *S32;              // [K/128][Np] float32 scales, zero past N
  int M, N, K, Np;
  int nchunks, nsplit;     // K / 128 chunks (groups) split into nsplit slices
};

struct SmallI8Args {
  const int8_t *A;         // [M][K] int8 codes
  const float *a_scale;    // [M][K/G]
  const uint32_t *W;       // packed int4 or int8, layout version 2
  const float *S;          // [K/G][N] float32
  const uint32_t *Z;       // [K/G][N/8] or null (int4 only)
  float *out;              // [M][N] float32 (nsplit == 1)
  float *partial;          // [nsplit][M][Np] (nsplit > 1)
  int M, N, K, G, Np;
  int nsplit;              // K / 128 chunks split into nsplit slices
};

struct SmallArgs {
  const uint16_t *A;       // [M][K] bf16, M <= 64
  const uint32_t *W;       // packed int4, layout version 2
  const uint16_t *S;       // [K/128][N] bf16
  const uint32_t *Z;       // [K/128][N/8] or null
  void *out;               // [M][N] bf16 or float32 (nsplit == 1)
  float *partial;          // [nsplit][M][Np] (nsplit > 1)
  int M, N, K, Np;
  int ngroups, nsplit;     // K / 128 groups split into nsplit slices
  int gu_d;                // see GemvArgs
  // grouped (MoE) launches only (see GemvArgs)
  const int *sorted_ids, *tile_experts, *num_post_pad;
  int topk, arows;         // activation row = slot / topk, of arows rows
  size_t w_expert_words, s_expert_elems, z_expert_words;
};

// Host-side launchers (defined next to their kernels). They return the HIP
// launch status; the dispatcher has validated every argument before.
hipError_t launch_gemv(int wfmt, int afmt, int sfmt, int ofmt, bool zp, int mb, const GemvArgs &a,
                       dim3 grid, size_t lds_bytes, hipStream_t stream);
// grouped (MoE) W4A16 GEMV: rows gathered through GemvArgs::sorted_ids
hipError_t launch_gemv_grouped(int ofmt, bool zp, int mb, const GemvArgs &a, dim3 grid, size_t lds_bytes,
                               hipStream_t stream);
// grouped (MoE) small-M MFMA path: blocks of 16 mb routed rows
hipError_t launch_gemm_small_grouped(int ofmt, bool zp, int mb, const SmallArgs &a, dim3 grid, hipStream_t stream);
// routing metadata for the grouped GEMV (counting sort by expert)
hipError_t launch_moe_align(const int *topk_ids, int numel, int E, int block, int max_tiles, int *sorted_ids,
                            int *tile_experts, int *num_post_pad, hipStream_t stream);
// int8 activations (float32 scales and output); dq: the activations are
// float32 and the kernel quantizes them per (row, group) itself
hipError_t launch_gemv_i8(int wfmt, bool zp, bool dq, int mb, const GemvArgs &a, dim3 grid, size_t lds_bytes,
                          hipStream_t stream);
// pre-pass (fp16 activations, exponents, float32 scales), then the MFMA
// kernel on grid (Np / 128, ceil(M / 128), nsplit)
// wide: 128 x 256 tiles (grid.x counts 128-column tiles; nsplit 1 and
// Np % 256 == 0 required)
hipError_t launch_gemm(int ofmt, bool zp, const GemmArgs &a, dim3 grid, bool wide, hipStream_t stream);
// mb = ceil(M / 16) row blocks; grid (Np / 64, nsplit)
hipError_t launch_gemm_small(int ofmt, bool zp, int mb, const SmallArgs &a, dim3 grid, hipStream_t stream);
// gu_d > 0 (int4 only): gate-up column order for a fused gate_up product of
// N = 2 gu_d columns (see gate_up_column)
hipError_t launch_pack(int wfmt, const void *src, uint32_t *dst, int K, int N, int Np, int gu_d,
                       hipStream_t stream);
// fixed-order z-split reduce followed by the SwiGLU gate step: out[m][j]
// (j < d, row stride d) = silu(g) * u of the summed partials of packed
// columns 64 (j / 32) + j % 32 (g) and that + 32 (u)
hipError_t launch_reduce_gate_up(int ofmt, const float *partial, void *out, int M, int d, int Np, int nsplit,
                                 hipStream_t stream);
// Aq[m][k], a_scale[m][k / G] = per-group int8 quantization of A[M][K]
// (float32); G in {32, 128}, K % G == 0, A 16-byte and Aq 4-byte aligned.
hipError_t launch_quant(const float *A, int8_t *Aq, float *a_scale, int M, int K, int G, hipStream_t stream);
// FP8 (E4M3) W8A8: dynamic quantization of bf16 activations (block 0: one
// scale per row; 128: one per 128 elements) and the GEMM (scaling 0: per
// token x per channel; 1: per 128 x 128 block).
hipError_t launch_fp8_quant(const uint16_t *A, uint8_t *Aq, float *a_scale, int M, int K, int block, hipStream_t stream);
// whole-matrix int4 -> bf16 dequantization (dequant.hip)
hipError_t launch_dequant_w4(const uint32_t *W, const uint16_t *S, const uint32_t *Z, uint16_t *out, int K, int N,
                             int G, hipStream_t st);
// small-M integer MFMA path for int8 activations (gemm_small_i8.hip)
hipError_t launch_gemm_small_i8(int wfmt, bool zp, int mb, const SmallI8Args &a, dim3 grid, hipStream_t st);
// per-token FP8 GEMM in 256 x 256 tiles (fp8_big.hip), for products with at
// least `cus` such tiles and 256 K below 2^31
bool fp8_big_tiles(int M, int N, int K, int cus);
hipError_t launch_fp8_gemm_big(const uint8_t *Aq, const float *a_scale, const uint8_t *Wq, const float *w_scale,
                               uint16_t *out, int M, int N, int K, hipStream_t stream);
hipError_t launch_fp8_gemm(int scaling, const uint8_t *Aq, const float *a_scale, const uint8_t *Wq,
                           const float *w_scale, uint16_t *out, float *partial, int M, int N, int K, int nsplit,
                           int Np, int cus, hipStream_t stream);
// plain streaming read of `bytes` (a multiple of 16, below 2^31) by `blocks`
// workgroups; out[4 * block + wave] receives an XOR of the data
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *out, int blocks, hipStream_t st);
// out[m][n] = sum_{z = 0..nsplit-1} partial[z][m][n], in that order.
hipError_t launch_reduce(int ofmt, const float *partial, void *out, int M, int N, int Np, int nsplit,
                         hipStream_t stream);

// Gate-up column order of a packed fused gate_up product (d = gate columns,
// N = 2d total, d % 32 == 0): packed column n (tile t = n / 64, j = n % 64)
// holds canonical column 32t + j for j < 32 (a gate column) and d + 32t + j -
// 32 for j >= 32 (its up column); N when 32t + j % 32 >= d (no column).
__host__ __device__ inline int gate_up_column(int n, int d, int N) {
  const int t = n / kTileCols, j = n % kTileCols;
  const int c = 32 * t + (j & 31);
  if (c >= d) return N;
  return j < 32 ? c : d + c;
}

// SiLU (x * sigmoid(x)) in float32; exp(-x) overflows to inf for x below
// about -88, giving -0 (the limit).
__device__ inline float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// Balanced contiguous partition of `count` items into `parts`: part z gets
// [begin, begin + size).
__host__ __device__ inline void split_range(int count, int parts, int z, int &begin, int &size) {
  int base = count / parts, rem = count % parts;
  begin = z * base + (z < rem ? z : rem);
  size = base + (z < rem ? 1 : 0);
}

}  // namespace qg
