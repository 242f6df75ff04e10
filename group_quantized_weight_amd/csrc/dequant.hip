// Whole-matrix dequantization of packed int4 weights to bf16, for comparing
// the fused kernels with the pages' prefill alternative: dequantize once, then
// run a dense bf16 GEMM (the switch vLLM's AWQ makes above a token count, page
// "quantization-and-fused-kernels" (arganzheng.life), section 三.2).
//
//   w_hat[k][n] = bf16(s[k/G][n] * (q[k][n] - z[k/G][n]))
//
// The product is exact in float32 (a bf16 scale, 8 significant bits, times an
// integer of magnitude at most 15), so the single round to nearest even gives
// the correctly rounded bf16 of the exact value. out is [K][N] bf16,
// row-major.
//
// A thread takes one packed word-row r and 4 adjacent columns (4 words, 16
// bytes: one load within a 64-column tile of the packed layout) and writes
// rows 8r .. 8r+7 of those columns (8 bytes per row when aligned, else one
// element at a time).
#include "common.h"

namespace qg {

namespace {
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_d;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_d;
typedef __attribute__((ext_vector_type(2))) float f32x2_d;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_d;

__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  const f32x2_d v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_d));
}
}  // namespace

template <bool ZP>
__global__ __launch_bounds__(256) void dequant_w4_kernel(const uint32_t *__restrict__ W,
                                                         const uint16_t *__restrict__ S,
                                                         const uint32_t *__restrict__ Z,
                                                         uint16_t *__restrict__ out, int K, int N, int G) {
  const int rows = K / 8;
  const int n = 4 * (blockIdx.x * blockDim.x + threadIdx.x);   // first of the thread's 4 columns
  const int r = blockIdx.y;
  if (n >= N) return;
  // the packed layout keeps each 64-column tile's word-rows contiguous; 4
  // adjacent columns never straddle a tile (64 % 4 == 0)
  const u32x4_d w = *(const u32x4_d *)(W + ((size_t)(n / kTileCols) * rows + r) * kTileCols + (n % kTileCols));
  const int g = (8 * r) / G;
  float s[4], zc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int nc = n + c < N ? n + c : n;
    s[c] = __uint_as_float((uint32_t)S[(size_t)g * N + nc] << 16);
    int z = 8;
    if constexpr (ZP) z = (int)((Z[(size_t)g * (N >> 3) + (nc >> 3)] >> (4 * (nc & 7))) & 0xFu);
    zc[c] = (float)z;
  }
  // nibble p of a word holds k = 8r + {0,2,4,6,1,3,5,7}[p]
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int p = (kk & 1) ? 4 + (kk >> 1) : (kk >> 1);
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = s[c] * ((float)((w[c] >> (4 * p)) & 0xFu) - zc[c]);
    const size_t o = (size_t)(8 * r + kk) * N + n;
    const uint32_t lo = bf16x2_bits(v[0], v[1]), hi = bf16x2_bits(v[2], v[3]);
    if (n + 4 <= N && (o & 3) == 0) {
      *(u32x2_d *)(out + o) = (u32x2_d){lo, hi};
    } else {
      const uint16_t e[4] = {(uint16_t)(lo & 0xFFFFu), (uint16_t)(lo >> 16), (uint16_t)(hi & 0xFFFFu),
                             (uint16_t)(hi >> 16)};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n + c < N) out[o + c] = e[c];
    }
  }
}

hipError_t launch_dequant_w4(const uint32_t *W, const uint16_t *S, const uint32_t *Z, uint16_t *out, int K, int N,
                             int G, hipStream_t st) {
  const dim3 block(256), grid((N + 4 * 256 - 1) / (4 * 256), K / 8);
  if (Z)
    dequant_w4_kernel<true><<<grid, block, 0, st>>>(W, S, Z, out, K, N, G);
  else
    dequant_w4_kernel<false><<<grid, block, 0, st>>>(W, S, Z, out, K, N, G);
  return hipGetLastError();
}

}  // namespace qg
