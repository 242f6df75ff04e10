// Repack of canonical weights into the kernel layout (layout version 2).
//
// Column-tile-major: the packed matrix is cut into tiles of 64 columns, and
// each tile stores its word-rows one after another (256 bytes per row), so a
// tile's whole K range is one contiguous block. A wave reading 4 consecutive
// rows of a tile reads 1 KiB of contiguous memory, both in the GEMV (lane =
// 4 adjacent columns x 1 row) and in the MFMA path (B fragments of a 64-column
// wave tile, 4 rows per 32-k step).
//
// Within a word:
//   int4: the eight codes of k = 8r..8r+7 with the even k in the low half-word
//     and the odd k in the high half-word (bits 4p..4p+3 hold
//     k = 8r + {0,2,4,6,1,3,5,7}[p]). With that order one and-or with
//     0x000F000F | magic yields a bf16 pair (k, k+1) in natural activation
//     order, and shifts by 4, 8 or 12 the next pairs. The page
//     "quantization-and-fused-kernels" (arganzheng.life), section 二.4,
//     explains why a magic-number dequant needs an interleaved nibble order
//     and a one-off repack; this is the bf16 / gfx950 form of that idea.
//   int8: the codes of k = 4r..4r+3 (byte j = k offset j).
//
// Columns n in [N, Np) are written as zero words.
//
// Gate-up order (gu_d = d > 0, N = 2d, d % 32 == 0): the canonical matrix
// holds a fused gate_up product's columns, gate columns 0..d-1 then up columns
// d..2d-1 (the layout of the page "quantization-and-fused-kernels", section
// 五.2). Packed tile t then holds gate columns 32t..32t+31 in its first 32
// columns and up columns d+32t..d+32t+31 in its last 32 (gate_up_column), so
// that one workgroup produces both inputs of its output columns 32t..32t+31.
#include "common.h"

namespace qg {

__device__ __forceinline__ size_t packed_index(int r, int n, int rows) {
  return ((size_t)(n / kTileCols) * rows + r) * kTileCols + (n % kTileCols);
}

__global__ void pack_w4_kernel(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst, int N,
                               int Np, int rows, int gu_d) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int r = blockIdx.y;
  if (n >= Np) return;
  uint32_t out = 0;
  const int c = gu_d > 0 ? gate_up_column(n, gu_d, N) : n;  // canonical column (N: none)
  if (c < N) {
    const uint32_t w = src[(size_t)r * N + c];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t code = (w >> (4 * j)) & 0xFu;
      const int p = (j & 1) ? 4 + (j >> 1) : (j >> 1);
      out |= code << (4 * p);
    }
  }
  dst[packed_index(r, n, rows)] = out;
}

__global__ void pack_w8_kernel(const int8_t *__restrict__ src, uint32_t *__restrict__ dst, int N,
                               int Np, int rows) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int r = blockIdx.y;
  if (n >= Np) return;
  uint32_t out = 0;
  if (n < N) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out |= (uint32_t)(uint8_t)src[(size_t)(4 * r + j) * N + n] << (8 * j);
  }
  dst[packed_index(r, n, rows)] = out;
}

hipError_t launch_pack(int wfmt, const void *src, uint32_t *dst, int K, int N, int Np, int gu_d,
                       hipStream_t stream) {
  const int rows = wfmt == W4 ? K / 8 : K / 4;
  dim3 block(256), grid((Np + 255) / 256, rows);
  if (wfmt == W4)
    pack_w4_kernel<<<grid, block, 0, stream>>>((const uint32_t *)src, dst, N, Np, rows, gu_d);
  else
    pack_w8_kernel<<<grid, block, 0, stream>>>((const int8_t *)src, dst, N, Np, rows);
  return hipGetLastError();
}

}  // namespace qg
