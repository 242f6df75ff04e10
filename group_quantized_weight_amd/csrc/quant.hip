// Dynamic per-group int8 quantization of float32 activations, the step
// ahead of the int8-activation product: the absmax -> scale -> round -> cast
// kernel of the page "quantization-and-fused-kernels" (arganzheng.life),
// section 四.5, here with int8 codes and one scale per (row, group of G) as
// the blockwise product of the page "04 · 分组量化 GEMM 内核"
// (developer.aliyun.com), section 二, consumes them. In float32:
//   a_scale[m][g] = max_{k in g} |a[m][k]| / 127   (1 for a group of zeros)
//   Aq[m][k]      = clamp(rint(a[m][k] / a_scale[m][g]), -127, 127)
// with rint rounding halves to even and the division correctly rounded, so
// every code is decided exactly as the definition decides it.
//
// Mapping: a thread takes 4 consecutive activations (one 16-byte load, one
// 4-byte store of codes); the G / 4 threads of a group are adjacent lanes
// and combine their maxima with lane exchanges (max is exact in any order).
#include "common.h"

namespace qg {

template <int G>
__global__ __launch_bounds__(256) void quant_kernel(const float *__restrict__ A, int8_t *__restrict__ Aq,
                                                   float *__restrict__ a_scale, size_t total) {
  constexpr int L = G / 4;   // lanes per group
  const size_t e = 4 * ((size_t)blockIdx.x * blockDim.x + threadIdx.x);
  // total % G == 0, so a group's lanes are all in range or all out
  if (e >= total) return;
  const float4 v = *(const float4 *)(A + e);
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int d = 1; d < L; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float sc = amax > 0.f ? amax / 127.f : 1.f;
  const float x[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float q = fminf(fmaxf(__builtin_rintf(x[j] / sc), -127.f), 127.f);
    packed |= ((uint32_t)(uint8_t)(int8_t)(int)q) << (8 * j);
  }
  *(uint32_t *)(Aq + e) = packed;
  if ((threadIdx.x & (L - 1)) == 0) a_scale[e / G] = sc;
}

hipError_t launch_quant(const float *A, int8_t *Aq, float *a_scale, int M, int K, int G, hipStream_t st) {
  const size_t total = (size_t)M * K;
  if (total == 0) return hipSuccess;
  const size_t threads = total / 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (G == 32)
    quant_kernel<32><<<grid, 256, 0, st>>>(A, Aq, a_scale, total);
  else if (G == 128)
    quant_kernel<128><<<grid, 256, 0, st>>>(A, Aq, a_scale, total);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qg
