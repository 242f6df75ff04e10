// Fixed-order reduction of K-slice partials: the second kernel of a call
// whose K is split into nsplit slices of whole groups (the z-split of the
// page "04 · 分组量化 GEMM 内核" (developer.aliyun.com), section 3.3: the
// slices' float32 partial sums are added in the fixed order z = 0..nsplit-1,
// which makes the result independent of scheduling), then rounded once to
// the output type.
#include "common.h"

namespace qg {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_r;
typedef __attribute__((ext_vector_type(2))) float f32x2_r;

__device__ __forceinline__ uint16_t to_bf16(float x) {
  f32x2_r v = {x, 0.f};
  bf16x2_r r = __builtin_convertvector(v, bf16x2_r);
  return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xFFFFu);
}

template <int OF>
__global__ __launch_bounds__(128) void reduce_kernel(const float *__restrict__ part, void *__restrict__ out,
                                                     int M, int N, int Np, int nsplit) {
  // thread: 4 adjacent columns of one row; the slices' partials are loaded 8
  // at a time (all loads issued before the adds) and added in z order
  const int n = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (n >= N) return;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const float *p = part + (size_t)m * Np + n;
    const size_t zstride = (size_t)M * Np;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z0 = 0; z0 < nsplit; z0 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = z0 + u < nsplit ? *(const float4 *)(p + (size_t)(z0 + u) * zstride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < nsplit) {
          s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
        }
    }
    const float r[4] = {s.x, s.y, s.z, s.w};
    const size_t o = (size_t)m * N + n;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (n + c < N) {
        if constexpr (OF == O_BF16)
          ((uint16_t *)out)[o + c] = to_bf16(r[c]);
        else
          ((float *)out)[o + c] = r[c];
      }
  }
}

hipError_t launch_reduce(int ofmt, const float *partial, void *out, int M, int N, int Np, int nsplit,
                         hipStream_t st) {
  dim3 grid((N + 4 * 128 - 1) / (4 * 128), M < 65535 ? M : 65535);
  if (ofmt == O_BF16)
    reduce_kernel<O_BF16><<<grid, 128, 0, st>>>(partial, out, M, N, Np, nsplit);
  else
    reduce_kernel<O_F32><<<grid, 128, 0, st>>>(partial, out, M, N, Np, nsplit);
  return hipGetLastError();
}

}  // namespace qg
