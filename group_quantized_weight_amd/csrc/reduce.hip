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
__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ part, void *__restrict__ out,
                                                     int M, int N, int Np, int nsplit) {
  // thread: 8 adjacent columns of one row (within the partials' padded row
  // of Np % 8 == 0 columns); the slices' partials are loaded 4 slices at a
  // time (all loads issued before the adds) and added in z order
  const int n = 8 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (n >= N) return;
  const size_t zstride = (size_t)M * Np;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const float *p = part + (size_t)m * Np + n;
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
    for (int z0 = 0; z0 < nsplit; z0 += 4) {
      float4 v[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          v[u][h] = z0 + u < nsplit ? *(const float4 *)(p + (size_t)(z0 + u) * zstride + 4 * h)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (z0 + u < nsplit) {
          s0.x += v[u][0].x; s0.y += v[u][0].y; s0.z += v[u][0].z; s0.w += v[u][0].w;
          s1.x += v[u][1].x; s1.y += v[u][1].y; s1.z += v[u][1].z; s1.w += v[u][1].w;
        }
    }
    const float r[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const size_t o = (size_t)m * N + n;
    if constexpr (OF == O_BF16) {
      if (n + 8 <= N && (o & 7) == 0) {   // 16-byte aligned: one store
        uint32_t w[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = (uint32_t)to_bf16(r[2 * c]) | ((uint32_t)to_bf16(r[2 * c + 1]) << 16);
        *(uint4 *)((uint16_t *)out + o) = make_uint4(w[0], w[1], w[2], w[3]);
        continue;
      }
    } else {
      if (n + 8 <= N && (o & 3) == 0) {
        *(float4 *)((float *)out + o) = s0;
        *(float4 *)((float *)out + o + 4) = s1;
        continue;
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (n + c < N) {
        if constexpr (OF == O_BF16)
          ((uint16_t *)out)[o + c] = to_bf16(r[c]);
        else
          ((float *)out)[o + c] = r[c];
      }
  }
}

// Gate-up packed product (d gate columns, d % 32 == 0): thread = 4 adjacent
// output columns j .. j + 3 of one row; their gate sums are those of packed
// columns p = 64 (j / 32) + j % 32 .. +3 and their up sums those of p + 32,
// each added over z in order; out[m][j] = silu(gate) * up, row stride d
// (SwiGLU's gate step, page "quantization-and-fused-kernels", section 五.2).
template <int OF>
__global__ __launch_bounds__(128) void reduce_gate_up_kernel(const float *__restrict__ part, void *__restrict__ out,
                                                             int M, int d, int Np, int nsplit) {
  const int j = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (j >= d) return;
  const int pg = 64 * (j / 32) + j % 32;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const float *p = part + (size_t)m * Np + pg;
    const size_t zstride = (size_t)M * Np;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < nsplit; ++z) {
      const float4 a = *(const float4 *)(p + (size_t)z * zstride);
      const float4 b = *(const float4 *)(p + (size_t)z * zstride + 32);
      g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
      u.x += b.x; u.y += b.y; u.z += b.z; u.w += b.w;
    }
    const float r[4] = {silu_f32(g.x) * u.x, silu_f32(g.y) * u.y, silu_f32(g.z) * u.z, silu_f32(g.w) * u.w};
    const size_t o = (size_t)m * d + j;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (OF == O_BF16)
        ((uint16_t *)out)[o + c] = to_bf16(r[c]);
      else
        ((float *)out)[o + c] = r[c];
    }
  }
}

hipError_t launch_reduce_gate_up(int ofmt, const float *partial, void *out, int M, int d, int Np, int nsplit,
                                 hipStream_t st) {
  dim3 grid((d + 4 * 128 - 1) / (4 * 128), M < 65535 ? M : 65535);
  if (ofmt == O_BF16)
    reduce_gate_up_kernel<O_BF16><<<grid, 128, 0, st>>>(partial, out, M, d, Np, nsplit);
  else
    reduce_gate_up_kernel<O_F32><<<grid, 128, 0, st>>>(partial, out, M, d, Np, nsplit);
  return hipGetLastError();
}

hipError_t launch_reduce(int ofmt, const float *partial, void *out, int M, int N, int Np, int nsplit,
                         hipStream_t st) {
  dim3 grid((N + 8 * 256 - 1) / (8 * 256), M < 65535 ? M : 65535);
  if (ofmt == O_BF16)
    reduce_kernel<O_BF16><<<grid, 256, 0, st>>>(partial, out, M, N, Np, nsplit);
  else
    reduce_kernel<O_F32><<<grid, 256, 0, st>>>(partial, out, M, N, Np, nsplit);
  return hipGetLastError();
}

}  // namespace qg
