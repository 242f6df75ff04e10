// A plain streaming read: the achievable HBM read rate for a byte count of
// the size the GEMV streams, measured beside it (a measurement aid, not part
// of the product's arithmetic). Each workgroup reads a contiguous, balanced
// range of 16-byte pieces with 8 non-temporal loads in flight per lane; the
// XOR of everything each wave read is stored (out[4 * block + wave]) so the
// loads are not removed.
#include "common.h"

namespace qg {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_r;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint32_t *__restrict__ src, long long pieces,
                                                          uint32_t *__restrict__ out) {
  long long begin, end;
  {
    const long long per = pieces / gridDim.x, rem = pieces % gridDim.x;
    const long long b = blockIdx.x;
    begin = b * per + (b < rem ? b : rem);
    end = begin + per + (b < rem ? 1 : 0);
  }
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, 0x7FFFFFFF, 0x00020000);
  uint32_t x = 0;
  constexpr int U = 8;
  // offsets are below 2^31 bytes (the caller checks): buffer loads with a
  // per-lane offset; pieces past the range read past it but inside the
  // buffer, or zeros past INT_MAX
  for (long long p = begin + threadIdx.x; p < end; p += 256 * U) {
    u32x4_r v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long q = p + 256 * u;
      const int off = q < end ? (int)(q * 16) : (int)(begin * 16);
      v[u] = __builtin_bit_cast(u32x4_r, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if ((threadIdx.x & 63) == 0) out[4 * blockIdx.x + (threadIdx.x >> 6)] = x;
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *out, int blocks, hipStream_t st) {
  stream_read_kernel<<<blocks, 256, 0, st>>>((const uint32_t *)src, (long long)(bytes / 16), out);
  return hipGetLastError();
}

}  // namespace qg
