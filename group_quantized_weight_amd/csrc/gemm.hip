// MFMA path of the group-quantized GEMM: bf16 activations, int4 weights,
// bf16 scales, optional int4 zero-points; for M large enough that the work
// is a dense contraction (prefill).
//
// Structure (the W4A16 main loop of the page "quantization-and-fused-kernels"
// (arganzheng.life), section 三.1: int4 tile -> unpack in registers -> matrix
// instruction in bf16 with float32 accumulation):
//   - workgroup tile 128 x 128 (4 waves, 2 x 2, each 64 x 64 = 4 x 4 MFMA
//     tiles of v_mfma_f32_16x16x32_bf16), K in chunks of 128;
//   - activations: global -> registers -> LDS (double buffered, rows padded
//     by 16 bytes against bank conflicts) -> MFMA A fragments;
//   - weights: each lane loads its packed words straight from global memory
//     (16 bytes = 4 adjacent columns x 8 k) and turns each word into four
//     bf16 pairs (128 + q) with one and-or per pair (bf16 magic number
//     0x4300, section 二.4 of the same page); the four columns of one load
//     feed the four MFMA column tiles of the wave, so MFMA column j of tile f
//     is physical column n + 4j + f;
//   - per group, the MFMA accumulates sum_k a_k (128 + q_k) on top of the
//     initial value -(128 + z) * sum_k a_k, which is sum_k a_k (q_k - z); the
//     group's scale is then applied in float32 (acc += s * P), the per-block
//     scale promotion of the same page, section 四.3. The (q - z) values are
//     exact in bf16 and the scale never rounds into a bf16 weight.
//   - with nsplit > 1, K-slices of whole chunks write float32 partial tiles
//     that a second kernel adds in the fixed order z = 0..nsplit-1 (the
//     z-split and fixed-order reduce of the page "04 · 分组量化 GEMM 内核"
//     (developer.aliyun.com), section 3.3).
#include "common.h"

namespace qg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_g;
typedef __attribute__((ext_vector_type(2))) float f32x2_g;

constexpr int kLdsRowBytes = kGemmKC * 2 + 16;              // padded A row in LDS
constexpr int kLdsABytes = kGemmBM * kLdsRowBytes;          // one A buffer

__device__ __forceinline__ float dot2_ones(uint32_t a, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_g, a),
                                         __builtin_bit_cast(bf16x2_g, 0x3F803F80u), c, false);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_g v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_g));
}

// The bf16 magic pattern 0x4300 in both halves as an opaque VGPR value, so
// that (w & mask) | magic compiles to one v_and_or_b32.
__device__ __forceinline__ uint32_t bf16_magic_pair() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(m));
  return m;
}

// One packed word (8 codes, even k low / odd k high) -> 8 bf16 values 128 + q
// in k order, as an MFMA operand.
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w, uint32_t magic) {
  u32x4_t x;
  x[0] = (w & 0x000F000Fu) | magic;
  x[1] = ((w >> 4) & 0x000F000Fu) | magic;
  x[2] = ((w >> 8) & 0x000F000Fu) | magic;
  x[3] = ((w >> 12) & 0x000F000Fu) | magic;
  return __builtin_bit_cast(bf16x8_t, x);
}

template <int OF, bool ZP, int G>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs a) {
  static_assert(G == 32 || G == 128, "group size");
  constexpr int GPC = kGemmKC / G;   // groups per chunk
  constexpr int SPG = G / 32;        // MFMA k-steps per group
  __shared__ __align__(16) unsigned char s_a[2][kLdsABytes];
  __shared__ __align__(16) float s_sum[2][GPC][kGemmBM];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lk = lane >> 4;
  const int m0 = blockIdx.y * kGemmBM;
  const int n0 = blockIdx.x * kGemmBN;
  const int nw = n0 + 64 * wn;              // first column of this wave
  const int ncol = nw + 4 * li;             // this lane's 4 columns (one per column tile)

  int cb, ccount;
  split_range(a.nchunks, a.nsplit, blockIdx.z, cb, ccount);

  // A staging role: row t/2, k half (t&1) of the chunk: 8 x 16 bytes
  const int ar = t >> 1, ah = t & 1;
  const bool a_ok = m0 + ar < a.M;
  const uint16_t *a_src = a.A + (size_t)(m0 + (a_ok ? ar : 0)) * a.K + 64 * ah;
  // B role: per k-step s, word-row 4s + lk of the chunk, columns 4 li .. +3 of
  // the wave's 64-column tile of the packed layout (tile-major: a wave load of
  // 4 consecutive rows is 1 KiB of contiguous memory)
  const int R = a.K / 8;
  const uint32_t *b_src = a.W + ((size_t)(nw / kTileCols) * R + lk) * kTileCols + 4 * li;

  u32x4_t areg[8];
  u32x4_t bcur[4], bnext[4];

  auto load_a = [&](int c) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      areg[i] = a_ok ? *(const u32x4_t *)(a_src + (size_t)c * kGemmKC + 8 * i) : (u32x4_t){0, 0, 0, 0};
  };
  auto load_b = [&](int c, u32x4_t *dst) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      dst[s] = __builtin_nontemporal_load(
          (const u32x4_t *)(b_src + (size_t)(c * (kGemmKC / 8) + 4 * s) * kTileCols));
  };
  auto stage_a = [&](int buf) {
    unsigned char *dst = &s_a[buf][ar * kLdsRowBytes + 128 * ah];
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t *)(dst + 16 * i) = areg[i];
    // activation sums per (row, group) of this chunk, fixed order
    if constexpr (G == 128) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s = dot2_ones(areg[i][j], s);
      const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), 0xB1, 0xF, 0xF, false));
      if (ah == 0) s_sum[buf][0][ar] = s + other;
    } else {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        float s = 0.f;
#pragma unroll
        for (int i = 4 * gg; i < 4 * gg + 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) s = dot2_ones(areg[i][j], s);
        s_sum[buf][2 * ah + gg][ar] = s;
      }
    }
  };

  const uint32_t magic = bf16_magic_pair();
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  if (ccount > 0) {
    load_a(cb);
    load_b(cb, bcur);
    stage_a(0);
  }
  __syncthreads();

  for (int it = 0; it < ccount; ++it) {
    const int c = cb + it;
    const int buf = it & 1;
    const bool more = it + 1 < ccount;
    if (more) {
      load_a(c + 1);
      load_b(c + 1, bnext);
    }
    const unsigned char *abuf = s_a[buf];
#pragma unroll
    for (int gi = 0; gi < GPC; ++gi) {
      const int g = c * GPC + gi;
      // scales (and zero-points) of this lane's 4 columns
      float sc[4] = {0.f, 0.f, 0.f, 0.f};
      int zp[4] = {8, 8, 8, 8};
      if (ncol < a.N) {
        const size_t si = (size_t)g * a.N + ncol;
        if ((a.N & 3) == 0) {
          const uint2 v = *(const uint2 *)(a.S + si);
          sc[0] = __uint_as_float(v.x << 16);
          sc[1] = __uint_as_float(v.x & 0xFFFF0000u);
          sc[2] = __uint_as_float(v.y << 16);
          sc[3] = __uint_as_float(v.y & 0xFFFF0000u);
        } else {
#pragma unroll
          for (int f = 0; f < 4; ++f)
            if (ncol + f < a.N) sc[f] = __uint_as_float((uint32_t)a.S[si + f] << 16);
        }
        if constexpr (ZP) {
          const uint32_t zw = a.Z[(size_t)g * (a.N >> 3) + (ncol >> 3)];
#pragma unroll
          for (int f = 0; f < 4; ++f) zp[f] = (int)((zw >> (4 * (ncol & 7) + 4 * f)) & 0xFu);
        }
      }
      // initial accumulators: -(128 + z) * sum_k a_k for the 4 rows each lane holds
      f32x4_t rs[4];
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
        rs[fm] = *(const f32x4_t *)&s_sum[buf][gi][64 * wm + 16 * fm + 4 * lk];
      f32x4_t P[4][4];
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) P[fm][fn] = rs[fm] * (float)(-(128 + zp[fn]));

#pragma unroll
      for (int ks = 0; ks < SPG; ++ks) {
        const int s = gi * SPG + ks;  // k-step within the chunk
        bf16x8_t bfr[4];
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) bfr[fn] = dequant_word(bcur[s][fn], magic);
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) {
          const bf16x8_t afr = *(const bf16x8_t *)(abuf + (64 * wm + 16 * fm + li) * kLdsRowBytes +
                                                   (32 * s + 8 * lk) * 2);
#pragma unroll
          for (int fn = 0; fn < 4; ++fn)
            P[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[fn], P[fm][fn], 0, 0, 0);
        }
      }
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[fm][fn][r] = __builtin_fmaf(sc[fn], P[fm][fn][r], acc[fm][fn][r]);
    }
    if (more) stage_a(buf ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) bcur[s] = bnext[s];
    }
  }

  // ---- epilogue ----
  const int row_base = m0 + 64 * wm + 4 * lk;
  if (a.nsplit > 1) {
    // K-slice partials; a second kernel adds them in the order z = 0..nsplit-1
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row_base + 16 * fm + r;
        if (row < a.M)
          *(f32x4_t *)&a.partial[((size_t)blockIdx.z * a.M + row) * a.Np + ncol] =
              (f32x4_t){acc[fm][0][r], acc[fm][1][r], acc[fm][2][r], acc[fm][3][r]};
      }
    return;
  }

#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row_base + 16 * fm + r;
      if (row >= a.M || ncol >= a.N) continue;
      const size_t o = (size_t)row * a.N + ncol;
      if constexpr (OF == O_BF16) {
        uint16_t *out = (uint16_t *)a.out;
        const uint32_t p01 = pack_bf16x2(acc[fm][0][r], acc[fm][1][r]);
        const uint32_t p23 = pack_bf16x2(acc[fm][2][r], acc[fm][3][r]);
        if ((a.N & 3) == 0) {
          *(uint2 *)(out + o) = make_uint2(p01, p23);
        } else {
          const uint16_t h[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23, (uint16_t)(p23 >> 16)};
#pragma unroll
          for (int f = 0; f < 4; ++f)
            if (ncol + f < a.N) out[o + f] = h[f];
        }
      } else {
        float *out = (float *)a.out;
        if ((a.N & 3) == 0) {
          *(f32x4_t *)(out + o) = (f32x4_t){acc[fm][0][r], acc[fm][1][r], acc[fm][2][r], acc[fm][3][r]};
        } else {
#pragma unroll
          for (int f = 0; f < 4; ++f)
            if (ncol + f < a.N) out[o + f] = acc[fm][f][r];
        }
      }
    }
}

template <int OF, bool ZP, int G>
static hipError_t go(const GemmArgs &a, dim3 grid, hipStream_t st) {
  gemm_kernel<OF, ZP, G><<<grid, kGemmThreads, 0, st>>>(a);
  return hipGetLastError();
}

// Only groups of 128 take this path (the dispatcher sends G = 32 to the GEMV).
hipError_t launch_gemm(int ofmt, bool zp, int G, const GemmArgs &a, dim3 grid, hipStream_t st) {
  if (G != 128) return hipErrorInvalidValue;
  if (ofmt == O_BF16) return zp ? go<O_BF16, true, 128>(a, grid, st) : go<O_BF16, false, 128>(a, grid, st);
  return zp ? go<O_F32, true, 128>(a, grid, st) : go<O_F32, false, 128>(a, grid, st);
}

}  // namespace qg
