// Small-M integer-MFMA path for int8 activations: int8 codes with float32
// per-group scales, int4 or int8 weight codes, float32 weight scales, optional
// int4 zero-points, groups of 32 or 128, float32 output. It computes the
// blockwise sum of the page "04 · 分组量化 GEMM 内核" (developer.aliyun.com),
// section 二:
//   out[m][n] = sum_g a_scale[m][g] * s[g][n] * D[m][g][n],
//   D[m][g][n] = sum_{k in g} Aq[m][k] * (q[k][n] - z[g][n])   (exact int32)
// with each group's integer dot finished before the scales multiply it, on
// v_mfma_i32_16x16x32_i8 (exact int32 accumulation) instead of the vector
// ALU's v_dot4: the integer-matrix-instruction path that the plan for the
// dynamic int8 quantization leads to (the small-M band of the page
// "quantization-and-fused-kernels" (arganzheng.life), section 三.3, item 6).
//
// Structure, as the bf16 small-M kernel (gemm_small.hip):
//   - a workgroup (8 waves for int4 weights and M <= 48, else 4) covers one
//     64-column tile of the packed layout and a K-slice of whole 128-wide
//     chunks (the z-split of the first page, section 3.3); each wave takes a
//     contiguous share of the slice's chunks (with 4 waves it loads the next
//     chunk while it computes the current one);
//   - M is padded to MB blocks of 16 rows; rows past M read zeros through the
//     buffer's range check and are not written;
//   - a chunk is 4 k-steps of 32; a group is one step (G = 32) or four
//     (G = 128); lane (l % 16, l / 16) of a step takes k = 8 (l / 16) .. +7 of
//     row l % 16 (activations) or of column l % 16 (weights), and MFMA column
//     j of tile f is physical column 4 j + f of the 64-column tile (a lane's
//     16-byte weight load is 4 adjacent columns);
//   - int4: a word's nibbles hold k + {0,2,4,6,1,3,5,7}, so (w & 0x0F0F0F0F)
//     and ((w >> 4) & 0x0F0F0F0F) are the unsigned codes of k + {0,4,1,5} and
//     k + {2,6,3,7}; the activation bytes are permuted into the same order.
//     The MFMA then sums Aq * q, and a second MFMA of the activations with an
//     all-ones operand gives sum Aq, so D = P - z * sum Aq (z = 8 without
//     zero-points), all in int32;
//   - int8: two word-rows per step, bytes in k order, D = P;
//   - per group: acc += (a_scale * s) * float(D);
//   - the waves' results are added in wave order through LDS, then written
//     to the output (nsplit == 1) or to float32 partials that a second kernel
//     adds in the order z = 0..nsplit-1.
#include "common.h"

namespace qg {

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_i;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_i;
typedef __attribute__((ext_vector_type(4))) int i32x4_i;
typedef __attribute__((ext_vector_type(4))) float f32x4_i;

constexpr int kBufWord3i = 0x00020000;
constexpr int kStreamPolicyI = 2;   // non-temporal
constexpr int kDeadI = (int)0x80000000u;

__device__ __forceinline__ long as_long(uint32_t lo, uint32_t hi) {
  return (long)(((unsigned long)hi << 32) | lo);
}

}  // namespace

// Waves per workgroup: 8 for int4 weights (4 loads per chunk; the second
// wave on each SIMD hides a chunk's latency, and twice the waves share the
// per-group float32 work: K = 2048, N = 11264, M = 32, 12.4 -> 11.4 us), 4
// for int8 weights, which load the next chunk while computing the current
// one (8 loads per chunk: 4 waves with that prefetch 12.4 us, 8 without it
// 13.3 us). Two chunk register sets do not fit in 256 VGPRs, the limit with
// two waves per SIMD, and neither does one with 4 row blocks (M > 48), which
// also keep 4 waves.
template <int WF, int MB>
constexpr int i8_waves() { return WF == W4 && MB <= 3 ? 8 : 4; }

template <int WF, int G, int MB, bool ZP>
__global__ __launch_bounds__((i8_waves<WF, MB>() * kWave)) void gemm_small_i8_kernel(SmallI8Args a) {
  constexpr int kWavesI = i8_waves<WF, MB>();
  extern __shared__ __align__(16) unsigned char s_red[];   // [waves - 1][MB * 16][64] float32
  constexpr int KPW = WF == W4 ? 8 : 4;          // k per packed word
  constexpr int RPC = 128 / KPW;                 // word-rows per chunk
  constexpr int SPG = G / 32;                    // k-steps per group
  static_assert(G == 32 || G == 128, "groups of 32 or 128");
  static_assert(!(ZP && WF == W8), "zero-points go with int4 weights");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int tile = blockIdx.x;
  const int z = blockIdx.y;
  const int R = a.K / KPW;
  const int nchunks = a.K / 128;

  int cb, ccount, wc0, wcc;
  split_range(nchunks, a.nsplit, z, cb, ccount);
  split_range(ccount, kWavesI, wave, wc0, wcc);

  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.W + (size_t)tile * R * kTileCols), (short)0, R * kTileCols * 4, kBufWord3i);
  const int w_voff = (lk * (WF == W4 ? 1 : 2) * kTileCols + 4 * li) * 4;   // the lane's word-row in a step
  const int ncol = tile * kTileCols + 4 * li;                               // the lane's first column
  const int scol = ncol + 3 < a.N ? ncol : 0;   // N % 4 == 0: a lane's 4 columns are all in or all out
  const bool col_ok = ncol < a.N;
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.S, (short)0, (a.K / G) * a.N * 4, kBufWord3i);
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.Z, (short)0, ZP ? (a.K / G) * (a.N >> 3) * 4 : 0, kBufWord3i);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.A, (short)0, a.M * a.K, kBufWord3i);
  const __amdgpu_buffer_rsrc_t q_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.a_scale, (short)0, a.M * (a.K / G) * 4, kBufWord3i);
  // the lane's activation row of fragment fm (rows past M: out-of-range
  // offset, zeros), and the rows 16 fm + 4 lk + r of its results
  int a_off[MB], q_row[MB][4];
#pragma unroll
  for (int fm = 0; fm < MB; ++fm) {
    const int row = 16 * fm + li;
    a_off[fm] = row < a.M ? row * a.K + 8 * lk : kDeadI;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 16 * fm + 4 * lk + r;
      q_row[fm][r] = rr < a.M ? rr * (a.K / G) * 4 : kDeadI;
    }
  }

  // One chunk's loads; a chunk past the wave's range gets out-of-range
  // offsets (zero results, no memory access) so issue stays straight-line.
  constexpr int NW = WF == W4 ? 4 : 8;      // 16-byte weight loads per chunk
  constexpr int GPC = 128 / G;              // groups per chunk
  struct ChunkLoads {
    u32x4_i w[NW];
    u32x2_i af[MB][4];
    u32x4_i sv[GPC];
    u32x4_i asc[MB][4];   // [fm][r]: the chunk's GPC activation scales of row 16 fm + 4 lk + r
    uint32_t zw[GPC];
  };
  auto issue = [&](int ci, ChunkLoads &L) {   // ci: the wave's chunk index
    const int dead = ci < wcc ? 0 : kDeadI;
    const int c = cb + wc0 + (ci < wcc ? ci : 0);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      // W4: step j, word-row 4 j + lk; W8: step j / 2, word-rows 8 (j / 2) + 2 lk + (j % 2)
      const int rowoff = WF == W4 ? 4 * j : 8 * (j >> 1) + (j & 1);
      L.w[j] = __builtin_bit_cast(u32x4_i, __builtin_amdgcn_raw_buffer_load_b128(
                                               w_rsrc, w_voff | dead, (c * RPC + rowoff) * kTileCols * 4,
                                               kStreamPolicyI));
    }
#pragma unroll
    for (int fm = 0; fm < MB; ++fm)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        L.af[fm][s] = __builtin_bit_cast(u32x2_i, __builtin_amdgcn_raw_buffer_load_b64(
                                                      a_rsrc, a_off[fm] | dead, c * 128 + 32 * s, 0));
    // a row's GPC scales of the chunk are contiguous: one load (16 bytes,
    // aligned since K / G is a multiple of 4, for G = 32; 4 bytes for G = 128)
#pragma unroll
    for (int fm = 0; fm < MB; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (GPC == 4)
          L.asc[fm][r] = __builtin_bit_cast(u32x4_i, __builtin_amdgcn_raw_buffer_load_b128(
                                                         q_rsrc, q_row[fm][r] | dead, c * GPC * 4, 0));
        else
          L.asc[fm][r][0] = __builtin_amdgcn_raw_buffer_load_b32(q_rsrc, q_row[fm][r] | dead, c * 4, 0);
      }
#pragma unroll
    for (int gi = 0; gi < GPC; ++gi) {
      const int g = c * GPC + gi;
      L.sv[gi] = __builtin_bit_cast(u32x4_i, __builtin_amdgcn_raw_buffer_load_b128(
                                                 s_rsrc, (scol * 4) | dead, g * a.N * 4, 0));
      L.zw[gi] = 0x88888888u;
      if constexpr (ZP)
        L.zw[gi] = __builtin_amdgcn_raw_buffer_load_b32(z_rsrc, ((scol >> 3) * 4) | dead, g * (a.N >> 3) * 4, 0) >>
                   (4 * (scol & 7));
    }
  };

  f32x4_i acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_i){0.f, 0.f, 0.f, 0.f};
  const long ones = as_long(0x01010101u, 0x01010101u);
  const i32x4_i zero4 = {0, 0, 0, 0};

  auto compute = [&](const ChunkLoads &L) {
    i32x4_i P[MB][4], SA[MB];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int gi = s / SPG;
      const bool first = s % SPG == 0;
      long bfr[4];
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        if constexpr (WF == W4) {
          const uint32_t w = L.w[s][fn];
          bfr[fn] = as_long(w & 0x0F0F0F0Fu, (w >> 4) & 0x0F0F0F0Fu);
        } else {
          bfr[fn] = as_long(L.w[2 * s][fn], L.w[2 * s + 1][fn]);
        }
      }
#pragma unroll
      for (int fm = 0; fm < MB; ++fm) {
        const u32x2_i c = L.af[fm][s];
        long afr;
        if constexpr (WF == W4)   // bytes k + {0,4,1,5}, k + {2,6,3,7}: the order of the weight bytes
          afr = as_long(__builtin_amdgcn_perm(c[1], c[0], 0x05010400u), __builtin_amdgcn_perm(c[1], c[0], 0x07030602u));
        else
          afr = as_long(c[0], c[1]);
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
          P[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x32_i8(afr, bfr[fn], first ? zero4 : P[fm][fn], 0, 0, 0);
        if constexpr (WF == W4) SA[fm] = __builtin_amdgcn_mfma_i32_16x16x32_i8(afr, ones, first ? zero4 : SA[fm], 0, 0, 0);
      }
      if (s % SPG == SPG - 1) {   // the group ends: D = P - z * sum Aq, then the scales
        float sc[4];
        int zc[4];
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          sc[fn] = col_ok ? __uint_as_float(L.sv[gi][fn]) : 0.f;
          zc[fn] = WF == W4 ? (int)((L.zw[gi] >> (4 * fn)) & 0xFu) : 0;
        }
#pragma unroll
        for (int fm = 0; fm < MB; ++fm)
#pragma unroll
          for (int fn = 0; fn < 4; ++fn)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int d = WF == W4 ? P[fm][fn][r] - zc[fn] * SA[fm][r] : P[fm][fn][r];
              acc[fm][fn][r] = __builtin_fmaf(__uint_as_float(L.asc[fm][r][gi]) * sc[fn], (float)d, acc[fm][fn][r]);
            }
      }
    }
  };

  if constexpr (kWavesI == 4) {
    ChunkLoads cur, nxt;
    issue(0, cur);
    for (int ci = 0; ci < wcc; ++ci) {
      issue(ci + 1, nxt);
      compute(cur);
      cur = nxt;
    }
  } else {
    ChunkLoads cur;
    for (int ci = 0; ci < wcc; ++ci) {
      issue(ci, cur);
      compute(cur);
    }
  }

  // ---- the waves' results, added in wave order: waves 1.. hand theirs
  // to wave 0 through LDS (element (16 fm + 4 lk + r, 4 li + fn) of wave w at
  // s_red[(((w - 1) * MB + fm) * 16 + 4 lk + r) * 64 + 4 li + fn]) ----
  float *red = (float *)s_red;
  if (wave > 0) {
#pragma unroll
    for (int fm = 0; fm < MB; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(f32x4_i *)&red[(((wave - 1) * MB + fm) * 16 + 4 * lk + r) * 64 + 4 * li] =
            (f32x4_i){acc[fm][0][r], acc[fm][1][r], acc[fm][2][r], acc[fm][3][r]};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if (wave > 0) return;

#pragma unroll
  for (int fm = 0; fm < MB; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * fm + 4 * lk + r;
      f32x4_i v = (f32x4_i){acc[fm][0][r], acc[fm][1][r], acc[fm][2][r], acc[fm][3][r]};
#pragma unroll
      for (int w = 1; w < kWavesI; ++w)
        v += *(const f32x4_i *)&red[(((w - 1) * MB + fm) * 16 + 4 * lk + r) * 64 + 4 * li];
      if (row >= a.M) continue;
      if (a.nsplit > 1)
        *(f32x4_i *)&a.partial[((size_t)z * a.M + row) * a.Np + ncol] = v;
      else if (col_ok)
        *(f32x4_i *)&a.out[(size_t)row * a.N + ncol] = v;
    }
}

template <int WF, int G, int MB, bool ZP>
static hipError_t go_i8(const SmallI8Args &a, dim3 grid, hipStream_t st) {
  constexpr int kWavesI = i8_waves<WF, MB>();
  const size_t lds = (size_t)(kWavesI - 1) * MB * 16 * 64 * 4;
  gemm_small_i8_kernel<WF, G, MB, ZP><<<grid, kWavesI * kWave, lds, st>>>(a);
  return hipGetLastError();
}

template <int WF, int G, bool ZP>
static hipError_t go_i8_mb(int mb, const SmallI8Args &a, dim3 grid, hipStream_t st) {
  switch (mb) {
    case 1: return go_i8<WF, G, 1, ZP>(a, grid, st);
    case 2: return go_i8<WF, G, 2, ZP>(a, grid, st);
    case 3: return go_i8<WF, G, 3, ZP>(a, grid, st);
    case 4: return go_i8<WF, G, 4, ZP>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

// The dispatcher sends only int8 activations, G in {32, 128}, K % 128 == 0,
// N % 4 == 0, M <= 64 (mb = ceil(M / 16) blocks of 16 rows) here.
hipError_t launch_gemm_small_i8(int wfmt, bool zp, int mb, const SmallI8Args &a, dim3 grid, hipStream_t st) {
  if (a.N % 4 != 0 || a.K % 128 != 0 || (a.G != 32 && a.G != 128) || mb < 1 || mb > 4 || a.M > 16 * mb ||
      (zp && wfmt != W4))
    return hipErrorInvalidValue;
  if (wfmt == W4) {
    if (a.G == 32) return zp ? go_i8_mb<W4, 32, true>(mb, a, grid, st) : go_i8_mb<W4, 32, false>(mb, a, grid, st);
    return zp ? go_i8_mb<W4, 128, true>(mb, a, grid, st) : go_i8_mb<W4, 128, false>(mb, a, grid, st);
  }
  return a.G == 32 ? go_i8_mb<W8, 32, false>(mb, a, grid, st) : go_i8_mb<W8, 128, false>(mb, a, grid, st);
}

}  // namespace qg
