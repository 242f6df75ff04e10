// GEMV path for int8 activations: int8 codes with float32 per-group scales,
// int4 or int8 weight codes, float32 weight scales and output. It computes
// the blockwise sum of the page "04 · 分组量化 GEMM 内核"
// (developer.aliyun.com), section 二:
//   out[m][n] = sum_g a_scale[m][g] * s[g][n] * D[m][g][n],
//   D[m][g][n] = sum_{k in g} Aq[m][k] * (q[k][n] - z[g][n])   (exact int32)
// where, as that section requires, each group's integer dot is finished
// before the two scales multiply it.
//
// Mapping (one workgroup = 4 waves = one 64-column tile of the packed layout):
//   lane l      : columns 4 (l % 16) .. +3 of the tile; the 16 "group lanes"
//                 (wave, l / 16) of the workgroup take balanced contiguous
//                 ranges of whole groups of the slice, so a lane reads every
//                 word-row of each of its groups and owns the group's whole
//                 integer dot for its 4 columns: no lane exchange per group.
//                 One wave load reads 16 bytes per lane at 4 word-rows (one
//                 per group lane), each 256 contiguous bytes.
//   blockIdx.y  : block of MB activation rows; blockIdx.z: K-slice (z-split of
//                 the same page, section 3.3), float32 partials added by the
//                 reduction kernel in the fixed order z = 0..nsplit-1.
//
// Per group the lane forms P = sum_k Aq (b + q) with v_dot4_i32_i8 (b = 0:
// unsigned nibbles 0..15 for int4, signed bytes for int8) and removes the
// bias of the unsigned int4 code with the group's code sum:
//   D = P - z * sum_{k in g} Aq[m][k]   (z = 8 without zero-points, 0 for int8)
// The code sums and the activation scales of the workgroup's rows and groups
// are computed / loaded once into LDS; the 4 group lanes sharing a column and
// then the waves are added in a fixed order at the end.
//
// With DQ the activations arrive in float32 and the prologue quantizes the
// rows and groups the workgroup needs (the dynamic per-group quantization
// ahead of the integer product, in float32: scale = max|a| / 127, or 1 for a
// group of zeros; code = clamp(rint(a / scale), -127, 127), the division
// correctly rounded), so the codes never leave LDS: a lane takes 8
// consecutive k of one (row, group), and the G / 8 lanes of a group combine
// their maxima and code sums with lane exchanges.
#include "common.h"

namespace qg {

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_v;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer: 32-bit data, no swizzle
constexpr int kCachePolicyStream = 2;     // non-temporal: weights are read once
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kGroupLanes = 4 * kWaves;   // lanes sharing a column, per workgroup
constexpr int kStageChunks = 4;           // 16-byte activation chunks per thread issued up front

template <int MB>
struct LoadsPerBatch {  // weight loads issued together, by register budget
  static constexpr int value = MB <= 2 ? 16 : (MB == 4 ? 8 : 4);
};

template <int AUX>
__device__ __forceinline__ u32x4_v load_b128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}

// 16 bytes of int8 codes (global k order) -> the LDS order of the dot
// products: int4 weights hold k + {0,2,4,6,1,3,5,7} in nibbles 0..7, so the
// low nibbles of a word pair with k + {0,4,1,5} and the high nibbles with
// k + {2,6,3,7}; int8 weights keep k order.
template <int WF>
__device__ __forceinline__ u32x4_v stage_order(u32x4_v c) {
  if constexpr (WF == W4) {
    u32x4_v o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      o[2 * h] = __builtin_amdgcn_perm(c[2 * h + 1], c[2 * h], 0x05010400u);
      o[2 * h + 1] = __builtin_amdgcn_perm(c[2 * h + 1], c[2 * h], 0x07030602u);
    }
    return o;
  } else {
    return c;
  }
}

}  // namespace

// 8 codes in k order -> the LDS order of stage_order.
template <int WF>
__device__ __forceinline__ uint2 stage_order8(uint32_t lo, uint32_t hi) {
  if constexpr (WF == W4)
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
  else
    return make_uint2(lo, hi);
}

template <int WF, bool ZP, int MB, int G, bool DQ>
__global__ __launch_bounds__(kThreads) void gemv_i8_kernel(GemvArgs a) {
  constexpr int KPW = WF == W4 ? 8 : 4;   // k per packed word = staged bytes per word-row
  constexpr int RPG = G / KPW;             // word-rows per group: 4, 8, 16 or 32
  constexpr int LPB = LoadsPerBatch<MB>::value;
  constexpr bool kMulti = LPB >= RPG;      // whole groups per batch, or a group over several batches
  constexpr int QPB = kMulti ? LPB / RPG : 1;   // groups per lane per batch
  constexpr int SPG = kMulti ? 1 : RPG / LPB;   // batches per group
  constexpr int LPG = kMulti ? RPG : LPB;       // loads per group per batch
  constexpr int zdef = WF == W4 ? 8 : 0;
  extern __shared__ __align__(16) unsigned char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lk = lane >> 4, c4 = lane & 15;
  const int tile = blockIdx.x;
  const int ncol = tile * kTileCols + 4 * c4;
  const bool col_ok = ncol < a.N;
  const int m0 = blockIdx.y * MB;
  const int z = blockIdx.z;
  const int R = a.K / KPW;

  int gb, gcount;  // the slice's groups
  split_range(a.ngroups, a.nsplit, z, gb, gcount);
  int g0, gcnt;    // this lane's groups, local to the slice
  split_range(gcount, kGroupLanes, wave * 4 + lk, g0, gcnt);
  const int nit = (gcount + kGroupLanes - 1) / kGroupLanes;  // most groups of any lane
  const int row_bytes = gcount * G;                          // staged codes per activation row

  unsigned char *s_act = lds;                                       // [MB][gcount * G] codes
  float *s_asc = (float *)(lds + (size_t)MB * row_bytes);          // [MB][gcount]
  int *s_gsum = (int *)(s_asc + MB * gcount);                       // [MB][gcount]

  // ---- buffer resources: per-lane offsets fixed, group offsets uniform ----
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.W + (size_t)tile * R * kTileCols), (short)0, R * kTileCols * 4, kBufferWord3);
  const int w_vbase = (gb + g0) * RPG * kTileCols * 4 + c4 * 16;
  const bool vec_s = (a.N & 3) == 0;
  const int scol = col_ok ? ncol : 0;
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.S, (short)0, a.ngroups * a.N * 4, kBufferWord3);
  const int s_vbase = vec_s ? ((gb + g0) * a.N + scol) * 4 : 0;
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.Z, (short)0, ZP ? a.ngroups * (a.N >> 3) * 4 : 0, kBufferWord3);
  const int z_vbase = ((gb + g0) * (a.N >> 3) + (scol >> 3)) * 4;

  u32x4_v wv[QPB * LPG];
  u32x4_v sv[QPB];
  uint32_t zv[QPB];
  // Straight-line issue: a lane past its groups sets the top offset bit,
  // which the buffer range check turns into a zero result with no memory
  // access (every resource here spans at most INT_MAX bytes).
  auto issue = [&](int b) {
#pragma unroll
    for (int q = 0; q < QPB; ++q) {
      const int j = kMulti ? b * QPB + q : b / SPG;   // lane-local group
      const int r0 = kMulti ? 0 : (b % SPG) * LPB;    // its first word-row in this batch
      const int dead = j < gcnt ? 0 : (int)0x80000000u;
#pragma unroll
      for (int i = 0; i < LPG; ++i)
        wv[q * LPG + i] = load_b128<kCachePolicyStream>(w_rsrc, w_vbase | dead, (j * RPG + r0 + i) * kTileCols * 4);
      // the scale (and zero-points) once per group, in the batch that finishes it
      const int sdead = (kMulti || b % SPG == SPG - 1) ? dead : (int)0x80000000u;
      sv[q] = load_b128<0>(s_rsrc, s_vbase | sdead, vec_s ? j * a.N * 4 : 0);
      if constexpr (ZP)
        zv[q] = __builtin_amdgcn_raw_buffer_load_b32(z_rsrc, z_vbase | sdead, j * (a.N >> 3) * 4, 0);
    }
  };

  const int nasc = MB * gcount;
  if constexpr (DQ) {
    // ---- prologue: float32 activations quantized into LDS (codes, scales,
    // code sums); the first weight batch is issued first ----
    constexpr int L8 = G / 8;                       // lanes per (row, group)
    const int ntask = nasc * L8;
    issue(0);
    for (int t0 = 0; t0 < ntask; t0 += kThreads) {  // uniform trip count: the exchanges see whole groups
      const int t = t0 + threadIdx.x;
      const int mg = t / L8, sub = t - mg * L8;
      const int m = mg / gcount, g = mg - m * gcount;
      const bool ok = t < ntask && m0 + m < a.M;
      u32x4_v v0 = {0, 0, 0, 0}, v1 = v0;
      if (ok) {
        const float *src = (const float *)a.A + (size_t)(m0 + m) * a.K + (size_t)(gb + g) * G + 8 * sub;
        v0 = *(const u32x4_v *)src;
        v1 = *(const u32x4_v *)(src + 4);
      }
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = __uint_as_float(v0[j]);
        x[4 + j] = __uint_as_float(v1[j]);
      }
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
      for (int d = 1; d < L8; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
      const float sc = amax > 0.f ? amax / 127.f : 1.f;
      uint32_t w[2] = {0u, 0u};
      int csum = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = (int)fminf(fmaxf(__builtin_rintf(x[j] / sc), -127.f), 127.f);
        csum += q;
        w[j >> 2] |= ((uint32_t)(q & 0xFF)) << (8 * (j & 3));
      }
#pragma unroll
      for (int d = 1; d < L8; d <<= 1) csum += __shfl_xor(csum, d);
      if (t < ntask) {
        *(uint2 *)(s_act + (size_t)m * row_bytes + (size_t)g * G + 8 * sub) = stage_order8<WF>(w[0], w[1]);
        if (sub == 0) {
          s_asc[mg] = ok ? sc : 0.f;
          s_gsum[mg] = csum;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  } else {
  // ---- prologue: activation and scale loads, the first weight batch, LDS ----
  // Vector loads complete in order: the activations are issued before the
  // weights, so waiting for them never waits for the weight stream.
  const int nchunks = MB * row_bytes / 16;
  u32x4_v st[kStageChunks];
#pragma unroll
  for (int s = 0; s < kStageChunks; ++s) {
    const int idx = threadIdx.x + kThreads * s;
    const int m = idx / (row_bytes / 16), c = idx - m * (row_bytes / 16);
    const bool ok = idx < nchunks && m0 + m < a.M;
    const size_t off = ok ? (size_t)(m0 + m) * a.K + (size_t)gb * G + 16 * c : (size_t)m0 * a.K;
    st[s] = *(const u32x4_v *)((const int8_t *)a.A + off);
    if (!ok) st[s] = (u32x4_v){0, 0, 0, 0};
  }
  float asc0 = 0.f;
  {
    const int idx = threadIdx.x < nasc ? threadIdx.x : 0;
    const int m = idx / gcount, g = idx - m * gcount;
    const bool ok = threadIdx.x < nasc && m0 + m < a.M;
    asc0 = a.a_scale[ok ? (size_t)(m0 + m) * a.ngroups + gb + g : 0];
    asc0 = ok ? asc0 : 0.f;
  }
  issue(0);
#pragma unroll
  for (int s = 0; s < kStageChunks; ++s) {
    const int idx = threadIdx.x + kThreads * s;
    if (idx < nchunks) *(u32x4_v *)(s_act + (size_t)idx * 16) = stage_order<WF>(st[s]);
  }
  for (int idx = threadIdx.x + kThreads * kStageChunks; idx < nchunks; idx += kThreads) {
    const int m = idx / (row_bytes / 16), c = idx - m * (row_bytes / 16);
    u32x4_v v = {0, 0, 0, 0};
    if (m0 + m < a.M) v = *(const u32x4_v *)((const int8_t *)a.A + (size_t)(m0 + m) * a.K + (size_t)gb * G + 16 * c);
    *(u32x4_v *)(s_act + (size_t)idx * 16) = stage_order<WF>(v);
  }
  if (threadIdx.x < nasc) s_asc[threadIdx.x] = asc0;
  for (int idx = threadIdx.x + kThreads; idx < nasc; idx += kThreads) {
    const int m = idx / gcount, g = idx - m * gcount;
    s_asc[idx] = m0 + m < a.M ? a.a_scale[(size_t)(m0 + m) * a.ngroups + gb + g] : 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  // code sum of every (row, group): signed bytes summed exactly in int32
  for (int idx = threadIdx.x; idx < nasc; idx += kThreads) {
    const uint32_t *src = (const uint32_t *)(s_act + (size_t)idx * G);  // row m, group g: G bytes
    int sum = 0;
#pragma unroll
    for (int w = 0; w < G / 4; ++w) sum = __builtin_amdgcn_sdot4((int)src[w], 0x01010101, sum, false);
    s_gsum[idx] = sum;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  // ---- main loop: batches of LPB loads, group epilogues as groups finish ----
  float acc[MB][4];
  int pi[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[m][c] = 0.f;
      pi[m][c] = 0;
    }
  const int nbatch = (nit * RPG + LPB - 1) / LPB;
  for (int b = 0; b < nbatch; ++b) {
    if (b > 0) issue(b);
#pragma unroll
    for (int q = 0; q < QPB; ++q) {
      const int j = kMulti ? b * QPB + q : b / SPG;
      if (j >= nit) break;
      const bool live = j < gcnt;
      const int gl = live ? g0 + j : (gcount > 0 ? gcount - 1 : 0);  // slice-local group (clamped)
      const int r0 = kMulti ? 0 : (b % SPG) * LPB;
#pragma unroll
      for (int i = 0; i < LPG; ++i) {
        const u32x4_v wq = wv[q * LPG + i];
        const unsigned char *arow = s_act + (size_t)(gl * RPG + r0 + i) * KPW;
        if constexpr (WF == W4) {
          uint32_t lo[4], hi[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            lo[c] = wq[c] & 0x0F0F0F0Fu;
            hi[c] = (wq[c] >> 4) & 0x0F0F0F0Fu;
          }
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const uint2 av = *(const uint2 *)(arow + (size_t)m * row_bytes);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              int p = pi[m][c];
              p = __builtin_amdgcn_sdot4((int)lo[c], (int)av.x, p, false);
              p = __builtin_amdgcn_sdot4((int)hi[c], (int)av.y, p, false);
              pi[m][c] = p;
            }
          }
        } else {
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const uint32_t av = *(const uint32_t *)(arow + (size_t)m * row_bytes);
#pragma unroll
            for (int c = 0; c < 4; ++c) pi[m][c] = __builtin_amdgcn_sdot4((int)wq[c], (int)av, pi[m][c], false);
          }
        }
      }
      if (kMulti || b % SPG == SPG - 1) {
        // ---- group epilogue: D = P - z * codesum, acc += a_scale * s * D ----
        float s[4];
        if (vec_s) {
#pragma unroll
          for (int c = 0; c < 4; ++c) s[c] = __uint_as_float(sv[q][c]);
        } else {  // N not a multiple of 4: one scale at a time, at use
          const size_t si = (size_t)(gb + gl) * a.N + ncol;
#pragma unroll
          for (int c = 0; c < 4; ++c) s[c] = ncol + c < a.N ? ((const float *)a.S)[si + c] : 0.f;
        }
        int zc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s[c] = col_ok && live ? s[c] : 0.f;
          zc[c] = zdef;
          if constexpr (ZP) zc[c] = (int)((zv[q] >> (4 * ((ncol & 7) + c))) & 0xFu);
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float asc = s_asc[m * gcount + gl];
          const int gs = s_gsum[m * gcount + gl];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int d = pi[m][c] - zc[c] * gs;
            acc[m][c] = __builtin_fmaf(asc * s[c], (float)d, acc[m][c]);
            pi[m][c] = 0;
          }
        }
      }
    }
  }

  // ---- reduction: the 4 group lanes of a column, then the waves (fixed order) ----
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v = acc[m][c];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[m][c] = v;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  float *s_red = (float *)lds;  // [waves][MB][64], reuses the staging area
  if (lk == 0) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
      *(float4 *)(s_red + ((size_t)wave * MB + m) * kTileCols + 4 * c4) =
          make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  for (int t = threadIdx.x; t < MB * kTileCols; t += kThreads) {
    const int m = t / kTileCols, col = t % kTileCols;
    if (m0 + m >= a.M) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += s_red[((size_t)w * MB + m) * kTileCols + col];
    const int n = tile * kTileCols + col;
    if (a.nsplit > 1)
      a.partial[((size_t)z * a.M + m0 + m) * a.Np + n] = v;
    else if (n < a.N)
      ((float *)a.out)[(size_t)(m0 + m) * a.N + n] = v;
  }
}

template <int WF, bool ZP, int MB, bool DQ>
static hipError_t go_i8(int G, const GemvArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  if (G == 32)
    gemv_i8_kernel<WF, ZP, MB, 32, DQ><<<grid, kThreads, lds, st>>>(a);
  else
    gemv_i8_kernel<WF, ZP, MB, 128, DQ><<<grid, kThreads, lds, st>>>(a);
  return hipGetLastError();
}

template <int WF, bool ZP, bool DQ>
static hipError_t go_i8_mb(int mb, int G, const GemvArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  switch (mb) {
    case 1: return go_i8<WF, ZP, 1, DQ>(G, a, grid, lds, st);
    case 2: return go_i8<WF, ZP, 2, DQ>(G, a, grid, lds, st);
    case 4: return go_i8<WF, ZP, 4, DQ>(G, a, grid, lds, st);
    default: return go_i8<WF, ZP, 8, DQ>(G, a, grid, lds, st);
  }
}

template <bool DQ>
static hipError_t go_i8_fmt(int wfmt, bool zp, int mb, const GemvArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  if (wfmt == W4)
    return zp ? go_i8_mb<W4, true, DQ>(mb, a.G, a, grid, lds, st) : go_i8_mb<W4, false, DQ>(mb, a.G, a, grid, lds, st);
  if (wfmt == W8 && !zp) return go_i8_mb<W8, false, DQ>(mb, a.G, a, grid, lds, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_i8(int wfmt, bool zp, bool dq, int mb, const GemvArgs &a, dim3 grid, size_t lds,
                          hipStream_t st) {
  return dq ? go_i8_fmt<true>(wfmt, zp, mb, a, grid, lds, st) : go_i8_fmt<false>(wfmt, zp, mb, a, grid, lds, st);
}

}  // namespace qg
