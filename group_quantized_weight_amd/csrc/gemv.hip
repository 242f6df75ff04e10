// GEMV path of the group-quantized GEMM: vector-ALU kernel for small M with
// bf16 or float32 activations (int8 activations have their own kernel).
//
// Mapping (one workgroup = 4 waves = one 64-column tile of the packed layout;
// blocks of 56 columns, which give N = 28672 two blocks per compute unit
// instead of 1.75 tiles, measured 10% slower at M = 1 on MI355X):
//   lane l       : columns 4 (l % 16) .. +3 of the tile and word-rows
//                  r = l / 16 (mod 4) of its wave's K range; one 16-byte load
//                  per lane per 4 rows, so each wave load reads 1 KiB of
//                  contiguous memory (weights dense, activations broadcast:
//                  the mapping of the page "04 · 分组量化 GEMM 内核"
//                  (developer.aliyun.com), section 3.2, on a 64-wide wave).
//   wave w       : groups w, w + 4, w + 8, ... of the workgroup's slice, so
//                  the 4 waves read neighbouring groups at the same time
//                  (measured 4-6% faster at M = 1 than contiguous ranges
//                  per wave).
//   blockIdx.y   : block of MB activation rows.
//   blockIdx.z   : K-slice z of nsplit balanced contiguous ranges of whole
//                  groups (the z-split of the same page, section 3.3), used
//                  only when the column tiles alone cannot fill the device;
//                  slices write float32 partials that a second kernel adds in
//                  the fixed order z = 0..nsplit-1.
//
// Per group, output element and lane the kernel forms the dot product of the
// activations with the exact integers q - z and then applies the group's
// scale, acc += s[g,n] * sum_k a_k (q_k - z) in float32 (the per-group scale
// of the teaching GEMV, arganzheng.life section 九.4). No biased sum is formed
// and no bias is removed afterwards, so a column whose codes all equal its
// zero-point gives exactly zero.
//   bf16 activations: the workgroup stages its rows' activations into LDS as
//     fp16, each row scaled by a power of two 2^e chosen from the row's
//     largest magnitude over the workgroup's K-slice (its largest scaled
//     magnitude lies in [2^14, 2^15): exact for every bf16 value down to
//     2^-14 scaled, that is 2^28 below the row's maximum). Each packed word
//     becomes four fp16 pairs q - z: the codes are placed into the mantissa
//     of 1024.0 (0x6400 | q, or 0x6400 | 16 q for the codes one nibble
//     higher; the fp16 magic number of the page "quantization-and-fused-kernels"
//     (arganzheng.life), section 二.4) and one packed fp16 add or fma per pair
//     subtracts 1024 + z (or scales by 1/16 and subtracts 64 + z), all exact.
//     v_dot2_f32_f16 multiplies two pairs (exact products) and accumulates in
//     float32; the row's result is multiplied by 2^-e at the end.
//   float32 activations: codes are converted with v_cvt_f32_ubyte (int4) and
//     z subtracted in float32, or sign-extended from their byte (int8 codes),
//     both exact; then float32 FMAs.
//
// Reduction: the 4 lanes of a column and then the waves are added in a
// fixed order (lane shuffles, then LDS), so results are reproducible.
//
// Latency hiding comes from many resident waves: each wave streams about one
// batch of loads and computes while the other waves' loads are in flight;
// single-row bf16 decode also issues its next (small) batch before computing
// the current one.
//
// Latency: each thread issues its activation loads first and its first batch
// of weight loads next, then finds the rows' largest magnitudes and writes
// the activations to LDS; since vector loads complete in order, waiting for
// the activations never waits for the weights, and the weight stream starts
// at the top of the kernel.
#include <type_traits>

#include "common.h"

namespace qg {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_v;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_v;

// Word 3 of a raw buffer resource (32-bit data format, no swizzle) and the
// cache policy for streamed weights (non-temporal).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCachePolicyStream = 2;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  f32x2_t v = {x, 0.f};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xFFFFu);
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

__device__ __forceinline__ f16x2_t h2(uint32_t x) { return __builtin_bit_cast(f16x2_t, x); }
__device__ __forceinline__ uint32_t u32h(f16x2_t x) { return __builtin_bit_cast(uint32_t, x); }

// two exact products of fp16 pairs, accumulated in float32
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(h2(a), h2(b), c, false);
}

// The fp16 magic pattern 0x6400 (1024.0) in both halves as an opaque VGPR
// value, so that (w & mask) | magic is one v_and_or_b32.
__device__ __forceinline__ uint32_t f16_magic_pair() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// Packed word (layout v2: the codes of k = 2i and 2i + 1 in bits 4i and
// 4i + 16) -> four fp16 pairs q - z, k ascending. c0 = -(1024 + z) and
// c1 = -(64 + z) in both halves.
__device__ __forceinline__ void dequant_f16(uint32_t w, uint32_t magic, f16x2_t c0, f16x2_t c1, uint32_t (&x)[4]) {
  const f16x2_t sixteenth = h2(0x2C002C00u);  // 1/16
  const uint32_t t = w >> 8;
  x[0] = u32h(h2((w & 0x000F000Fu) | magic) + c0);
  x[1] = u32h(__builtin_elementwise_fma(h2((w & 0x00F000F0u) | magic), sixteenth, c1));
  x[2] = u32h(h2((t & 0x000F000Fu) | magic) + c0);
  x[3] = u32h(__builtin_elementwise_fma(h2((t & 0x00F000F0u) | magic), sixteenth, c1));
}

// fp16 constants -(1024 + z) and -(64 + z) in both halves, for a nibble z
__device__ __forceinline__ void zp_consts(uint32_t z, f16x2_t &c0, f16x2_t &c1) {
  const uint32_t zz = z | (z << 16);
  c0 = h2(0xE400E400u | zz);
  c1 = h2(0xD400D400u | (zz << 4));
}

// bf16 magnitude bits -> the exponent e that brings the value into
// [2^14, 2^15) (141 - biased exponent; zero and subnormals get 141)
__device__ __forceinline__ int scale_exponent(uint32_t mag_bits) { return 141 - (int)(mag_bits >> 7); }

// the largest bf16 magnitude (as integer bits) among the 8 values of c0
__device__ __forceinline__ uint32_t max_mag8(const u32x4_v &c0) {
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = c0[j] & 0x7FFFu, hi = (c0[j] >> 16) & 0x7FFFu;
    r = r > lo ? r : lo;
    r = r > hi ? r : hi;
  }
  return r;
}

// 8 bf16 values -> 8 fp16 values a * 2^e (round to nearest even)
__device__ __forceinline__ u32x4_v to_f16_scaled(const u32x4_v &c0, int e) {
  u32x4_v r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2_t f = {__builtin_amdgcn_ldexpf(__uint_as_float(c0[j] << 16), e),
                 __builtin_amdgcn_ldexpf(__uint_as_float(c0[j] & 0xFFFF0000u), e)};
    r[j] = u32h(__builtin_convertvector(f, f16x2_t));
  }
  return r;
}

// Staged activations: bytes per packed word-row per activation row.
template <int WF, int AF>
struct Stage {
  static constexpr int kpw = WF == W4 ? 8 : 4;  // k per packed word
  static constexpr int bytes = AF == A_BF16 ? 2 * kpw : 4 * kpw;
};

// Global -> registers: the activations of one word-row (kpw values). The
// address is always valid (callers clamp it), so the load sits outside any
// divergent branch and the compiler need not wait for it right away.
template <int WF, int AF>
__device__ __forceinline__ void load_row(const void *A, size_t k, u32x4_v &c0, u32x4_v &c1) {
  c0 = (u32x4_v){0, 0, 0, 0};
  c1 = c0;
  if constexpr (AF == A_BF16) {
    c0 = *(const u32x4_v *)((const uint16_t *)A + k);
  } else if constexpr (AF == A_F32 && WF == W4) {
    c0 = *(const u32x4_v *)((const float *)A + k);
    c1 = *(const u32x4_v *)((const float *)A + k + 4);
  } else {
    c0 = *(const u32x4_v *)((const float *)A + k);
  }
}

__device__ __forceinline__ void mask_row(bool ok, u32x4_v &c0, u32x4_v &c1) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c0[j] = ok ? c0[j] : 0u;
    c1[j] = ok ? c1[j] : 0u;
  }
}

// Registers -> LDS in the order the dot products consume (bf16 activations:
// as fp16 scaled by 2^e).
template <int WF, int AF>
__device__ __forceinline__ void store_row(unsigned char *dst, const u32x4_v &c0, const u32x4_v &c1, int e) {
  if constexpr (AF == A_BF16) {
    *(u32x4_v *)dst = to_f16_scaled(c0, e);
  } else if constexpr (AF == A_F32 && WF == W4) {
    // byte conversions of an interleaved word give k + {0,4,1,5} (low nibbles)
    // and k + {2,6,3,7} (high nibbles)
    *(u32x4_v *)dst = (u32x4_v){c0[0], c1[0], c0[1], c1[1]};
    *(u32x4_v *)(dst + 16) = (u32x4_v){c0[2], c1[2], c0[3], c1[3]};
  } else {
    *(u32x4_v *)dst = c0;
  }
}

template <int MB>
struct BatchRows {  // weight load instructions issued together, by register budget
  static constexpr int value = MB <= 2 ? 16 : (MB == 4 ? 8 : 4);
};

template <int WF, int AF, int SF, int OF, bool ZP, int MB, int G, bool GR>
__global__ __launch_bounds__(gemv_waves(MB) * kWave)
void gemv_kernel(GemvArgs a) {
  constexpr int kGemvWaves = gemv_waves(MB);
  constexpr int kGemvThreads = kGemvWaves * kWave;
  extern __shared__ __align__(16) unsigned char lds[];
  using St = Stage<WF, AF>;
  constexpr int KPW = St::kpw;
  constexpr int AB = St::bytes;
  constexpr int RPG = G / KPW;                        // word-rows per group: 4, 8, 16 or 32
  constexpr int IPG = RPG / 4;                        // wave loads per group (4 rows each)
  constexpr int BMAX = BatchRows<MB>::value;
  // Single-row bf16 decode issues the next small batch (4 loads) before it
  // computes the current one (NB = 2 register slots); the other
  // configurations, heavier in vector ALU work per byte, issue one large
  // batch and compute it before issuing the next (NB = 1). Each measured
  // best for its cases on MI355X.
  constexpr bool kSmallBatches = MB == 1 && AF == A_BF16;
  constexpr int GPB = kSmallBatches ? (IPG >= 4 ? 1 : 4 / IPG)
                                    : (IPG >= BMAX ? 1 : (BMAX / IPG < 8 ? BMAX / IPG : 8));  // groups per batch
  constexpr int IPB = GPB * IPG;                      // wave loads per batch
  constexpr int NB = kSmallBatches ? 2 : 1;           // batch slots in registers
  constexpr int SMAX = 2;                             // activation rows staged per thread up front
  static_assert(AF == A_BF16 || AF == A_F32, "int8 activations use gemv_i8_kernel");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lk = lane >> 4, c4 = lane & 15;
  const int n0 = blockIdx.x * kTileCols;
  const int ncol = n0 + 4 * c4;                       // first of this lane's 4 columns
  // the canonical column of its scales and zero-points: the packed column,
  // or, in a gate-up packed product, the gate or up column it holds (a.N:
  // none; the lane's 4 columns lie in one half of the tile)
  const int lcol = a.gu_d > 0 ? gate_up_column(ncol, a.gu_d, a.N) : ncol;
  const bool col_ok = lcol < a.N;
  const int m0 = blockIdx.y * MB;
  const int z = blockIdx.z;
  const int R = a.K / KPW;                            // word-rows of the whole matrix

  // Grouped (MoE) row blocks: block y holds the routed rows (slots)
  // sorted_ids[m0 .. m0 + MB - 1] of one expert; their activations are the
  // token rows slot / topk, the expert's weights, scales and zero-points
  // follow one another, and row `slot` of the output is written. Blocks past
  // the padded row count, or without an expert, have nothing to do.
  const uint32_t *Wb = a.W;
  const char *Sb = (const char *)a.S;
  const uint32_t *Zb = a.Z;
  if constexpr (GR) {
    if (m0 >= *a.num_post_pad) return;
    const int e = a.tile_experts[blockIdx.y];
    if (e < 0) return;
    Wb += (size_t)e * a.w_expert_words;
    Sb += (size_t)e * a.s_expert_bytes;
    if constexpr (ZP) Zb += (size_t)e * a.z_expert_words;
  }
  // output row of block row m (valid when < M) and its activation row (a
  // grouped block reads its slot from memory at each use: the rows are
  // used at runtime indices, and a register array behind a select was
  // turned back into an indexed stack array)
  auto out_row = [&](int m) {
    if constexpr (GR)
      return a.sorted_ids[m0 + (m < MB ? m : MB - 1)];
    else
      return m0 + m;
  };
  auto act_row = [&](int m) { return GR ? out_row(m) / a.topk : m0 + m; };
  const int act_row0 = GR ? 0 : m0;                   // a valid row for lanes without one

  int gb, gcount;
  split_range(a.ngroups, a.nsplit, z, gb, gcount);
  // this wave's groups, local to the slice: j-th group wave + kGemvWaves * j
  const int wgc = gcount > wave ? (gcount - wave + kGemvWaves - 1) / kGemvWaves : 0;
  auto wave_group = [&](int j) { return wave + kGemvWaves * j; };
  const int rows = gcount * RPG;

  // [MB][rows] staged rows plus one spare slot that threads without a row
  // write to, so the staging stores need no divergent branch
  const int nstage = MB * rows;
  unsigned char *s_act = lds;                                          // [nstage + 1][AB]
  // bf16 activations: the largest magnitude (bf16 bits) of each row's slice
  uint32_t *s_max = (uint32_t *)(lds + (size_t)(nstage + 1) * AB);    // [MB]
  if constexpr (AF == A_BF16) {
    if (threadIdx.x < MB) s_max[threadIdx.x] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  // Weights, scales and zero-points are read through buffer resources: the
  // tile's base and the group's offset are wave-uniform (SGPRs) and each lane
  // adds one fixed byte offset, so issuing a load costs no vector arithmetic.
  // (A buffer load past num_records returns 0 instead of faulting.)
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(Wb + (size_t)blockIdx.x * R * kTileCols), (short)0, R * kTileCols * 4, kBufferWord3);
  const int w_voff = (lk * kTileCols + 4 * c4) * 4;

  // Scale and zero-point prefetch goes to registers with no divergent control
  // flow (a lane past column N reads a clamped, valid address and masks the
  // value at use), so issuing it never waits on the weight loads in flight.
  const bool vec_s = (a.N & 3) == 0;                // 4 scales per lane in one load
  const int scol = col_ok ? lcol : 0;
  constexpr int SB = SF == S_BF16 ? 2 : 4;          // bytes per scale
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)Sb, (short)0, a.ngroups * a.N * SB, kBufferWord3);
  const int s_voff = vec_s ? scol * SB : 0;
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)Zb, (short)0, ZP ? a.ngroups * (a.N >> 3) * 4 : 0, kBufferWord3);
  const int z_voff = (scol >> 3) * 4;
  using SRaw = typename std::conditional<SF == S_BF16, u32x2_v, u32x4_v>::type;
  u32x4_v wv[NB][IPB];
  SRaw sv[NB][GPB];
  uint32_t zv[NB][GPB];
  // Issue is straight-line: a group past the end of the wave's range uses
  // the last group's offsets, and a batch wholly past the end sets the top
  // bit of the per-lane offset, which the buffer's range check turns into a
  // zero result without a memory access (every resource here has at most
  // INT_MAX bytes). Compute skips both.
  auto issue_batch = [&](int jfirst, int slot) {  // the wave's ordinal of the batch's first group
    const int jlast = wgc > 0 ? wgc - 1 : 0;
    const int dead = (wgc == 0 || jfirst > jlast) ? (int)0x80000000u : 0;
#pragma unroll
    for (int gi = 0; gi < GPB; ++gi) {
      const int gl = wave_group(jfirst + gi < jlast ? jfirst + gi : jlast);
#pragma unroll
      for (int i = 0; i < IPG; ++i)
        wv[slot][gi * IPG + i] = __builtin_bit_cast(
            u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff | dead,
                                                           ((gb + gl) * RPG + 4 * i) * kTileCols * 4,
                                                           kCachePolicyStream));
      // without 4-aligned rows (N % 4 != 0) the scales are read one by one at
      // use; this load then reads the first element and is ignored
      const int s_soff = vec_s ? (gb + gl) * a.N * SB : 0;
      if constexpr (SF == S_BF16)
        sv[slot][gi] =
            __builtin_bit_cast(u32x2_v, __builtin_amdgcn_raw_buffer_load_b64(s_rsrc, s_voff | dead, s_soff, 0));
      else
        sv[slot][gi] =
            __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(s_rsrc, s_voff | dead, s_soff, 0));
      if constexpr (ZP)
        zv[slot][gi] = __builtin_amdgcn_raw_buffer_load_b32(z_rsrc, z_voff | dead, (gb + gl) * (a.N >> 3) * 4, 0);
    }
  };
  auto scales_of = [&](int slot, int gi, int gl, float *s) {
    if (vec_s) {
      if constexpr (SF == S_BF16) {
        s[0] = bf16_lo(sv[slot][gi][0]); s[1] = bf16_hi(sv[slot][gi][0]);
        s[2] = bf16_lo(sv[slot][gi][1]); s[3] = bf16_hi(sv[slot][gi][1]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) s[c] = __uint_as_float(sv[slot][gi][c]);
      }
    } else {  // N not a multiple of 4: one scale at a time (not prefetched)
      const size_t si = (size_t)(gb + gl) * a.N + lcol;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s[c] = 0.f;
        if (lcol + c < a.N) {
          if constexpr (SF == S_BF16)
            s[c] = __uint_as_float((uint32_t)((const uint16_t *)Sb)[si + c] << 16);
          else
            s[c] = ((const float *)Sb)[si + c];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] = col_ok ? s[c] : 0.f;
  };

  // ---- prologue: activation loads, first weight batch, activations to LDS ----
  u32x4_v st0[SMAX], st1[SMAX];
  bool st_ok[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const int idx = threadIdx.x + kGemvThreads * s;
    const int m = idx / rows, r = idx - (idx / rows) * rows;
    st_ok[s] = idx < nstage && out_row(m) < a.M;
    const size_t k = st_ok[s] ? (size_t)act_row(m) * a.K + (size_t)(gb * RPG + r) * KPW : (size_t)act_row0 * a.K;
    load_row<WF, AF>(a.A, k, st0[s], st1[s]);
  }
  // the first batch (NB - 1 batches with NB > 1); a wave without groups
  // issues dead batches and computes nothing
#pragma unroll
  for (int b = 0; b < (NB > 1 ? NB - 1 : 1); ++b) issue_batch(b * GPB, b);
#pragma unroll
  for (int s = 0; s < SMAX; ++s) mask_row(st_ok[s], st0[s], st1[s]);
  // bf16: each row's largest magnitude over the slice (LDS atomic maxima),
  // then the row's exponent; the staged rows past the register batch are
  // loaded twice (the second time from the cache)
  int rexp[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) rexp[m] = 0;
  if constexpr (AF == A_BF16) {
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int idx = threadIdx.x + kGemvThreads * s;
      if (st_ok[s]) __hip_atomic_fetch_max(&s_max[idx / rows], max_mag8(st0[s]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    for (int idx = threadIdx.x + kGemvThreads * SMAX; idx < nstage; idx += kGemvThreads) {
      const int m = idx / rows, r = idx - (idx / rows) * rows;
      if (out_row(m) >= a.M) continue;
      u32x4_v c0, c1;
      load_row<WF, AF>(a.A, (size_t)act_row(m) * a.K + (size_t)(gb * RPG + r) * KPW, c0, c1);
      __hip_atomic_fetch_max(&s_max[m], max_mag8(c0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int m = 0; m < MB; ++m) rexp[m] = scale_exponent(s_max[m]);
  }
  // a row's exponent at a runtime row index, from LDS (a select over rexp[]
  // was turned back into an indexed load of a stack array)
  auto row_exp = [&](int m) {
    if constexpr (AF == A_BF16)
      return scale_exponent(s_max[m < MB ? m : MB - 1]);
    else
      return 0;
  };
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const int idx = threadIdx.x + kGemvThreads * s;
    const int slot = idx < nstage ? idx : nstage;
    store_row<WF, AF>(s_act + (size_t)slot * AB, st0[s], st1[s], row_exp(idx / rows));
  }
  for (int idx = threadIdx.x + kGemvThreads * SMAX; idx < nstage; idx += kGemvThreads) {
    const int m = idx / rows, r = idx - (idx / rows) * rows;
    const bool ok = out_row(m) < a.M;
    u32x4_v c0, c1;
    load_row<WF, AF>(a.A, ok ? (size_t)act_row(m) * a.K + (size_t)(gb * RPG + r) * KPW : (size_t)act_row0 * a.K,
                     c0, c1);
    mask_row(ok, c0, c1);
    store_row<WF, AF>(s_act + (size_t)idx * AB, c0, c1, row_exp(m));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  // ---- main loop over this wave's groups, GPB groups per batch ----
  const uint32_t magic = f16_magic_pair();
  float acc[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = 0.f;

  // batch b sits in slot b % NB
  const int nbatch = (wgc + GPB - 1) / GPB;
  for (int b0 = 0; b0 < nbatch; b0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int gg = (b0 + u) * GPB;  // the wave's ordinal of the batch's first group
      if (gg >= wgc) break;
      if constexpr (NB > 1)
        issue_batch(gg + (NB - 1) * GPB, (u + NB - 1) % NB);  // into the slot computed last
      else if (gg > 0)
        issue_batch(gg, 0);
#pragma unroll
      for (int gi = 0; gi < GPB; ++gi) {
        if (gg + gi >= wgc) break;
        const int gl = wave_group(gg + gi);
        // the zero-point of each of the lane's 4 columns (8 without
        // zero-points for int4, 0 for int8 codes)
        uint32_t zn[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          zn[c] = WF == W8 ? 0u : 8u;
          if constexpr (ZP) zn[c] = (zv[u][gi] >> (4 * ((lcol & 7) + c))) & 0xFu;
        }
        float pf[MB][4];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) pf[m][c] = 0.f;
        f16x2_t zc0[4], zc1[4];
        if constexpr (AF == A_BF16) {
#pragma unroll
          for (int c = 0; c < 4; ++c) zp_consts(zn[c], zc0[c], zc1[c]);
        }
#pragma unroll
        for (int i = 0; i < IPG; ++i) {
          const u32x4_v wq = wv[u][gi * IPG + i];
          const int lr = gl * RPG + 4 * i + lk;  // local word-row
          const unsigned char *arow = s_act + (size_t)lr * AB;
          if constexpr (AF == A_BF16) {
            uint32_t x[4][4];
#pragma unroll
            for (int c = 0; c < 4; ++c) dequant_f16(wq[c], magic, zc0[c], zc1[c], x[c]);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
              const u32x4_v av = *(const u32x4_v *)(arow + (size_t)m * rows * AB);
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                float p = pf[m][c];
                p = dot2_f16(x[c][0], av[0], p);
                p = dot2_f16(x[c][1], av[1], p);
                p = dot2_f16(x[c][2], av[2], p);
                p = dot2_f16(x[c][3], av[3], p);
                pf[m][c] = p;
              }
            }
          } else if constexpr (AF == A_F32 && WF == W4) {
            float q[4][8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t lo = wq[c] & 0x0F0F0F0Fu, hi = (wq[c] >> 4) & 0x0F0F0F0Fu;
              const float zf = (float)zn[c];
#pragma unroll
              for (int j = 0; j < 4; ++j) {  // q - z, exact in float32
                q[c][j] = (float)((lo >> (8 * j)) & 0xFFu) - zf;
                q[c][4 + j] = (float)((hi >> (8 * j)) & 0xFFu) - zf;
              }
            }
#pragma unroll
            for (int m = 0; m < MB; ++m) {
              const u32x4_v a0 = *(const u32x4_v *)(arow + (size_t)m * rows * AB);
              const u32x4_v a1 = *(const u32x4_v *)(arow + (size_t)m * rows * AB + 16);
              const float av[8] = {__uint_as_float(a0[0]), __uint_as_float(a0[1]), __uint_as_float(a0[2]),
                                   __uint_as_float(a0[3]), __uint_as_float(a1[0]), __uint_as_float(a1[1]),
                                   __uint_as_float(a1[2]), __uint_as_float(a1[3])};
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                float p = pf[m][c];
#pragma unroll
                for (int j = 0; j < 8; ++j) p = __builtin_fmaf(q[c][j], av[j], p);
                pf[m][c] = p;
              }
            }
          } else if constexpr (AF == A_F32 && WF == W8) {
            float q[4][4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int j = 0; j < 4; ++j) q[c][j] = (float)(int8_t)(wq[c] >> (8 * j));  // the signed code
#pragma unroll
            for (int m = 0; m < MB; ++m) {
              const u32x4_v a0 = *(const u32x4_v *)(arow + (size_t)m * rows * AB);
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                float p = pf[m][c];
#pragma unroll
                for (int j = 0; j < 4; ++j) p = __builtin_fmaf(q[c][j], __uint_as_float(a0[j]), p);
                pf[m][c] = p;
              }
            }
          }
        }

        // ---- group epilogue: apply the group scale ----
        float s[4];
        scales_of(u, gi, gl, s);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[m][c] = __builtin_fmaf(s[c], pf[m][c], acc[m][c]);
      }
    }
  }
  // bf16 activations were scaled by 2^e per row: undo it (exact)
  if constexpr (AF == A_BF16) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[m][c] = __builtin_amdgcn_ldexpf(acc[m][c], -rexp[m]);
  }

  // ---- reduction: the 4 lanes of a column, then the waves (fixed order) ----
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

  if (a.gu_d > 0 && a.nsplit == 1) {
    // gate-up packed product: SwiGLU's gate step on the tile's packed
    // columns j (gate) and 32 + j (up), written to output column 32 t + j of
    // [M][gu_d] (with a K-split the partials below keep the packed columns
    // and the reduce applies it)
    for (int t = threadIdx.x; t < MB * 32; t += kGemvThreads) {
      const int m = t / 32, j = t % 32;
      const int orow = out_row(m);
      const int n = 32 * (int)blockIdx.x + j;
      if (orow >= a.M || n >= a.gu_d) continue;
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < kGemvWaves; ++w) {
        g += s_red[((size_t)w * MB + m) * kTileCols + j];
        u += s_red[((size_t)w * MB + m) * kTileCols + 32 + j];
      }
      const float v = silu_f32(g) * u;
      const size_t o = (size_t)orow * a.gu_d + n;
      if constexpr (OF == O_BF16)
        ((uint16_t *)a.out)[o] = f32_to_bf16(v);
      else
        ((float *)a.out)[o] = v;
    }
    return;
  }
  for (int t = threadIdx.x; t < MB * kTileCols; t += kGemvThreads) {
    const int m = t / kTileCols, col = t % kTileCols;
    const int orow = out_row(m);
    if (orow >= a.M) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kGemvWaves; ++w) v += s_red[((size_t)w * MB + m) * kTileCols + col];
    const int n = n0 + col;
    if (n >= a.N) continue;  // the last block may reach past column N (and Np)
    if (a.nsplit > 1) {
      a.partial[((size_t)z * a.M + orow) * a.Np + n] = v;
    } else {
      const size_t o = (size_t)orow * a.N + n;
      if constexpr (OF == O_BF16)
        ((uint16_t *)a.out)[o] = f32_to_bf16(v);
      else
        ((float *)a.out)[o] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// launcher: (wfmt, afmt, sfmt, ofmt, zp, mb, G) -> kernel instance
// ---------------------------------------------------------------------------
template <int WF, int AF, int SF, int OF, bool ZP, int MB, int G, bool GR>
static hipError_t go(const GemvArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  gemv_kernel<WF, AF, SF, OF, ZP, MB, G, GR><<<grid, gemv_waves(MB) * kWave, lds, st>>>(a);
  return hipGetLastError();
}

template <int WF, int AF, int SF, int OF, bool ZP, bool GR = false>
static hipError_t go_mb(int mb, int G, const GemvArgs &a, dim3 grid, size_t lds, hipStream_t st) {
#define QG_G(MBV)                                                       \
  return G == 32 ? go<WF, AF, SF, OF, ZP, MBV, 32, GR>(a, grid, lds, st) \
                 : go<WF, AF, SF, OF, ZP, MBV, 128, GR>(a, grid, lds, st)
  switch (mb) {
    case 1: QG_G(1);
    case 2: QG_G(2);
    case 4: QG_G(4);
    default: QG_G(8);
  }
#undef QG_G
}

hipError_t launch_gemv(int wfmt, int afmt, int sfmt, int ofmt, bool zp, int mb, const GemvArgs &a,
                       dim3 grid, size_t lds, hipStream_t st) {
  const int G = a.G;
  if (wfmt == W4 && afmt == A_BF16 && sfmt == S_BF16) {
    if (ofmt == O_BF16)
      return zp ? go_mb<W4, A_BF16, S_BF16, O_BF16, true>(mb, G, a, grid, lds, st)
                : go_mb<W4, A_BF16, S_BF16, O_BF16, false>(mb, G, a, grid, lds, st);
    return zp ? go_mb<W4, A_BF16, S_BF16, O_F32, true>(mb, G, a, grid, lds, st)
              : go_mb<W4, A_BF16, S_BF16, O_F32, false>(mb, G, a, grid, lds, st);
  }
  if (wfmt == W4 && afmt == A_F32)
    return zp ? go_mb<W4, A_F32, S_F32, O_F32, true>(mb, G, a, grid, lds, st)
              : go_mb<W4, A_F32, S_F32, O_F32, false>(mb, G, a, grid, lds, st);
  if (wfmt == W8 && afmt == A_F32)
    return go_mb<W8, A_F32, S_F32, O_F32, false>(mb, G, a, grid, lds, st);
  return hipErrorInvalidValue;
}

// Grouped (MoE) W4A16: bf16 activations and scales; bf16 or float32 output.
hipError_t launch_gemv_grouped(int ofmt, bool zp, int mb, const GemvArgs &a, dim3 grid, size_t lds,
                               hipStream_t st) {
  const int G = a.G;
  if (ofmt == O_BF16)
    return zp ? go_mb<W4, A_BF16, S_BF16, O_BF16, true, true>(mb, G, a, grid, lds, st)
              : go_mb<W4, A_BF16, S_BF16, O_BF16, false, true>(mb, G, a, grid, lds, st);
  return zp ? go_mb<W4, A_BF16, S_BF16, O_F32, true, true>(mb, G, a, grid, lds, st)
            : go_mb<W4, A_BF16, S_BF16, O_F32, false, true>(mb, G, a, grid, lds, st);
}

}  // namespace qg
