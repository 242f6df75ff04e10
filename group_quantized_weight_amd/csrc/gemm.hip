// MFMA path of the group-quantized GEMM: bf16 activations, int4 weights,
// bf16 scales, optional int4 zero-points, groups of 128; for M large enough
// that the work is a dense contraction (prefill).
//
// The page "quantization-and-fused-kernels" (arganzheng.life) describes the
// W4A16 main loop (section 三.1: int4 tile -> unpack in registers -> matrix
// instruction with float32 accumulation), the fp16 magic-number dequant
// (section 二.4) and the per-block float32 promotion of a blockwise-scaled
// product (section 四.3). Here:
//
//   - The weight operand is the exact integer q - z in fp16. The word's codes
//     are placed into the low mantissa bits of 1024.0 (0x6400 | q, and
//     0x6400 | 16 q for the codes one nibble higher), and one packed fp16
//     add or fma per pair subtracts 1024 + z (or scales by 1/16 and subtracts
//     64 + z). Every step is exact, so a column whose codes equal its
//     zero-point contributes exactly zero: no biased sum is formed and no
//     bias is removed afterwards.
//   - The activation operand is fp16: a pre-pass writes a(m, k) * 2^e(m),
//     with one power of two per row chosen so that the row's largest
//     magnitude lands in [2^14, 2^15). That is exact for every bf16 value
//     whose scaled magnitude is at least 2^-14 (fp16's normal range; the
//     rest, 2^28 or more below the row's maximum, round to fp16 subnormals).
//     The epilogue multiplies by 2^-e(m), exactly. The pre-pass also widens
//     the bf16 scales to float32 in a zero-padded [K/128][Np] array.
//   - Products of fp16 a and small integers are exact in float32, so the
//     MFMA accumulates sum_k a_k (q_k - z) per group in float32; then
//     acc += s(g, n) * P in float32 (the promotion), overlapped with the next
//     group's MFMAs. The scale never rounds into an fp16 weight.
//
// Tiling: workgroup tile 128 x 128, 8 waves (two per SIMD). Waves w and w + 4
// share all 128 rows and the 32 columns 32 (w % 4) .. +31, as 4 tiles of
// v_mfma_f32_32x32x16_f16 (each dequantized weight fragment feeds 4 MFMAs);
// wave w takes k-steps 0..3 of every chunk and wave w + 4 k-steps 4..7; at
// the end each of the two hands the other two of its four row tiles through
// LDS and finishes the other two (the sum always first + second).
// The weights are the MFMA's first operand: a lane holds output row
// 32 fm + (l % 32) and, by the choice of the weight row-to-column map, the 16
// adjacent columns 32 (w % 4) + 16 (l / 32) .. +15.
// K is processed in chunks of 128 (one group). A chunk's activations (fp16,
// 32 KiB), packed weights (8 KiB), float32 scales and zero-points are copied
// by buffer loads straight into LDS (buffer_load ... lds), 2 chunks ahead,
// into a ring of 3 stages (weights and activations) and 4 stages (scales and
// zero-points: a chunk's scales are still read during the next chunk). The
// group's products go to one of two accumulator sets that alternate between
// chunks, so the promotion of a chunk is spread over the next chunk's MFMAs
// (two float32 FMAs per MFMA).
//
// With nsplit > 1, K-slices of whole chunks write float32 partial tiles that
// a second kernel adds in the fixed order z = 0..nsplit-1 (the z-split and
// fixed-order reduce of the page "04 · 分组量化 GEMM 内核"
// (developer.aliyun.com), section 3.3).
#include "common.h"

#include <type_traits>

namespace qg {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBufWord3 = 0x00020000;

// Main ring stage: [activations 128 rows x 256 B][weights 16 word-rows x 128 columns x 4 B].
constexpr int kARow = 256;
constexpr int kAOff = 0;
constexpr int kWOff = 128 * kARow;               // 32 KiB
constexpr int kStage = kWOff + 16 * 128 * 4;     // 40 KiB
constexpr int kST = 3;
// Small ring stage: one 1 KiB slot per wave, each written by one
// 16-byte-per-lane copy: [scales 128 x 4 B][zero-points 16 x 4 B][six idle
// slots] (lanes past the useful part fill the slot's tail, never read).
constexpr int kSOff = 0;
constexpr int kZOff = 1024;
constexpr int kSmall = 8192;
constexpr int kSR = 4;

// Wait until at most N of this wave's global loads (including the copies
// into LDS) are outstanding and its LDS reads are done, then the workgroup
// barrier; the memory clobber keeps the compiler from moving memory
// accesses across it. Vector memory loads complete in issue order.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_g;
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_g));
}

// fp16 pairs: h(x) reinterprets a 32-bit word.
__device__ __forceinline__ f16x2_t h2(uint32_t x) { return __builtin_bit_cast(f16x2_t, x); }
__device__ __forceinline__ uint32_t u32(f16x2_t x) { return __builtin_bit_cast(uint32_t, x); }

// Packed word (layout v2: the codes of k = 2i and 2i + 1 in bits 4i and
// 4i + 16) -> the 8 exact values q - z in fp16, k ascending, as an MFMA
// operand. c0 = -(1024 + z) and c1 = -(64 + z) in both halves.
__device__ __forceinline__ f16x8_t dequant_f16(uint32_t w, uint32_t magic, f16x2_t c0, f16x2_t c1) {
  const f16x2_t sixteenth = h2(0x2C002C00u);  // 1/16
  const uint32_t t = w >> 8;
  u32x4_t x;
  x[0] = u32(h2((w & 0x000F000Fu) | magic) + c0);
  x[1] = u32(__builtin_elementwise_fma(h2((w & 0x00F000F0u) | magic), sixteenth, c1));
  x[2] = u32(h2((t & 0x000F000Fu) | magic) + c0);
  x[3] = u32(__builtin_elementwise_fma(h2((t & 0x00F000F0u) | magic), sixteenth, c1));
  return __builtin_bit_cast(f16x8_t, x);
}

// The fp16 magic pattern 0x6400 (1024.0) in both halves as an opaque VGPR
// value, so that (w & mask) | magic is one v_and_or_b32.
__device__ __forceinline__ uint32_t f16_magic_pair() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

template <typename T>
__device__ __forceinline__ T lds_read(const unsigned char *base, int off) {
  return *(const T *)(base + off);
}

template <int OF, bool ZP>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(GemmArgs a) {
  // One LDS object for both rings: the kernel orders its copies and reads
  // itself (waits at the top of each chunk), and with separate objects the
  // compiler adds a wait for every copy in flight before each LDS read.
  __shared__ __align__(16) unsigned char s_lds[kST * kStage + kSR * kSmall];
  unsigned char *const s_ring = s_lds;
  unsigned char *const s_small = s_lds + kST * kStage;
  constexpr int FM = 4;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // 0..7
  const int cg = wave & 3;                                    // column group: 32 columns
  const int kh = wave >> 2;                                   // k-steps 4 kh .. 4 kh + 3 of each chunk
  const int j = lane & 31, h = lane >> 5;
  // Tile order. Workgroups go to the 8 dies (XCDs, each with its own L2) in
  // turn by launch order; without a K-split the launch order is remapped so
  // that each die gets a compact block of tiles (up to 4 row tiles by
  // tiles/4 columns) and its L2 serves the shared activation rows and weight
  // columns of that block.
  int tx = blockIdx.x, ty = blockIdx.y;
  {
    const int TX = gridDim.x, TY = gridDim.y, T = TX * TY;
    if (gridDim.z == 1 && T % 8 == 0) {
      const int L = blockIdx.x + TX * blockIdx.y;
      const int Lx = (L & 7) * (T >> 3) + (L >> 3);   // consecutive per die
      const int GM = TY < 4 ? TY : 4;                  // row tiles per group
      const int per = GM * TX;
      const int g = Lx / per, first = g * GM;
      const int gs = TY - first < GM ? TY - first : GM;
      const int r = Lx - g * per;
      ty = first + r % gs;
      tx = r / gs;
    }
  }
  const int m0 = ty * kGemmBM;
  const int n0 = tx * kGemmBN;

  int cb, ccount;
  split_range(a.nchunks, a.nsplit, blockIdx.z, cb, ccount);

  const int R = a.K / 8;
  // weight row j of the MFMA (lane j of each half) is column fj of the
  // group's 32: the lane's output elements are then 16 adjacent columns
  const int fj = 16 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3);
  const int cw = 32 * cg + fj;                          // within the workgroup's 128 columns

  // A copy for a chunk past the slice goes through a resource of zero size,
  // which the buffer's range check turns into zeros without a memory
  // access; such copies fill a stage no later chunk reads. Issue stays
  // straight-line and every wave issues the same number of loads per chunk.

  // Buffer resources. Activation rows past M read zeros through the range
  // check (the row is in the VGPR offset; the chunk offset in the SGPR one
  // stays inside a valid row).
  const int a_rows = a.M - m0 < kGemmBM ? a.M - m0 : kGemmBM;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.A16 + (size_t)m0 * a.K), (short)0, a_rows * a.K * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.W + (size_t)(n0 / kTileCols) * R * kTileCols), (short)0, 2 * R * kTileCols * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.S32, (short)0, a.nchunks * a.Np * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.Z, (short)0, ZP ? a.nchunks * (a.N >> 3) * 4 : 0, kBufWord3);
  const __amdgpu_buffer_rsrc_t none_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, 0, kBufWord3);

  // Activation copy c = wave + 8 tt (tt = 0..3) writes LDS bytes c KiB of the
  // tile: row r = 32 tt + 4 wave + lane / 16, physical 16-byte slot
  // lane % 16, holding logical piece (lane % 16) ^ (r % 16) of the row
  // (r % 16 does not depend on tt), so the fragment reads of 16 rows hit 16
  // different slots.
  const int ar0 = 4 * wave + (lane >> 4);
  const int a_voff0 = ar0 * (a.K * 2) + (((lane & 15) ^ (ar0 & 15)) << 4);
  const int a_vstep = 32 * a.K * 2;
  // Weight copy of wave w writes word-rows 2w, 2w + 1 of the chunk: lane ->
  // word-row 2w + lane / 32, columns 4 (lane % 32) .. +3 of the workgroup
  // (LDS row-major [word-row][128 columns]).
  const int w_voff0 = ((((lane & 31) >> 4) * R) + (lane >> 5)) * 256 + (lane & 15) * 16;

  auto copy_a = [&](int chunk, int stage, int tt, const __amdgpu_buffer_rsrc_t &rs) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(s_ring + stage * kStage + kAOff + (wave + 8 * tt) * 1024),
                                             16, a_voff0 + tt * a_vstep, chunk * 256, 0, 0);
  };
  auto copy_w = [&](int chunk, int stage, const __amdgpu_buffer_rsrc_t &rs) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(s_ring + stage * kStage + kWOff + wave * 1024), 16,
                                             w_voff0, chunk * 4096 + wave * 512, 0, 0);
  };
  // the scales (wave 0) and zero-points (wave 1, with zero-points) of a
  // chunk; the other waves issue a copy with an out-of-range offset (every
  // resource here has at most INT_MAX bytes) into a slot of their own, so
  // that every wave issues the same loads per chunk with no branch in the
  // loop (a branch here measured about 5 us slower at M = 1024)
  constexpr int kDead = (int)0x80000000u;
  const __amdgpu_buffer_rsrc_t small_rsrc = wave == 0 ? s_rsrc : z_rsrc;
  const int small_voff = wave == 0 ? n0 * 4 + lane * 16 : ((ZP && wave == 1) ? (n0 >> 3) * 4 + lane * 16 : kDead);
  const int small_cstride = wave == 0 ? a.Np * 4 : (ZP && wave == 1 ? (a.N >> 3) * 4 : 0);
  const int small_slot = wave * 1024;
  auto copy_small = [&](int chunk, int sstage, const __amdgpu_buffer_rsrc_t &rs) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(s_small + sstage * kSmall + small_slot), 16,
                                             chunk * small_cstride + small_voff, 0, 0, 0);
  };

  const uint32_t magic = f16_magic_pair();
  f16x2_t c0 = h2(0xE408E408u), c1 = h2(0xD480D480u);  // -(1024 + 8), -(64 + 8)

  f32x16_t acc[FM], P[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = P[i][e] = 0.f;

  // LDS read offsets inside a stage (the stage's base is added per chunk)
  const int s_rd = kSOff + (32 * cg + 16 * h) * 4;       // the lane's 16 scales in a small stage
  const int w_rd = kWOff + (h * 128 + cw) * 4 + kh * 4096;  // + s * 1024: word-row 2 (4 kh + s) + h
  int a_rd[4];                                           // k-step 4 kh + s, row tile 0; + fm * 32 rows
#pragma unroll
  for (int s = 0; s < 4; ++s) a_rd[s] = kAOff + j * kARow + (((2 * (4 * kh + s) + h) ^ (j & 15)) << 4);

  // The lane's 16 scales of a chunk serve 16 consecutive slots: tiles 0 and 1
  // of the chunk (its slots 8..15) and tiles 2 and 3 (the next chunk's slots
  // 0..7). Two register sets alternate between chunks; a chunk's set is read
  // at its slot 2.
  f32x4_t scA[4], scB[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) scA[u] = scB[u] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  typedef __attribute__((address_space(3))) const uint32_t lds_u32;
  typedef __attribute__((address_space(3))) const f16x8_t lds_f16x8;
  typedef __attribute__((address_space(3))) const f32x4_t lds_f32x4;

  // One chunk = 16 MFMA slots of this wave's 4 k-steps. Slots 0..7 run row
  // tiles 0 and 1 (k-step s = slot / 2; each weight word dequantized just
  // before its first use), slots 8..15 tiles 2 and 3 with the same words.
  // Each slot also promotes 4 elements (a quad of scales): slots 0..7 tiles
  // 2 and 3 of the previous chunk (their products stay in P until slot 8
  // restarts them), slots 8..15 tiles 0 and 1 of this chunk (finished at
  // slot 7). Activation fragments are read three slots ahead; the copies of
  // chunk i + 2 are issued between the MFMAs.
  auto run_chunk = [&](int i, f32x4_t(&scp)[4], f32x4_t(&scc)[4]) __attribute__((always_inline)) {
    const int sbase = (i % kST) * kStage;
    const unsigned char *sm = s_small + (i % kSR) * kSmall;
    const bool live = i + 2 < ccount;
    const __amdgpu_buffer_rsrc_t ar = live ? a_rsrc : none_rsrc, wr = live ? w_rsrc : none_rsrc,
                                 sr = live ? small_rsrc : none_rsrc;
    const int cn = cb + i + 2, stn = (i + 2) % kST;
    if constexpr (ZP) {
      const uint32_t zw = *(const uint32_t *)(sm + kZOff + (cw >> 3) * 4);
      const uint32_t z = (zw >> (4 * (cw & 7))) & 0xFu;
      const uint32_t zz = z | (z << 16);
      c0 = h2(0xE400E400u | zz);          // -(1024 + z)
      c1 = h2(0xD400D400u | (zz << 4));   // -(64 + z)
    }
    // Per-chunk base addresses, made opaque to the compiler so that the
    // constant parts (row tile, k-step, quad) stay in the LDS instructions'
    // offset fields instead of being hoisted into extra registers and added
    // at every read.
    uint32_t ab[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      ab[s] = (uint32_t)(uintptr_t)(s_ring + sbase) + a_rd[s];
      asm volatile("" : "+v"(ab[s]));
    }
    uint32_t wb = (uint32_t)(uintptr_t)(s_ring + sbase) + w_rd;
    uint32_t qm = (uint32_t)(uintptr_t)sm + s_rd;
    asm volatile("" : "+v"(wb), "+v"(qm));
    uint32_t wraw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) wraw[s] = *(lds_u32 *)(wb + s * 1024);
    auto frag = [&](int q) {
      const int half = q >> 3, s = (q & 7) >> 1, fm = 2 * half + (q & 1);
      return *(lds_f16x8 *)(ab[s] + fm * 32 * kARow);
    };
    f16x8_t af[4];
    af[0] = frag(0);
    af[1] = frag(1);
    af[2] = frag(2);

    f16x8_t wq[4];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int half = q >> 3, s = (q & 7) >> 1, fm = 2 * half + (q & 1);
      if (q + 3 < 16) af[(q + 3) & 3] = frag(q + 3);
      if (q == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) scc[u] = *(lds_f32x4 *)(qm + u * 16);
      }
      if (half == 0 && (q & 1) == 0) wq[s] = dequant_f16(wraw[s], magic, c0, c1);
      if (s == 0)
        P[fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wq[s], af[q & 3], (f32x16_t){}, 0, 0, 0);
      else
        P[fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wq[s], af[q & 3], P[fm], 0, 0, 0);
      {
        const int r = q & 7;                        // slot within the half
        const int tt = half == 0 ? 2 + (r >> 2) : (r >> 2);
        const int e0 = 4 * (r & 3);
        const f32x4_t sc = half == 0 ? scp[r & 3] : scc[r & 3];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tt][e0 + e] = __builtin_fmaf(sc[e], P[tt][e0 + e], acc[tt][e0 + e]);
      }
      // copies of chunk i + 2 (small first), spread over the MFMAs
      if (q == 1) copy_small(cn, (i + 2) % kSR, sr);
      if (q == 3 || q == 6 || q == 9 || q == 12) copy_a(cn, stn, q / 3 - 1, ar);
      if (q == 14) copy_w(cn, stn, wr);
      // keep the slots in this order (the scheduler would otherwise hoist
      // the fragment reads of many slots and run out of registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: the copies of chunks 0 and 1, each chunk's small copy first
  // (the waits count on that: at the top of chunk i at most the 5 main
  // copies of chunk i + 1 may be in flight)
  {
    const __amdgpu_buffer_rsrc_t r0a = ccount > 0 ? a_rsrc : none_rsrc, r0w = ccount > 0 ? w_rsrc : none_rsrc,
                                 r0s = ccount > 0 ? small_rsrc : none_rsrc;
    const __amdgpu_buffer_rsrc_t r1a = ccount > 1 ? a_rsrc : none_rsrc, r1w = ccount > 1 ? w_rsrc : none_rsrc,
                                 r1s = ccount > 1 ? small_rsrc : none_rsrc;
    copy_small(cb, 0, r0s);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) copy_a(cb, 0, tt, r0a);
    copy_w(cb, 0, r0w);
    copy_small(cb + 1, 1, r1s);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) copy_a(cb + 1, 1, tt, r1a);
    copy_w(cb + 1, 1, r1w);
  }
  // chunk 0 promotes the zero products of a "previous chunk" with zero scales
  int i = 0;
  for (; i + 1 < ccount; i += 2) {
    wait_then_barrier<5>();
    run_chunk(i, scB, scA);
    wait_then_barrier<5>();
    run_chunk(i + 1, scA, scB);
  }
  if (i < ccount) {
    wait_then_barrier<5>();
    run_chunk(i, scB, scA);
  }
  // the last chunk's tiles 2 and 3 (tiles 0 and 1 were promoted inside it),
  // with that chunk's scales (set A after an odd count, else set B)
  {
    const bool odd = (ccount & 1) != 0;
#pragma unroll
    for (int fm = 2; fm < FM; ++fm)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4_t sc = odd ? scA[e4] : scB[e4];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[fm][4 * e4 + e] = __builtin_fmaf(sc[e], P[fm][4 * e4 + e], acc[fm][4 * e4 + e]);
      }
  }
  // The two waves of a column group hold partial sums over complementary
  // k-steps. Each finishes two of the four row tiles: the first wave (kh 0)
  // row tiles 0 and 1, the second 2 and 3; each hands the other's two to it
  // through LDS (the ring is free now) and adds the two in the fixed order
  // first + second. The row exponents are read before the exchange, so that
  // their latency is spent on it.
  int rex[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = m0 + 32 * (2 * kh + i) + j;
    rex[i] = a.rexp[row < a.M ? row : a.M - 1];
  }
  __syncthreads();
  float *s_mine = (float *)s_lds + (size_t)(2 * cg + kh) * (2 * 16 * 64);     // what this wave hands over
  const float *s_other = (float *)s_lds + (size_t)(2 * cg + 1 - kh) * (2 * 16 * 64);
  auto put = [&](int i, const f32x16_t &x) {
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      *(f32x4_t *)(s_mine + ((i * 4 + e4) * 64 + lane) * 4) = (f32x4_t){x[4 * e4], x[4 * e4 + 1], x[4 * e4 + 2], x[4 * e4 + 3]};
  };
  auto take = [&](int i, f32x16_t &x, bool first) {  // x = first ? x + other : other + x
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const f32x4_t o = *(const f32x4_t *)(s_other + ((i * 4 + e4) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * e4 + e] = first ? x[4 * e4 + e] + o[e] : o[e] + x[4 * e4 + e];
    }
  };
  const int n16 = n0 + 32 * cg + 16 * h;
  // row m0 + 32 fm + j, columns n16 .. n16 + 15 (register indices stay
  // compile-time constants: a runtime index would put acc in memory)
  auto finish = [&](auto kh_c) __attribute__((always_inline)) {
    constexpr int KH = decltype(kh_c)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i) put(i, acc[2 * (1 - KH) + i]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) take(i, acc[2 * KH + i], KH == 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int fm = 2 * KH + i;
      const int row = m0 + 32 * fm + j;
      if (row >= a.M) continue;
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = __builtin_amdgcn_ldexpf(acc[fm][q], -rex[i]);
      if (a.nsplit > 1) {
        // K-slice partials; a second kernel adds them in the order z = 0..nsplit-1
        float *p = &a.partial[((size_t)blockIdx.z * a.M + row) * a.Np + n16];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4_t *)(p + 4 * q) = (f32x4_t){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        continue;
      }
      // N % 8 == 0: each half of the lane's 16 columns is all in or all out
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int n = n16 + 8 * half;
        if (n >= a.N) continue;
        const size_t o = (size_t)row * a.N + n;
        const float *x = v + 8 * half;
        if constexpr (OF == O_BF16) {
          *(u32x4_t *)((uint16_t *)a.out + o) = (u32x4_t){pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                          pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        } else {
          *(f32x4_t *)((float *)a.out + o) = (f32x4_t){x[0], x[1], x[2], x[3]};
          *(f32x4_t *)((float *)a.out + o + 4) = (f32x4_t){x[4], x[5], x[6], x[7]};
        }
      }
    }
  };
  if (kh == 0)
    finish(std::integral_constant<int, 0>{});
  else
    finish(std::integral_constant<int, 1>{});
}

// ---------------------------------------------------------------------------
// 128 x 256 tiles, for unsplit products that finish sooner on them
// (no K-split): the same operands, chunks, copies and promotion as
// gemm_kernel, but wave w takes the 32 columns 32 w .. +31 and all 8 k-steps
// of every chunk. Against a 128 x 128 tile this halves the activation bytes
// copied per product and the float32 promotions per MFMA (one per group of 8
// k-steps instead of 4), and the waves hand nothing to each other at the
// end. A chunk's stage holds the activations (32 KiB) and 16 word-rows x 256
// columns of weights (16 KiB); the small ring holds 256 scales and 32
// zero-point words per stage, and the waves without a small copy write into
// one shared dead slot.
// ---------------------------------------------------------------------------
constexpr int kWideBN = 256;
constexpr int kWideWOff = 128 * kARow;                      // 32 KiB
constexpr int kWideStage = kWideWOff + 16 * kWideBN * 4;    // 48 KiB
constexpr int kWideSmall = 2048;                            // [256 scales][32 zero-point words]
constexpr int kWideZOff = 1024;

template <int OF, bool ZP>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_wide_kernel(GemmArgs a) {
  __shared__ __align__(16) unsigned char s_lds[kST * kWideStage + kSR * kWideSmall + 1024];
  unsigned char *const s_ring = s_lds;
  unsigned char *const s_small = s_lds + kST * kWideStage;
  unsigned char *const s_dead = s_small + kSR * kWideSmall;   // the dead copies' slot, never read
  constexpr int FM = 4;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // 0..7: columns 32 wave .. +31
  const int j = lane & 31, h = lane >> 5;
  // tile order: compact blocks of tiles per die, as in gemm_kernel
  int tx = blockIdx.x, ty = blockIdx.y;
  {
    const int TX = gridDim.x, TY = gridDim.y, T = TX * TY;
    if (T % 8 == 0) {
      const int L = blockIdx.x + TX * blockIdx.y;
      const int Lx = (L & 7) * (T >> 3) + (L >> 3);
      const int GM = TY < 4 ? TY : 4;
      const int per = GM * TX;
      const int g = Lx / per, first = g * GM;
      const int gs = TY - first < GM ? TY - first : GM;
      const int r = Lx - g * per;
      ty = first + r % gs;
      tx = r / gs;
    }
  }
  const int m0 = ty * kGemmBM;
  const int n0 = tx * kWideBN;
  const int nch = a.nchunks;

  const int R = a.K / 8;
  // weight row j of the MFMA is column fj of the wave's 32 (as in gemm_kernel)
  const int fj = 16 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3);
  const int cw = 32 * wave + fj;                         // within the workgroup's 256 columns

  const int a_rows = a.M - m0 < kGemmBM ? a.M - m0 : kGemmBM;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.A16 + (size_t)m0 * a.K), (short)0, a_rows * a.K * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.W + (size_t)(n0 / kTileCols) * R * kTileCols), (short)0, 4 * R * kTileCols * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.S32, (short)0, a.nchunks * a.Np * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.Z, (short)0, ZP ? a.nchunks * (a.N >> 3) * 4 : 0, kBufWord3);
  const __amdgpu_buffer_rsrc_t none_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a.W, (short)0, 0, kBufWord3);

  // activation copies: as in gemm_kernel (copy c = wave + 8 tt, 1 KiB each)
  const int ar0 = 4 * wave + (lane >> 4);
  const int a_voff0 = ar0 * (a.K * 2) + (((lane & 15) ^ (ar0 & 15)) << 4);
  const int a_vstep = 32 * a.K * 2;
  // weight copy i (0, 1) of wave w: word-row 2 w + i of the chunk, all 256
  // columns: lane -> 64-column tile lane / 16, columns 4 (lane % 16) .. +3
  // of it (LDS row-major [word-row][256 columns])
  const int w_voff0 = ((lane >> 4) * R + 2 * wave) * 256 + (lane & 15) * 16;

  auto copy_a = [&](int chunk, int stage, int tt, const __amdgpu_buffer_rsrc_t &rs) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(s_ring + stage * kWideStage + kAOff + (wave + 8 * tt) * 1024),
                                             16, a_voff0 + tt * a_vstep, chunk * 256, 0, 0);
  };
  auto copy_w = [&](int chunk, int stage, int i, const __amdgpu_buffer_rsrc_t &rs) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(s_ring + stage * kWideStage + kWideWOff + (2 * wave + i) * 1024),
                                             16, w_voff0 + i * 256, chunk * 4096, 0, 0);
  };
  // scales (wave 0: 256 floats) and zero-points (wave 1, with zero-points:
  // 32 words; lanes past them fill the slot's tail); the other waves issue
  // a copy with an out-of-range offset into the shared dead slot
  constexpr int kDead = (int)0x80000000u;
  const __amdgpu_buffer_rsrc_t small_rsrc = wave == 0 ? s_rsrc : z_rsrc;
  const int small_voff = wave == 0 ? n0 * 4 + lane * 16 : ((ZP && wave == 1) ? (n0 >> 3) * 4 + lane * 16 : kDead);
  const int small_cstride = wave == 0 ? a.Np * 4 : (ZP && wave == 1 ? (a.N >> 3) * 4 : 0);
  const bool small_real = wave == 0 || (ZP && wave == 1);
  auto copy_small = [&](int chunk, int sstage, const __amdgpu_buffer_rsrc_t &rs) {
    unsigned char *dst = small_real ? s_small + sstage * kWideSmall + (wave == 0 ? 0 : kWideZOff) : s_dead;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, chunk * small_cstride + small_voff, 0, 0, 0);
  };

  const uint32_t magic = f16_magic_pair();
  f16x2_t c0 = h2(0xE408E408u), c1 = h2(0xD480D480u);  // -(1024 + 8), -(64 + 8)

  f32x16_t acc[FM], P[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = P[i][e] = 0.f;

  const int s_rd = (32 * wave + 16 * h) * 4;            // the lane's 16 scales in a small stage
  const int w_rd = kWideWOff + (h * kWideBN + cw) * 4;  // + s * 2048: word-row 2 s + h
  int a_rd[8];                                          // k-step s, row tile 0; + fm * 32 rows
#pragma unroll
  for (int s = 0; s < 8; ++s) a_rd[s] = kAOff + j * kARow + (((2 * s + h) ^ (j & 15)) << 4);

  f32x4_t scA[4], scB[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) scA[u] = scB[u] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  typedef __attribute__((address_space(3))) const uint32_t lds_u32;
  typedef __attribute__((address_space(3))) const f16x8_t lds_f16x8;
  typedef __attribute__((address_space(3))) const f32x4_t lds_f32x4;

  // One chunk = 32 MFMA slots: slots 0..15 row tiles 0 and 1 (k-step
  // s = slot / 2, each weight word dequantized just before its first use and
  // kept for the second half), slots 16..31 tiles 2 and 3. Each slot also
  // promotes 2 elements: slots 0..15 tiles 2 and 3 of the previous chunk,
  // slots 16..31 tiles 0 and 1 of this chunk. Activation fragments are read
  // three slots ahead; the copies of chunk i + 2 (small first) are issued
  // between the MFMAs.
  auto run_chunk = [&](int i, f32x4_t(&scp)[4], f32x4_t(&scc)[4]) __attribute__((always_inline)) {
    const int sbase = (i % kST) * kWideStage;
    const unsigned char *sm = s_small + (i % kSR) * kWideSmall;
    const bool live = i + 2 < nch;
    const __amdgpu_buffer_rsrc_t ar = live ? a_rsrc : none_rsrc, wr = live ? w_rsrc : none_rsrc,
                                 sr = live ? small_rsrc : none_rsrc;
    const int cn = i + 2, stn = (i + 2) % kST;
    if constexpr (ZP) {
      const uint32_t zw = *(const uint32_t *)(sm + kWideZOff + (cw >> 3) * 4);
      const uint32_t z = (zw >> (4 * (cw & 7))) & 0xFu;
      const uint32_t zz = z | (z << 16);
      c0 = h2(0xE400E400u | zz);
      c1 = h2(0xD400D400u | (zz << 4));
    }
    uint32_t ab[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      ab[s] = (uint32_t)(uintptr_t)(s_ring + sbase) + a_rd[s];
      asm volatile("" : "+v"(ab[s]));
    }
    uint32_t wb = (uint32_t)(uintptr_t)(s_ring + sbase) + w_rd;
    uint32_t qm = (uint32_t)(uintptr_t)sm + s_rd;
    asm volatile("" : "+v"(wb), "+v"(qm));
    auto frag = [&](int q) {
      const int half = q >> 4, s = (q & 15) >> 1, fm = 2 * half + (q & 1);
      return *(lds_f16x8 *)(ab[s] + fm * 32 * kARow);
    };
    f16x8_t af[4];
    af[0] = frag(0);
    af[1] = frag(1);
    af[2] = frag(2);
    uint32_t wraw[2];
    wraw[0] = *(lds_u32 *)(wb);
    f16x8_t wq[8];
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int half = q >> 4, r = q & 15, s = r >> 1, fm = 2 * half + (q & 1);
      if (q + 3 < 32) af[(q + 3) & 3] = frag(q + 3);
      if (q == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) scc[u] = *(lds_f32x4 *)(qm + u * 16);
      }
      if (half == 0 && (q & 1) == 0) {
        // the word of k-step s + 1 is read one k-step ahead
        if (s + 1 < 8) wraw[(s + 1) & 1] = *(lds_u32 *)(wb + (s + 1) * 2048);
        wq[s] = dequant_f16(wraw[s & 1], magic, c0, c1);
      }
      if (s == 0)
        P[fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wq[s], af[q & 3], (f32x16_t){}, 0, 0, 0);
      else
        P[fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wq[s], af[q & 3], P[fm], 0, 0, 0);
      {
        const int tt = half == 0 ? 2 + (r >> 3) : (r >> 3);
        const int e0 = 2 * (r & 7);
        const f32x4_t sc = half == 0 ? scp[e0 >> 2] : scc[e0 >> 2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          acc[tt][e0 + e] = __builtin_fmaf(sc[(e0 & 3) + e], P[tt][e0 + e], acc[tt][e0 + e]);
      }
      if (q == 1) copy_small(cn, (i + 2) % kSR, sr);
      if (q == 5 || q == 11 || q == 17 || q == 23) copy_a(cn, stn, (q - 5) / 6, ar);
      if (q == 27 || q == 30) copy_w(cn, stn, q == 27 ? 0 : 1, wr);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  {
    const __amdgpu_buffer_rsrc_t r0a = nch > 0 ? a_rsrc : none_rsrc, r0w = nch > 0 ? w_rsrc : none_rsrc,
                                 r0s = nch > 0 ? small_rsrc : none_rsrc;
    const __amdgpu_buffer_rsrc_t r1a = nch > 1 ? a_rsrc : none_rsrc, r1w = nch > 1 ? w_rsrc : none_rsrc,
                                 r1s = nch > 1 ? small_rsrc : none_rsrc;
    copy_small(0, 0, r0s);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) copy_a(0, 0, tt, r0a);
    copy_w(0, 0, 0, r0w);
    copy_w(0, 0, 1, r0w);
    copy_small(1, 1, r1s);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) copy_a(1, 1, tt, r1a);
    copy_w(1, 1, 0, r1w);
    copy_w(1, 1, 1, r1w);
  }
  // at the top of chunk i at most the 6 main copies of chunk i + 1 are in
  // flight (its small copy, issued first, has landed)
  int i = 0;
  for (; i + 1 < nch; i += 2) {
    wait_then_barrier<6>();
    run_chunk(i, scB, scA);
    wait_then_barrier<6>();
    run_chunk(i + 1, scA, scB);
  }
  if (i < nch) {
    wait_then_barrier<6>();
    run_chunk(i, scB, scA);
  }
  {
    const bool odd = (nch & 1) != 0;
#pragma unroll
    for (int fm = 2; fm < FM; ++fm)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4_t sc = odd ? scA[e4] : scB[e4];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[fm][4 * e4 + e] = __builtin_fmaf(sc[e], P[fm][4 * e4 + e], acc[fm][4 * e4 + e]);
      }
  }
  // the copies past the last chunk (zeros into stages no one reads) land
  // before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // row m0 + 32 fm + j, columns n16 .. n16 + 15
  const int n16 = n0 + 32 * wave + 16 * h;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int row = m0 + 32 * fm + j;
    if (row >= a.M) continue;
    const int rex = a.rexp[row];
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = __builtin_amdgcn_ldexpf(acc[fm][q], -rex);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int n = n16 + 8 * half;
      if (n >= a.N) continue;
      const size_t o = (size_t)row * a.N + n;
      const float *x = v + 8 * half;
      if constexpr (OF == O_BF16) {
        *(u32x4_t *)((uint16_t *)a.out + o) = (u32x4_t){pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                        pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      } else {
        *(f32x4_t *)((float *)a.out + o) = (f32x4_t){x[0], x[1], x[2], x[3]};
        *(f32x4_t *)((float *)a.out + o + 4) = (f32x4_t){x[4], x[5], x[6], x[7]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pre-pass. Blocks [0, M): one workgroup (4 waves) per row m: e(m) = 141 - E,
// with E the biased exponent of the row's largest |a| (so that the largest
// scaled magnitude lies in [2^14, 2^15)), and A16[m][k] = fp16(a * 2^e(m))
// (round to nearest even; exact unless the scaled value is below 2^-14).
// Blocks past those: scales S32[g][n] = float(S[g][n]) for n < N, 0 for
// N <= n < Np (8 per thread). A workgroup per row (rather than a wave) puts
// every compute unit to work from M = 256 on and keeps the row in registers.
// ---------------------------------------------------------------------------
template <int PPT>  // 16-byte pieces per thread held in registers (K <= 2048 PPT); 0: two passes
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t *__restrict__ A, uint16_t *__restrict__ A16,
                                                   int *__restrict__ rexp, const uint16_t *__restrict__ S,
                                                   float *__restrict__ S32, int M, int K, int N, int Np,
                                                   int ngroups, int row_blocks) {
  __shared__ uint32_t s_wmax[4];
  if ((int)blockIdx.x >= row_blocks) {
    const long long idx = ((long long)(blockIdx.x - row_blocks) * 256 + threadIdx.x) * 8;
    if (idx >= (long long)ngroups * Np) return;
    const int g = (int)(idx / Np), n = (int)(idx % Np);
    u32x4_t v = {0, 0, 0, 0};
    if (n < N) v = *(const u32x4_t *)(S + (size_t)g * N + n);
    f32x4_t lo = {__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                  __uint_as_float(v[1] & 0xFFFF0000u)};
    f32x4_t hi = {__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xFFFF0000u), __uint_as_float(v[3] << 16),
                  __uint_as_float(v[3] & 0xFFFF0000u)};
    *(f32x4_t *)(S32 + idx) = lo;
    *(f32x4_t *)(S32 + idx + 4) = hi;
    return;
  }
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pieces = K / 8;  // 16-byte pieces of the row
  const u32x4_t *src = (const u32x4_t *)(A + (size_t)m * K);
  u32x4_t *dst = (u32x4_t *)(A16 + (size_t)m * K);
  // largest magnitude: bf16 magnitudes compare as integers
  auto mag = [](const u32x4_t &x) {
    uint32_t r = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t lo = x[c] & 0x7FFFu, hi = (x[c] >> 16) & 0x7FFFu;
      r = r > lo ? r : lo;
      r = r > hi ? r : hi;
    }
    return r;
  };
  u32x4_t v[PPT > 0 ? PPT : 1];
  uint32_t mb = 0;
  if constexpr (PPT > 0) {
    // pieces past the row re-read the row's last piece (in bounds; the
    // maximum is unchanged and nothing is stored for them)
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int p = threadIdx.x + 256 * u;
      v[u] = src[p < pieces ? p : pieces - 1];
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const uint32_t x = mag(v[u]);
      mb = mb > x ? mb : x;
    }
  } else {
    for (int p = threadIdx.x; p < pieces; p += 256) {
      const uint32_t x = mag(src[p]);
      mb = mb > x ? mb : x;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)mb, o);
    mb = mb > y ? mb : y;
  }
  if (lane == 0) s_wmax[wave] = mb;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 4; ++w) mb = mb > s_wmax[w] ? mb : s_wmax[w];
  const int e = 141 - (int)(mb >> 7);  // bf16 exponent field: bits 14..7 of the magnitude
  if (threadIdx.x == 0) rexp[m] = e;
  auto convert = [&](const u32x4_t &x) {
    u32x4_t r;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x2_t f = {__builtin_amdgcn_ldexpf(__uint_as_float(x[c] << 16), e),
                   __builtin_amdgcn_ldexpf(__uint_as_float(x[c] & 0xFFFF0000u), e)};
      r[c] = u32(__builtin_convertvector(f, f16x2_t));
    }
    return r;
  };
  if constexpr (PPT > 0) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int p = threadIdx.x + 256 * u;
      if (p < pieces) dst[p] = convert(v[u]);
    }
  } else {
    for (int p = threadIdx.x; p < pieces; p += 256) dst[p] = convert(src[p]);
  }
}

// from this many rows (256 workgroups of 4 rows) the pre-pass takes a wave per
// row
constexpr int kPrepWaveMinRows = 1024;

// The same pre-pass with one wave per row (4 rows per workgroup), the row
// held in registers (NCH 16-byte pieces per lane, K <= 512 NCH) and its
// maximum found by lane exchanges alone; used when the rows alone give every
// compute unit a workgroup. Blocks past ceil(M / 4) convert the scales.
template <int NCH>
__global__ __launch_bounds__(256) void prep_wave_kernel(const uint16_t *__restrict__ A, uint16_t *__restrict__ A16,
                                                        int *__restrict__ rexp, const uint16_t *__restrict__ S,
                                                        float *__restrict__ S32, int M, int K, int N, int Np,
                                                        int ngroups, int row_blocks) {
  if ((int)blockIdx.x >= row_blocks) {
    const long long idx = ((long long)(blockIdx.x - row_blocks) * 256 + threadIdx.x) * 8;
    if (idx >= (long long)ngroups * Np) return;
    const int g = (int)(idx / Np), n = (int)(idx % Np);
    u32x4_t v = {0, 0, 0, 0};
    if (n < N) v = *(const u32x4_t *)(S + (size_t)g * N + n);
    f32x4_t lo = {__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                  __uint_as_float(v[1] & 0xFFFF0000u)};
    f32x4_t hi = {__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xFFFF0000u), __uint_as_float(v[3] << 16),
                  __uint_as_float(v[3] & 0xFFFF0000u)};
    *(f32x4_t *)(S32 + idx) = lo;
    *(f32x4_t *)(S32 + idx + 4) = hi;
    return;
  }
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;   // whole waves
  const int pieces = K / 8;
  const u32x4_t *src = (const u32x4_t *)(A + (size_t)m * K);
  u32x4_t *dst = (u32x4_t *)(A16 + (size_t)m * K);
  u32x4_t v[NCH];
  // pieces past the row re-read its last piece (in bounds; not stored)
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int p = lane + 64 * u;
    v[u] = src[p < pieces ? p : pieces - 1];
  }
  uint32_t mb = 0;
#pragma unroll
  for (int u = 0; u < NCH; ++u)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t lo = v[u][c] & 0x7FFFu, hi = (v[u][c] >> 16) & 0x7FFFu;
      mb = mb > lo ? mb : lo;
      mb = mb > hi ? mb : hi;
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)mb, o);
    mb = mb > y ? mb : y;
  }
  const int e = 141 - (int)(mb >> 7);  // as in prep_kernel
  if (lane == 0) rexp[m] = e;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int p = lane + 64 * u;
    if (p >= pieces) continue;
    u32x4_t r;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x2_t f = {__builtin_amdgcn_ldexpf(__uint_as_float(v[u][c] << 16), e),
                   __builtin_amdgcn_ldexpf(__uint_as_float(v[u][c] & 0xFFFF0000u), e)};
      r[c] = u32(__builtin_convertvector(f, f16x2_t));
    }
    dst[p] = r;
  }
}

template <int OF, bool ZP>
static hipError_t go(const GemmArgs &a, dim3 grid, bool wide, hipStream_t st) {
  if (wide)
    gemm_wide_kernel<OF, ZP><<<dim3(grid.x / 2, grid.y), kGemmThreads, 0, st>>>(a);
  else
    gemm_kernel<OF, ZP><<<grid, kGemmThreads, 0, st>>>(a);
  return hipGetLastError();
}

// The dispatcher sends only K % 128 == 0, N % 8 == 0 here, with
// M * K * 2 <= INT_MAX and (K / 128) * Np * 4 <= INT_MAX.
hipError_t launch_gemm(int ofmt, bool zp, const GemmArgs &a, dim3 grid, bool wide, hipStream_t st) {
  if (a.K % kGemmKC != 0 || a.N % 8 != 0) return hipErrorInvalidValue;
  if (wide && (a.nsplit != 1 || a.Np % kWideBN != 0 || grid.x % 2 != 0)) return hipErrorInvalidValue;
  const long long sblocks = ((long long)a.nchunks * a.Np / 8 + 255) / 256;
  const int nch = (a.K / 8 + 63) / 64;    // pieces per lane with a wave per row
  if (a.M >= kPrepWaveMinRows && nch <= 16) {
    const int row_blocks = (a.M + 3) / 4;
    const dim3 pgrid((unsigned)(row_blocks + sblocks));
#define QG_PREPW(P) \
  prep_wave_kernel<P><<<pgrid, 256, 0, st>>>(a.A, a.A16, a.rexp, a.S, a.S32, a.M, a.K, a.N, a.Np, a.nchunks, row_blocks)
    if (nch <= 4)
      QG_PREPW(4);
    else if (nch <= 8)
      QG_PREPW(8);
    else
      QG_PREPW(16);
#undef QG_PREPW
  } else {
  const int row_blocks = a.M;
  const dim3 pgrid((unsigned)(row_blocks + sblocks));
  const int ppl = (a.K / 8 + 255) / 256;  // pieces per thread
#define QG_PREP(P) \
  prep_kernel<P><<<pgrid, 256, 0, st>>>(a.A, a.A16, a.rexp, a.S, a.S32, a.M, a.K, a.N, a.Np, a.nchunks, row_blocks)
  if (ppl <= 1)
    QG_PREP(1);
  else if (ppl <= 2)
    QG_PREP(2);
  else if (ppl <= 4)
    QG_PREP(4);
  else if (ppl <= 8)
    QG_PREP(8);
  else
    QG_PREP(0);
#undef QG_PREP
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ofmt == O_BF16) return zp ? go<O_BF16, true>(a, grid, wide, st) : go<O_BF16, false>(a, grid, wide, st);
  return zp ? go<O_F32, true>(a, grid, wide, st) : go<O_F32, false>(a, grid, wide, st);
}

}  // namespace qg
