// MFMA path of the group-quantized GEMM: bf16 activations, int4 weights,
// bf16 scales, optional int4 zero-points, groups of 128; for M large enough
// that the work is a dense contraction (prefill).
//
// Structure (the W4A16 main loop of the page "quantization-and-fused-kernels"
// (arganzheng.life), section 三.1: int4 tile -> unpack in registers -> matrix
// instruction in bf16 with float32 accumulation; and the multi-stage
// global-to-shared pipeline of its section 三.3, item 2):
//   - workgroup tile 128 x 128, K in chunks of 128 = one group; 4 waves, one
//     per SIMD, each owning all 128 rows and 32 columns (8 x 2 tiles of
//     v_mfma_f32_16x16x32_bf16, so each dequantized weight fragment feeds 8
//     MFMAs);
//   - the chunk's activation tile, scales, zero-points and activation sums
//     are copied by buffer loads straight into LDS (no registers on the way),
//     into a ring of ST stages: 3 (one chunk in use, two in flight; 103 KiB,
//     one workgroup per compute unit) when the grid is about one workgroup
//     per compute unit, 2 (one in flight; 69 KiB, so two workgroups share a
//     compute unit and cover each other's waits) when there are at least two
//     tiles per compute unit (measured on MI355X, K = N = 4096: M = 4096 151
//     -> 136 us, M = 2048 77 -> 70 us). Each wave waits for its own copies,
//     then a barrier makes every wave's copies visible;
//   - the activation tile's 16-byte pieces are XOR-swizzled with the row
//     index, so the MFMA fragment reads of 16 rows hit 16 different 4-bank
//     groups; rows past M read zeros through the buffer's range check (their
//     results are not written);
//   - weights: each lane loads 8 bytes of packed words (2 adjacent columns x
//     8 k) into registers one chunk ahead, and turns each word into four bf16
//     pairs (128 + q) with one and-or per pair (bf16 magic number 0x4300,
//     section 二.4 of the same page); the two columns feed the two column
//     tiles of the wave, so column j of tile f is physical column n + 2j + f.
//     The weight fragment is the MFMA's first operand and the activation
//     fragment its second, so each tile is computed transposed: a lane holds
//     row 16 fm + l % 16 and, over its two tiles, the 8 adjacent columns
//     32 w + 8 (l / 16) .. +7, which the epilogue writes with one 16-byte
//     store (8-byte stores of 2 columns x 4 rows per lane before: measured
//     M = 4096 142 -> 135 us, M = 2048 75 -> 69 us, M = 1024 about 2% faster,
//     M = 256 2% slower);
//   - per group, the MFMA accumulates sum_k a_k (128 + q_k) on top of the
//     initial value -(128 + z) * sum_k a_k, which gives sum_k a_k (q_k - z);
//     the group's scale is then applied in float32 (acc += s * P), the
//     per-block promotion of the same page, section 四.3, overlapped with the
//     next chunk's MFMAs. The (q - z) values are exact in bf16 and the scale
//     never rounds into a bf16 weight. The per-(group, row) activation sums
//     come from asum_kernel, a pre-pass that adds each group's 128 values in
//     a fixed order;
//   - with nsplit > 1, K-slices of whole chunks write float32 partial tiles
//     that a second kernel adds in the fixed order z = 0..nsplit-1 (the
//     z-split and fixed-order reduce of the page "04 · 分组量化 GEMM 内核"
//     (developer.aliyun.com), section 3.3).
#include "common.h"

namespace qg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_g;
typedef __attribute__((ext_vector_type(2))) float f32x2_g;
typedef __attribute__((address_space(3))) void lds_void;

// One LDS stage holds the operands of one chunk that all waves share:
// [activations 128 x 256 B][scales 128 x 2 B][activation sums 128 x 4 B]
// [zero-points 16 x 4 B]. Each small slot is as large as one wave-wide copy
// writes (lanes past the useful part copy neighbouring data into the slot's
// tail, never read). The packed weights go straight to registers.
constexpr int kARow = kGemmKC * 2;                   // 256 B per activation row
constexpr int kAOff = 0;
constexpr int kSOff = kAOff + kGemmBM * kARow;       // 32 KiB
constexpr int kQOff = kSOff + 1024;
constexpr int kZOff = kQOff + 1024;
constexpr int kStageBytes = kZOff + 256;             // 35072
constexpr int kBufWord3 = 0x00020000;
constexpr int kPolicyStream = 2;                     // non-temporal

// Wait until at most N of this wave's global loads (including the copies
// into LDS) are outstanding and its LDS reads are done, then the workgroup
// barrier; the memory clobber keeps the compiler from moving memory
// accesses across it. Loads complete in issue order.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
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

template <typename T>
__device__ __forceinline__ T lds_read(const unsigned char *base, int off) {
  return *(const T *)(base + off);
}

// 4 waves, one per SIMD: wave w owns all 128 rows and the 32 columns
// n0 + 32 w .. +31 of the tile (8 x 2 MFMA tiles), so a weight fragment is
// dequantized once and feeds 8 MFMAs.
template <int OF, bool ZP, int ST>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) unsigned char s_ring[ST * kStageBytes];
  constexpr int FM = 8, FN = 2;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int m0 = blockIdx.y * kGemmBM;
  const int n0 = blockIdx.x * kGemmBN;
  const int cw = 32 * wave + 2 * li;                   // this lane's 2 columns, within the tile

  int cb, ccount;
  split_range(a.nchunks, a.nsplit, blockIdx.z, cb, ccount);

  const int R = a.K / 8;
  // activation rows past M read zeros through the range check (the row
  // offset is in the VGPR operand; the chunk offset in the SGPR one stays
  // inside a valid row)
  const int a_rows = a.M - m0 < kGemmBM ? a.M - m0 : kGemmBM;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.A + (size_t)m0 * a.K), (short)0, a_rows * a.K * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.W + (size_t)(n0 / kTileCols) * R * kTileCols), (short)0, 2 * R * kTileCols * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.S, (short)0, a.nchunks * a.N * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t q_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.asum, (short)0, a.nchunks * a.Mp * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.Z, (short)0, ZP ? a.nchunks * (a.N >> 3) * 4 : 0, kBufWord3);
  // Every load is issued unconditionally (straight-line code, so the
  // compiler counts the loads in flight exactly); a load for a chunk past
  // the slice sets the top bit of its VGPR offset, which the range check of
  // the buffer (every resource here has at most INT_MAX bytes) turns into a
  // zero result without a memory access. Such copies write zeros into a
  // stage no later chunk uses.
  constexpr int kDead = (int)0x80000000u;

  // activations: copy j of wave w writes LDS bytes (4j + w) KiB of the tile:
  // pieces p = 64 (4j + w) + lane; piece p is row p/16 = 16 j + r0, physical
  // slot p%16, holding logical 16-byte chunk (p%16) ^ (row%16) of the row
  // (row%16 = r0%16 does not depend on j).
  const int r0 = 4 * wave + lk;
  const int a_voff0 = r0 * (a.K * 2) + ((lane & 15) ^ (r0 & 15)) * 16;
  const int a_vstep = 16 * a.K * 2;          // + j rows of 16
  // weights: per k-step s, word-row 4s + lk of the chunk and the lane's two
  // adjacent columns (8 bytes; 16 lanes read a 128-byte row segment). MFMA
  // column j of tile f is column n0 + 32 w + 2j + f.
  const int b_voff = ((cw >> 6) * R * kTileCols + lk * kTileCols + (cw & 63)) * 4;

  auto load_b = [&](int chunk, int s, int dead) {
    return __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(w_rsrc, b_voff | dead, (chunk * 16 + 4 * s) * kTileCols * 4,
                                                      kPolicyStream));
  };
  // The small copies read past their useful part and, at the last chunk,
  // past the end of their array: those lanes rely on the buffer's range
  // check (which returns zeros), so the whole offset is in the VGPR operand
  // (the SGPR offset is not range-checked).
  auto copy_small = [&](int chunk, int stage, int dead) {
    unsigned char *st = s_ring + stage * kStageBytes;
    if (wave == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_void *)(st + kSOff), 16,
                                               ((chunk * a.N + n0) * 2 + lane * 16) | dead, 0, 0, 0);
    } else if (wave == 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q_rsrc, (lds_void *)(st + kQOff), 16,
                                               ((chunk * a.Mp + m0) * 4 + lane * 16) | dead, 0, 0, 0);
    } else if (ZP && wave == 2) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(z_rsrc, (lds_void *)(st + kZOff), 4,
                                               ((chunk * (a.N >> 3) + (n0 >> 3)) * 4 + lane * 4) | dead, 0, 0,
                                               0);
    }
  };
  auto copy_a = [&](int chunk, int stage, int j, int dead) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void *)(s_ring + stage * kStageBytes + kAOff +
                                                                  (4 * j + wave) * 1024),
                                             16, (a_voff0 + j * a_vstep) | dead, chunk * kGemmKC * 2, 0, 0);
  };

  const uint32_t magic = bf16_magic_pair();
  const int c8 = 32 * wave + 8 * lk;                 // first of the lane's 8 output columns, within the tile
  const int s_off = kSOff + c8 * 2;
  const int q_off = kQOff + li * 4;                  // + 64 fm
  const int z_off = kZOff + (c8 >> 3) * 4;

  f32x4_t acc[FM][FN], P[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = P[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float sc[FN][4] = {};   // scales of the chunk whose sums are in P: column 2 r + fn of the lane's 8
  u32x2_t bcur[4], bnext[4];

  // Chunk i (local) lives in stage i % ST. While chunk i is computed, its
  // MFMA sequence also issues, one piece per activation fragment, the
  // weight loads of chunk i + 1 (first, into registers) and then the copies
  // of chunk i + ST - 1 into the stage chunk i - 1 used: every wave has
  // passed the barrier at the top of chunk i, so every wave is done with it.
  // Spreading the loads keeps the compute unit's address unit from stalling
  // every wave with one burst. With 3 stages, at the top of chunk i at most
  // the 9 copies of chunk i + 1 may still be in flight (they were issued
  // after the weight loads of chunk i), so vmcnt(8) covers chunk i's copies
  // and weights on every wave (waves 0..2 also wait for their small copy,
  // issued early); with 2 stages nothing may be (vmcnt(0)).
  //
  // One chunk on the MFMA units is software-pipelined with the promotion of
  // the previous chunk: tile (fm, fn) of P is first added into acc with the
  // previous chunk's scales, then restarted from -(128 + z) * sum(a) by the
  // chunk's first k-step. (Without zero-points the pre-pass already stores
  // -136 * sum(a).)
  auto run_chunk = [&](int i) {
    const unsigned char *sb = s_ring + (i % ST) * kStageBytes;
    constexpr int AH = ST - 1;   // copies run AH chunks ahead
    const int db = i + 1 < ccount ? 0 : kDead, dc = i + AH < ccount ? 0 : kDead;
    const int cs = (i + AH) % ST;
    const u32x4_t sv = lds_read<u32x4_t>(sb, s_off);
    f32x4_t bias[FN] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
    if constexpr (ZP) {
      const uint32_t zw = lds_read<uint32_t>(sb, z_off);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int r = 0; r < 4; ++r) bias[fn][r] = -(float)(128 + (int)((zw >> (4 * (2 * r + fn))) & 0xFu));
    }
    // The 32 activation fragments of the chunk (k-step s, row tile fm) are
    // read from LDS two fragments ahead of their MFMAs.
    auto a_frag = [&](int q) {
      const int s = q / FM, fm = q % FM;
      return lds_read<bf16x8_t>(sb, kAOff + (16 * fm + li) * kARow + 16 * ((4 * s + lk) ^ li));
    };
    bf16x8_t af[3];
    af[0] = a_frag(0);
    af[1] = a_frag(1);
    bf16x8_t bfr[FN];
#pragma unroll
    for (int q = 0; q < 4 * FM; ++q) {
      const int s = q / FM, fm = q % FM;
      if (q + 2 < 4 * FM) af[(q + 2) % 3] = a_frag(q + 2);
      // loads for later chunks, one piece per fragment
      if (q < 4)
        bnext[q] = load_b(cb + i + 1, q, db);
      else if (q == 4)
        copy_small(cb + i + AH, cs, dc);
      else if (q >= 6 && (q - 6) % 3 == 0 && (q - 6) / 3 < 8)
        copy_a(cb + i + AH, cs, (q - 6) / 3, dc);
      if (fm == 0) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) bfr[fn] = dequant_word(bcur[s][fn], magic);
      }
      const bf16x8_t afr = af[q % 3];
      float rs = 0.f;
      if (s == 0) rs = lds_read<float>(sb, q_off + 64 * fm);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        if (s == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[fm][fn][r] = __builtin_fmaf(sc[fn][r], P[fm][fn][r], acc[fm][fn][r]);
          const f32x4_t init = ZP ? rs * bias[fn] : (f32x4_t){rs, rs, rs, rs};
          P[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[fn], afr, init, 0, 0, 0);
        } else {
          P[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[fn], afr, P[fm][fn], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[0][r] = __uint_as_float(sv[r] << 16);
      sc[1][r] = __uint_as_float(sv[r] & 0xFFFF0000u);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) bcur[s] = bnext[s];
  };

  // prologue: copies of chunk 0, weights of chunk 0, copies of chunk 1
  {
    const int d0 = ccount > 0 ? 0 : kDead, d1 = ccount > 1 ? 0 : kDead;
    copy_small(cb, 0, d0);
#pragma unroll
    for (int j = 0; j < 8; ++j) copy_a(cb, 0, j, d0);
#pragma unroll
    for (int s = 0; s < 4; ++s) bcur[s] = load_b(cb, s, d0);
    if constexpr (ST == 3) {
      copy_small(cb + 1, 1, d1);
#pragma unroll
      for (int j = 0; j < 8; ++j) copy_a(cb + 1, 1, j, d1);
    }
  }
  for (int i = 0; i < ccount; ++i) {
    wait_then_barrier<ST == 3 ? 8 : 0>();
    run_chunk(i);
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[fm][fn][q] = __builtin_fmaf(sc[fn][q], P[fm][fn][q], acc[fm][fn][q]);

  // ---- epilogue: row m0 + 16 fm + li, columns n0 + c8 .. +7 (element (fn, r) is column 2 r + fn) ----
  const int n8 = n0 + c8;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int row = m0 + 16 * fm + li;
    if (row >= a.M) continue;
    const f32x4_t lo = {acc[fm][0][0], acc[fm][1][0], acc[fm][0][1], acc[fm][1][1]};
    const f32x4_t hi = {acc[fm][0][2], acc[fm][1][2], acc[fm][0][3], acc[fm][1][3]};
    if (a.nsplit > 1) {
      // K-slice partials; a second kernel adds them in the order z = 0..nsplit-1
      float *p = &a.partial[((size_t)blockIdx.z * a.M + row) * a.Np + n8];
      *(f32x4_t *)p = lo;
      *(f32x4_t *)(p + 4) = hi;
      continue;
    }
    if (n8 >= a.N) continue;   // N % 8 == 0: the lane's 8 columns are all in or all out
    const size_t o = (size_t)row * a.N + n8;
    if constexpr (OF == O_BF16) {
      *(u32x4_t *)((uint16_t *)a.out + o) = (u32x4_t){pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                                      pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
    } else {
      *(f32x4_t *)((float *)a.out + o) = lo;
      *(f32x4_t *)((float *)a.out + o + 4) = hi;
    }
  }
}

// ---------------------------------------------------------------------------
// Activation sums: asum[g][m] = mult * sum_{k in group g} a[m][k] (groups of
// 128), for m < M; row stride Mp. One wave per row: lane l reads 16 bytes of each
// 1 KiB block of the row (block j covers groups 4j .. 4j+3; lanes 16i .. 16i+15
// hold group 4j + i), adds its 8 values in k order, and the 16 lanes of a
// group (one DPP row) combine in a fixed order of row rotations. Up to 8
// blocks are loaded before any is added, so every lane keeps 8 loads in
// flight.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void asum_kernel(const uint16_t *__restrict__ A, float *__restrict__ asum, int M,
                                                  int K, int Mp, float mult) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int ngroups = K / 128;
  const int nblocks = (ngroups + 3) / 4;
  const uint16_t *row = A + (size_t)m * K;
  for (int j0 = 0; j0 < nblocks; j0 += 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // past the row's last group: re-read its first piece (in bounds), unused
      const int g = 4 * (j0 + u) + (lane >> 4);
      const int off = g < ngroups ? g * 128 + 8 * (lane & 15) : 0;
      v[u] = *(const u32x4_t *)(row + off);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = 4 * (j0 + u) + (lane >> 4);
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s += __uint_as_float(v[u][q] << 16);
        s += __uint_as_float(v[u][q] & 0xFFFF0000u);
      }
      // fixed-order sum over the 16 lanes of the group with DPP row rotations
      // (lane 0 of the row ends with ((s0 + s8) + (s4 + s12)) + ...)
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x128, 0xF, 0xF, false));  // row_ror:8
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x124, 0xF, 0xF, false));  // row_ror:4
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x122, 0xF, 0xF, false));  // row_ror:2
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x121, 0xF, 0xF, false));  // row_ror:1
      if (g < ngroups && (lane & 15) == 0) asum[(size_t)g * Mp + m] = s * mult;
    }
  }
}

template <int OF, bool ZP>
static hipError_t go(const GemmArgs &a, dim3 grid, hipStream_t st) {
  if (a.stages == 2)
    gemm_kernel<OF, ZP, 2><<<grid, kGemmThreads, 0, st>>>(a);
  else
    gemm_kernel<OF, ZP, 3><<<grid, kGemmThreads, 0, st>>>(a);
  return hipGetLastError();
}

// The dispatcher sends only G == 128, K % 128 == 0, N % 8 == 0 here.
hipError_t launch_gemm(int ofmt, bool zp, int G, const GemmArgs &a, dim3 grid, hipStream_t st) {
  if (G != 128 || a.K % kGemmKC != 0 || a.N % 8 != 0) return hipErrorInvalidValue;
  // without zero-points the MFMA starts from -(128 + 8) * sum(a): store that
  asum_kernel<<<(a.M + 3) / 4, 256, 0, st>>>(a.A, a.asum, a.M, a.K, a.Mp, zp ? 1.f : -136.f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ofmt == O_BF16) return zp ? go<O_BF16, true>(a, grid, st) : go<O_BF16, false>(a, grid, st);
  return zp ? go<O_F32, true>(a, grid, st) : go<O_F32, false>(a, grid, st);
}

}  // namespace qg
