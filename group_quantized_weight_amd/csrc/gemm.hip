// MFMA path of the group-quantized GEMM: bf16 activations, int4 weights,
// bf16 scales, optional int4 zero-points, groups of 128; for M large enough
// that the work is a dense contraction (prefill).
//
// Structure (the W4A16 main loop of the page "quantization-and-fused-kernels"
// (arganzheng.life), section 三.1: int4 tile -> unpack in registers -> matrix
// instruction in bf16 with float32 accumulation; and the multi-stage
// global-to-shared pipeline of its section 三.3, item 2):
//   - workgroup tile 128 x 128, K in chunks of 128 = one group; 8 waves in
//     two halves of 2 x 2 (each wave 64 x 64 = 4 x 4 tiles of
//     v_mfma_f32_16x16x32_bf16). The halves take alternate chunks of the
//     workgroup's K-range, so each SIMD runs two waves; at the end half 1
//     hands its accumulators to half 0 through LDS;
//   - the chunk's activation tile, scales, zero-points and activation sums
//     are copied by buffer loads straight into LDS (no registers on the way),
//     into a ring of 4 stages (two chunks in use, two in flight). Each wave
//     waits for its own copies, then a barrier makes every wave's copies
//     visible;
//   - the activation tile's 16-byte pieces are XOR-swizzled with the row
//     index, so the MFMA fragment reads of 16 rows hit 16 different 4-bank
//     groups; rows past M are clamped to row M-1 (their results are dropped);
//   - weights: each lane loads 16 bytes of packed words (4 adjacent columns x
//     8 k) into registers one chunk ahead, and turns each word into four bf16
//     pairs (128 + q) with one and-or per pair (bf16 magic number 0x4300,
//     section 二.4 of the same page); the four columns feed the four MFMA
//     column tiles of the wave, so MFMA column j of tile f is physical column
//     n + 4j + f;
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

// One LDS stage holds one chunk's operands that every wave of a half shares:
// [activations 128 x 256 B][scales 128 x 2 B][activation sums 128 x 4 B]
// [zero-points 16 x 4 B]. Each small slot is as large as one wave-wide copy
// writes (lanes past the useful part copy neighbouring data into the slot's
// tail, never read). The packed weights go straight to registers.
constexpr int kHalves = 2;                           // the workgroup's K-split
constexpr int kStages = 4;                           // 2 chunks in use, 2 in flight
constexpr int kARow = kGemmKC * 2;                   // 256 B per activation row
constexpr int kAOff = 0;
constexpr int kSOff = kAOff + kGemmBM * kARow;       // 32 KiB
constexpr int kQOff = kSOff + 1024;
constexpr int kZOff = kQOff + 1024;
constexpr int kStageBytes = kZOff + 256;             // 35072
constexpr int kBufWord3 = 0x00020000;
constexpr int kPolicyStream = 2;                     // non-temporal
static_assert(kStages * kStageBytes >= 4 * 64 * 64 * 4, "the ring also holds one half's accumulators");

// Wait for this wave's outstanding global loads (including the copies into
// LDS) and LDS reads, then the workgroup barrier; the memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void wait_all_then_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// 8 waves: two halves of 4 (2 x 2, each wave 64 x 64 of the tile). Half h
// takes the chunks cb + h, cb + h + 2, ... of the workgroup's K-slice, so
// two waves share each SIMD and one's MFMAs cover the other's waits. At the
// end, half 1 hands its accumulators to half 0 through LDS, which adds them
// (half 0 + half 1, a fixed order) and writes the tile.
template <int OF, bool ZP>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) unsigned char s_ring[kStages * kStageBytes];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int half = wave >> 2, qw = wave & 3;           // qw: wave within its half
  const int wm = qw >> 1, wn = qw & 1;
  const int li = lane & 15, lk = lane >> 4;
  const int m0 = blockIdx.y * kGemmBM;
  const int n0 = blockIdx.x * kGemmBN;
  const int ncol = n0 + 64 * wn + 4 * li;   // this lane's 4 columns (one per column tile)

  int cb, ccount;
  split_range(a.nchunks, a.nsplit, blockIdx.z, cb, ccount);

  const int R = a.K / 8;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.A + (size_t)m0 * a.K), (short)0, 0x7FFFFFFF, kBufWord3);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.W + (size_t)(n0 / kTileCols) * R * kTileCols), (short)0, 0x7FFFFFFF, kBufWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.S, (short)0, a.nchunks * a.N * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t q_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.asum, (short)0, a.nchunks * a.Mp * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.Z, (short)0, ZP ? a.nchunks * (a.N >> 3) * 4 : 0, kBufWord3);

  // activations: copy j of wave qw writes LDS bytes (4j + qw) KiB of the
  // tile: pieces p = 64 (4j + qw) + lane; piece p is row p/16, physical
  // slot p%16, holding logical 16-byte chunk (p%16) ^ (row%16) of the row.
  int a_voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = (4 * j + qw) * 64 + lane;
    const int r = p >> 4, c = (p & 15) ^ (r & 15);
    const int row = min(m0 + r, a.M - 1) - m0;
    a_voff[j] = row * (a.K * 2) + c * 16;
  }
  // weights: per k-step s, word-row 4s + lk of the chunk, columns 4 li .. +3
  // of the wave's 64-column tile (a wave reads 1 KiB of contiguous memory)
  const int b_voff = wn * R * 256 + lk * 256 + li * 16;

  // The copies of a chunk into LDS, issued by the 4 waves of the half that
  // uses it. The small copies read past their useful part and, at the last
  // chunk, past the end of their array: those lanes rely on the buffer's
  // range check (which returns zeros), so the whole offset is in the VGPR
  // operand (the SGPR offset is not range-checked).
  auto issue = [&](int chunk, int stage) {
    unsigned char *st = s_ring + stage * kStageBytes;
    if (qw == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_void *)(st + kSOff), 16,
                                               (chunk * a.N + n0) * 2 + lane * 16, 0, 0, 0);
    } else if (qw == 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q_rsrc, (lds_void *)(st + kQOff), 16,
                                               (chunk * a.Mp + m0) * 4 + lane * 16, 0, 0, 0);
    } else if (ZP && qw == 2) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(z_rsrc, (lds_void *)(st + kZOff), 4,
                                               (chunk * (a.N >> 3) + (n0 >> 3)) * 4 + lane * 4, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void *)(st + kAOff + (4 * j + qw) * 1024), 16,
                                               a_voff[j], chunk * kGemmKC * 2, 0, 0);
  };
  auto load_b = [&](int chunk, u32x4_t *dst) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      dst[s] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, b_voff, (chunk * 16 + 4 * s) * 256, kPolicyStream));
  };

  const uint32_t magic = bf16_magic_pair();
  const int a_row0 = 64 * wm + li;                   // + 16 fm
  const int s_off = kSOff + (64 * wn + 4 * li) * 2;
  const int q_off = kQOff + (64 * wm + 4 * lk) * 4;  // + 64 fm
  const int z_off = kZOff + ((64 * wn + 4 * li) >> 3) * 4;
  const int z_shift = (4 * li) & 7;                  // 0 or 4: first nibble of the lane's 4 columns

  f32x4_t acc[4][4], P[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = P[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float sc[4] = {0.f, 0.f, 0.f, 0.f};   // scales of the chunk whose sums are in P

  // One chunk on the MFMA units, software-pipelined with the promotion of
  // the wave's previous chunk: tile (fm, fn) of P is first added into acc
  // with the previous chunk's scales, then restarted from -(128 + z) * sum(a)
  // by the chunk's first k-step, so the float32 promotion overlaps the MFMAs.
  auto run_chunk = [&](const unsigned char *sb, const u32x4_t *bw) {
    const u32x2_t sv = lds_read<u32x2_t>(sb, s_off);
    f32x4_t rs[4];
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) rs[fm] = lds_read<f32x4_t>(sb, q_off + 64 * fm);
    float bias[4] = {-136.f, -136.f, -136.f, -136.f};
    if constexpr (ZP) {
      const uint32_t zw = lds_read<uint32_t>(sb, z_off) >> (4 * z_shift);
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) bias[fn] = -(float)(128 + (int)((zw >> (4 * fn)) & 0xFu));
    }
    // The 16 activation fragments of the chunk (k-step s, row tile fm) are
    // read from LDS two fragments ahead of their MFMAs, so the read latency
    // is covered by the MFMAs of the two previous fragments.
    auto a_frag = [&](int q) {
      const int s = q >> 2, fm = q & 3;
      return lds_read<bf16x8_t>(sb, kAOff + (a_row0 + 16 * fm) * kARow + 16 * ((4 * s + lk) ^ li));
    };
    bf16x8_t af[3];
    af[0] = a_frag(0);
    af[1] = a_frag(1);
    bf16x8_t bfr[4];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int s = q >> 2, fm = q & 3;
      if (q + 2 < 16) af[(q + 2) % 3] = a_frag(q + 2);
      if (fm == 0) {
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) bfr[fn] = dequant_word(bw[s][fn], magic);
      }
      const bf16x8_t afr = af[q % 3];
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        if (s == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[fm][fn][r] = __builtin_fmaf(sc[fn], P[fm][fn][r], acc[fm][fn][r]);
          const f32x4_t init = rs[fm] * bias[fn];
          P[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[fn], init, 0, 0, 0);
        } else {
          P[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[fn], P[fm][fn], 0, 0, 0);
        }
      }
    }
    sc[0] = __uint_as_float(sv[0] << 16);
    sc[1] = __uint_as_float(sv[0] & 0xFFFF0000u);
    sc[2] = __uint_as_float(sv[1] << 16);
    sc[3] = __uint_as_float(sv[1] & 0xFFFF0000u);
  };

  // Local chunk i (= cb + i) lives in stage i % 4 and belongs to half i % 2.
  // Round r uses chunks 2r (half 0) and 2r + 1 (half 1); the copies for
  // round r + 1 are issued right after the barrier that opens round r, into
  // the stages round r - 1 used (every wave has passed that barrier, so
  // every wave is done with them).
  const int rounds = (ccount + 1) >> 1;
  const int mine = half;                 // local chunk of round 0 for this wave
  u32x4_t bcur[4], bnext[4];
  if (mine < ccount) {
    issue(cb + mine, mine);
    load_b(cb + mine, bcur);
  }
  for (int r = 0; r < rounds; ++r) {
    const int i = 2 * r + mine;          // this wave's local chunk of round r
    wait_all_then_barrier();
    const bool more = i + 2 < ccount;
    if (more) {
      issue(cb + i + 2, (i + 2) & 3);
      load_b(cb + i + 2, bnext);
    }
    if (i < ccount) run_chunk(s_ring + (i & 3) * kStageBytes, bcur);
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) bcur[s] = bnext[s];
    }
  }
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[fm][fn][q] = __builtin_fmaf(sc[fn], P[fm][fn][q], acc[fm][fn][q]);

  // ---- half 1 hands its accumulators to half 0 (LDS, lane-major so the
  // accesses are contiguous: element e of lane l at (qw, e, l)) ----
  wait_all_then_barrier();
  float *s_acc = (float *)s_ring;
  if (half == 1) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) s_acc[((qw * 64 + (fm * 16 + fn * 4 + q)) * 64) + lane] = acc[fm][fn][q];
  }
  wait_all_then_barrier();
  if (half == 1) return;
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[fm][fn][q] += s_acc[((qw * 64 + (fm * 16 + fn * 4 + q)) * 64) + lane];

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
  if (ncol >= a.N) return;   // N % 8 == 0: a lane's 4 columns are all in or all out
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row_base + 16 * fm + r;
      if (row >= a.M) continue;
      const size_t o = (size_t)row * a.N + ncol;
      if constexpr (OF == O_BF16) {
        *(u32x2_t *)((uint16_t *)a.out + o) =
            (u32x2_t){pack_bf16x2(acc[fm][0][r], acc[fm][1][r]), pack_bf16x2(acc[fm][2][r], acc[fm][3][r])};
      } else {
        *(f32x4_t *)((float *)a.out + o) = (f32x4_t){acc[fm][0][r], acc[fm][1][r], acc[fm][2][r], acc[fm][3][r]};
      }
    }
}

// ---------------------------------------------------------------------------
// Activation sums: asum[g][m] = sum_{k in group g} a[m][k] (groups of 128),
// for m < M; row stride Mp. One wave per row: lane l reads 16 bytes of each
// 1 KiB block of the row (block j covers groups 4j .. 4j+3; lanes 16i .. 16i+15
// hold group 4j + i), adds its 8 values in k order, and the 16 lanes of a
// group (one DPP row) combine in a fixed order of row rotations. Up to 8
// blocks are loaded before any is added, so every lane keeps 8 loads in
// flight.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void asum_kernel(const uint16_t *__restrict__ A, float *__restrict__ asum, int M,
                                                  int K, int Mp) {
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
      if (g < ngroups && (lane & 15) == 0) asum[(size_t)g * Mp + m] = s;
    }
  }
}

template <int OF, bool ZP>
static hipError_t go(const GemmArgs &a, dim3 grid, hipStream_t st) {
  gemm_kernel<OF, ZP><<<grid, kGemmThreads, 0, st>>>(a);
  return hipGetLastError();
}

// The dispatcher sends only G == 128, K % 128 == 0, N % 8 == 0 here.
hipError_t launch_gemm(int ofmt, bool zp, int G, const GemmArgs &a, dim3 grid, hipStream_t st) {
  if (G != 128 || a.K % kGemmKC != 0 || a.N % 8 != 0) return hipErrorInvalidValue;
  asum_kernel<<<(a.M + 3) / 4, 256, 0, st>>>(a.A, a.asum, a.M, a.K, a.Mp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ofmt == O_BF16) return zp ? go<O_BF16, true>(a, grid, st) : go<O_BF16, false>(a, grid, st);
  return zp ? go<O_F32, true>(a, grid, st) : go<O_F32, false>(a, grid, st);
}

}  // namespace qg
