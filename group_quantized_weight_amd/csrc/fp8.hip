// FP8 (E4M3) W8A8 path: dynamic activation quantization and the FP8 GEMM,
// the variant the page "quantization-and-fused-kernels" (arganzheng.life)
// contrasts with W4A16 in section 四: weights and activations both in FP8,
// products accumulated in float32 on the matrix cores, scales either outside
// the K sum (per token x per output channel, section 四.2) or per 128-wide K
// block inside it, promoted into a float32 accumulator once per block
// (section 四.3).
//
// E4M3 here is the OCP "fn" variant (bias 7, largest finite 448, no
// infinities), the format gfx950's FP8 conversions and matrix instructions
// use.
#include "common.h"

namespace qg {

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_v;
typedef __attribute__((ext_vector_type(8))) int i32x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(2))) float f32x2_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_v;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBufWord3 = 0x00020000;   // raw buffer: 32-bit data, no swizzle
constexpr int kDead = (int)0x80000000u; // out-of-range buffer offset: zero result, no access

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// float32 -> E4M3 after the saturation of the page's conversion (section
// 二.3: values are first clamped to +-448), rounded to nearest even by
// v_cvt_pk_fp8_f32. Returns the two codes in the low 16 bits.
__device__ __forceinline__ uint32_t to_fp8x2(float x0, float x1) {
  x0 = fminf(fmaxf(x0, -448.f), 448.f);
  x1 = fminf(fmaxf(x1, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xFFFFu;
}

// Division of bf16 values by one scale, as the E4M3 conversion needs it.
// For a finite scale sc >= 2^-100 it takes r = RN(1 / sc) once and, per
// value, q = RN(x r) and RN(q + RN(x - sc q) r) (Markstein's correction
// step, the residual exact by fma): 3 instructions instead of the ~10 of a
// correctly rounded division. That quotient can differ from RN(x / sc) in
// the last place, but only for quotients far below E4M3's smallest
// subnormal, so the codes are those of the correctly rounded quotient
// (checked over every bf16 x and every scale amax / 448 >= 2^-100, amax a
// bf16 magnitude: tests/test_fp8_division.py). Other scales divide.
struct ScaleDiv {
  float sc, r;
  bool fast;
  __device__ explicit ScaleDiv(float s) : sc(s), r(1.0f / s), fast(s >= 0x1p-100f && s < __builtin_inff()) {}
  __device__ float operator()(float x) const {
    if (!fast) return x / sc;
    const float q = x * r;
    return __builtin_fmaf(__builtin_fmaf(-sc, q, x), r, q);
  }
};

// 8 bf16 values (one 16-byte load) divided by the scale -> 8 codes (8 bytes).
__device__ __forceinline__ uint2 quant8(u32x4_v v, const ScaleDiv &d) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = to_fp8x2(d(bf16_lo(v[j])), d(bf16_hi(v[j])));
  return make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
}

__device__ __forceinline__ float absmax8(u32x4_v v) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[j])), fabsf(bf16_hi(v[j]))));
  return m;
}

}  // namespace

// ---------------------------------------------------------------------------
// Dynamic quantization (section 四.5): scale = max|a| / 448 (1 for an all-zero
// row or block), code = E4M3(clamp(a / scale, -448, 448)), all in float32
// with the division correctly rounded.
// ---------------------------------------------------------------------------

// One 128-element block per 16 lanes (8 values per lane); the 16 lanes
// combine their maxima with lane exchanges (max is exact in any order).
__global__ __launch_bounds__(256) void fp8_quant_block_kernel(const uint16_t *__restrict__ A, uint8_t *__restrict__ Aq,
                                                             float *__restrict__ a_scale, size_t total) {
  const size_t e = 8 * ((size_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (e >= total) return;  // total % 128 == 0: a block's 16 lanes are all in range or all out
  const u32x4_v v = *(const u32x4_v *)(A + e);
  float amax = absmax8(v);
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  *(uint2 *)(Aq + e) = quant8(v, ScaleDiv(sc));
  if ((threadIdx.x & 15) == 0) a_scale[e / 128] = sc;
}

// Long rows (K > 8192), one workgroup per row (per-token scale): the row's
// maximum over the workgroup (lane exchanges, then LDS), then a second pass
// over the row.
__global__ __launch_bounds__(256) void fp8_quant_row_kernel(const uint16_t *__restrict__ A, uint8_t *__restrict__ Aq,
                                                           float *__restrict__ a_scale, int K) {
  __shared__ float s_max[4];
  const uint16_t *row = A + (size_t)blockIdx.x * K;
  uint8_t *qrow = Aq + (size_t)blockIdx.x * K;
  float amax = 0.f;
  for (int k = 8 * threadIdx.x; k < K; k += 8 * 256) amax = fmaxf(amax, absmax8(*(const u32x4_v *)(row + k)));
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  const ScaleDiv d(sc);
  for (int k = 8 * threadIdx.x; k < K; k += 8 * 256) *(uint2 *)(qrow + k) = quant8(*(const u32x4_v *)(row + k), d);
  if (threadIdx.x == 0) a_scale[blockIdx.x] = sc;
}

// Rows of up to 512 NCH values: one wave per row (4 rows per workgroup), the
// row held in registers (NCH 16-byte pieces per lane), so it is read once;
// the wave's maximum by lane exchanges.
template <int NCH>
__global__ __launch_bounds__(256) void fp8_quant_row_wave_kernel(const uint16_t *__restrict__ A,
                                                                uint8_t *__restrict__ Aq,
                                                                float *__restrict__ a_scale, int M, int K) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;   // whole waves: every lane of a wave has the same row
  const uint16_t *src = A + (size_t)row * K;
  u32x4_v v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int k = 8 * (lane + 64 * c);
    v[c] = k < K ? *(const u32x4_v *)(src + k) : (u32x4_v){0, 0, 0, 0};
  }
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) amax = fmaxf(amax, absmax8(v[c]));
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  uint8_t *dst = Aq + (size_t)row * K;
  const ScaleDiv d(sc);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int k = 8 * (lane + 64 * c);
    if (k < K) *(uint2 *)(dst + k) = quant8(v[c], d);
  }
  if (lane == 0) a_scale[row] = sc;
}

hipError_t launch_fp8_quant(const uint16_t *A, uint8_t *Aq, float *a_scale, int M, int K, int block,
                            hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (block == 128) {
    const size_t total = (size_t)M * K;
    fp8_quant_block_kernel<<<(unsigned)((total / 8 + 255) / 256), 256, 0, st>>>(A, Aq, a_scale, total);
  } else if (K <= 512 * 16) {
    const dim3 grid((M + 3) / 4);
    const int nch = (K + 511) / 512;
    if (nch <= 2)
      fp8_quant_row_wave_kernel<2><<<grid, 256, 0, st>>>(A, Aq, a_scale, M, K);
    else if (nch <= 4)
      fp8_quant_row_wave_kernel<4><<<grid, 256, 0, st>>>(A, Aq, a_scale, M, K);
    else if (nch <= 8)
      fp8_quant_row_wave_kernel<8><<<grid, 256, 0, st>>>(A, Aq, a_scale, M, K);
    else
      fp8_quant_row_wave_kernel<16><<<grid, 256, 0, st>>>(A, Aq, a_scale, M, K);
  } else {
    fp8_quant_row_kernel<<<M, 256, 0, st>>>(A, Aq, a_scale, K);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP8 GEMM: out[m][n] (bf16) from Aq [M][K] and Wq [N][K] (E4M3 codes).
//   per-token scaling:  out = a_scale[m] * (w_scale[n] * sum_k a w)  (the
//                       epilogue order of section 四.2: weight scale first)
//   blockwise scaling:  out = sum_b (a_scale[m][b] * w_scale[n/128][b]) * P_b,
//                       P_b = sum_{k in block b} a w, promoted in float32 per
//                       block (section 四.3); a_scale [M][K/128],
//                       w_scale [N/128][K/128].
//
// Workgroup tile 128 x 128, 4 waves (2 x 2), each 64 x 64 = 2 x 2 tiles of
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, float32 accumulate), two
// instructions per tile per 128-wide K step (one scale block). Against the
// 16x16x128 form (4 x 4 tiles, one instruction each) this issues half the
// matrix instructions for the same work, with the same LDS fragment reads.
// The K step's operand tiles (128 rows x 128 bytes each) are copied by buffer
// loads straight into LDS, into a ring of STAGES stages: 3 (two steps in
// flight) when the grid is about one workgroup per compute unit, 2 (67 KiB,
// so two workgroups share a compute unit and hide each other's waits) when
// there are at least two tiles per compute unit (measured on MI355X: M = 4096,
// K = N = 4096 per token 116 -> 85 us; M = 1024 prefers 3 stages, 32 vs
// 38 us). The 16-byte pieces of a row are XOR-swizzled with the row index
// (mod 8), so the fragment reads of 8 consecutive rows hit 8 different bank
// groups. A lane's fragment for half-step h (k = 64 h .. 64 h + 63) is the
// 32 consecutive bytes k = 64 h + 32 (lane / 32) .. +31 of one row, the same
// k for both operands. The weight fragment is the instruction's first
// operand and the activation fragment its second, so each tile is computed
// transposed: a lane holds one output row (activation row lane % 32) and 16
// output columns. Instruction row i of a weight tile is weight row
// 16 ((i / 4) % 2) + 4 (i / 8) + i % 4, which makes a lane's 16 columns the
// adjacent 16 (lane / 32) .. +15 of the tile: the epilogue scales them (one
// activation scale per row, 16 consecutive weight scales) and writes them
// with two 16-byte stores.
// ---------------------------------------------------------------------------
constexpr int kF8Tile = 128;
constexpr int kF8Row = 128;                       // bytes per operand row per K step
constexpr int kF8OpBytes = kF8Tile * kF8Row;      // 16 KiB
constexpr int kF8Stage = 2 * kF8OpBytes + 512;    // A, B, and the block's 128 activation scales

typedef __attribute__((ext_vector_type(16))) float f32x16_v;

template <bool BLOCKWISE, int STAGES>
__global__ __launch_bounds__(256) void fp8_gemm_kernel(const uint8_t *__restrict__ Aq, const float *__restrict__ a_scale,
                                                      const uint8_t *__restrict__ Wq, const float *__restrict__ w_scale,
                                                      uint16_t *__restrict__ out, float *__restrict__ partial, int M,
                                                      int N, int K, int nsplit, int Np) {
  static_assert(STAGES == 2 || STAGES == 3, "ring depth");
  __shared__ __align__(16) unsigned char s_ring[STAGES * kF8Stage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wr = wave >> 1, wc = wave & 1;
  const int m0 = blockIdx.y * kF8Tile, n0 = blockIdx.x * kF8Tile;
  const int nsteps = K / 128;
  // K-slice blockIdx.z of nsplit: steps s0 .. s0 + cnt - 1
  int s0, cnt;
  split_range(nsteps, nsplit, blockIdx.z, s0, cnt);

  // operand resources start at the tile's first row; rows past M (or N) fall
  // outside num_records and read zeros
  const int a_rows = M - m0 < kF8Tile ? M - m0 : kF8Tile;
  const int b_rows = N - n0 < kF8Tile ? N - n0 : kF8Tile;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(Aq + (size_t)m0 * K), (short)0, a_rows * K, kBufWord3);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(Wq + (size_t)n0 * K), (short)0, b_rows * K, kBufWord3);
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(BLOCKWISE ? a_scale + (size_t)m0 * nsteps : a_scale), (short)0, BLOCKWISE ? a_rows * nsteps * 4 : 0,
      kBufWord3);

  // Copy j (0..3) of wave w moves LDS bytes 1 KiB * (4 j + w) of an operand
  // tile: piece p = 64 (4 j + w) + lane of 16 bytes, row p / 8, physical slot
  // p % 8 = lane % 8 holding logical piece (lane % 8) ^ (row % 8).
  const int crow0 = 8 * wave + (lane >> 3);                      // + 32 j
  const int cpiece = (lane & 7) ^ (crow0 & 7);
  const int c_voff = crow0 * K + 16 * cpiece;                     // + 32 K j, + 128 step (SGPR)
  auto copy_step = [&](int step, int stage, int dead) {
    unsigned char *sb = s_ring + stage * kF8Stage;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void *)(sb + 1024 * (4 * j + wave)), 16,
                                               (c_voff + 32 * K * j) | dead, step * 128, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_void *)(sb + kF8OpBytes + 1024 * (4 * j + wave)), 16,
                                               (c_voff + 32 * K * j) | dead, step * 128, 0, 0);
    }
    if constexpr (BLOCKWISE) {
      // the step's 128 activation scales a_scale[m0 + r][step], 4 bytes per
      // lane, by waves 0 and 1 (issued last: waiting for the 8 operand copies
      // of a later step also waits for this one)
      if (wave < 2) {
        const int r = 64 * wave + lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(q_rsrc, (lds_void *)(sb + 2 * kF8OpBytes + 256 * wave), 4,
                                                 ((r * nsteps + step) * 4) | dead, 0, 0, 0);
      }
    }
  };
  // At the top of step i at most the next step's copies may be in flight
  // (3 stages): 8 operand copies per wave (waves 0 and 1 add one scale copy
  // after them, which vmcnt(8) then also waits for); with 2 stages none.
  constexpr int kInFlight = STAGES == 3 ? 8 : 0;

  // 32 bytes of one row: pieces 4 h + 2 (lane / 32) and the next
  auto frag = [&](const unsigned char *op, int row, int h) {
    const int p = 4 * h + 2 * hl;
    const u32x4_v lo = *(const u32x4_v *)(op + row * kF8Row + 16 * (p ^ (row & 7)));
    const u32x4_v hi = *(const u32x4_v *)(op + row * kF8Row + 16 * ((p + 1) ^ (row & 7)));
    return (i32x8_v){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // this lane's rows: activation row 64 wr + 32 fm + l32 of tile fm; weight
  // row 64 wc + 32 fn + wperm of tile fn
  const int wperm = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);

  f32x16_v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  struct Frags {
    i32x8_v a[2][2], b[2][2];   // [tile][half-step]
  };
  auto read_step = [&](int step, Frags &F) {
    const unsigned char *sb = s_ring + (step % STAGES) * kF8Stage;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        F.a[f][h] = frag(sb, 64 * wr + 32 * f + l32, h);
        F.b[f][h] = frag(sb + kF8OpBytes, 64 * wc + 32 * f + wperm, h);
      }
  };

  if constexpr (!BLOCKWISE) {
    // Per token: the fragments of step i + 1 are read from LDS while the
    // MFMAs of step i run, alternating one MFMA and two LDS reads (two
    // register sets, so no copies between them). This needs step i + 1 in
    // LDS at the top of step i, so the ring takes step i + STAGES into the
    // stage step i used (read into registers during step i - 1).
    auto step = [&](int i, const Frags &C, Frags &Nx) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(8 * (STAGES - 2)) : "memory");
      const int nx = i + STAGES;
      copy_step(s0 + nx, i % STAGES, nx < cnt ? 0 : kDead);
      read_step(i + 1, Nx);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int fn = 0; fn < 2; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(C.b[fn][h], C.a[fm][h], acc[fm][fn], 0, 0,
                                                                          0, 127, 0, 127);
      __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    };
#pragma unroll
    for (int p = 0; p < STAGES; ++p) copy_step(s0 + p, p, cnt > p ? 0 : kDead);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(8 * (STAGES - 1)) : "memory");
    Frags f0, f1;
    read_step(0, f0);
    for (int i = 0; i < cnt; i += 2) {
      step(i, f0, f1);
      if (i + 1 < cnt) step(i + 1, f1, f0);
    }
  } else {
    copy_step(s0, 0, cnt > 0 ? 0 : kDead);
    if constexpr (STAGES == 3) copy_step(s0 + 1, 1, cnt > 1 ? 0 : kDead);
    for (int i = 0; i < cnt; ++i) {
      // this step's copies are done when at most the next step's remain in flight
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kInFlight) : "memory");
      // every wave is past step i - 1: its stage takes step i + STAGES - 1
      const int nx = i + STAGES - 1;
      copy_step(s0 + nx, nx % STAGES, nx < cnt ? 0 : kDead);
      const unsigned char *sb = s_ring + (i % STAGES) * kF8Stage;
      Frags F;
      read_step(i, F);
      const float sb_w = w_scale[(size_t)(n0 / 128) * nsteps + s0 + i];   // one per workgroup tile and block
      const float *sa = (const float *)(sb + 2 * kF8OpBytes);
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) {
        const float s1 = sa[64 * wr + 32 * fm + l32] * sb_w;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
          f32x16_v pz;
#pragma unroll
          for (int e = 0; e < 16; ++e) pz[e] = 0.f;
          f32x16_v p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[fn][0], F.a[fm][0], pz, 0, 0, 0, 127, 0,
                                                                       127);
          p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[fn][1], F.a[fm][1], p, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[fm][fn][e] = __builtin_fmaf(s1, p[e], acc[fm][fn][e]);
        }
      }
    }
  }

  // ---- epilogue: tile (fm, fn) element e is row 64 wr + 32 fm + l32, column
  // 64 wc + 32 fn + 16 (lane / 32) + e ----
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    const int m = m0 + 64 * wr + 32 * fm + l32;
    if (m >= M) continue;
    const float as = BLOCKWISE ? 1.f : a_scale[m];
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
      const int n = n0 + 64 * wc + 32 * fn + 16 * hl;
      if (n >= N) continue;
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        v[e] = BLOCKWISE ? acc[fm][fn][e] : as * ((n + e < N ? w_scale[n + e] : 0.f) * acc[fm][fn][e]);
      if (nsplit > 1) {
        // the slice's scaled float32 partial (columns up to Np, a multiple of
        // 128); the reduce adds slices z = 0..nsplit-1
        float *pp = &partial[((size_t)blockIdx.z * M + m) * Np + n];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          *(f32x4_v *)(pp + 4 * e4) = (f32x4_v){v[4 * e4], v[4 * e4 + 1], v[4 * e4 + 2], v[4 * e4 + 3]};
        continue;
      }
      uint32_t b[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const f32x2_v pr = {v[2 * e2], v[2 * e2 + 1]};
        b[e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_v));
      }
      uint16_t *o = out + (size_t)m * N + n;
      if (n + 16 <= N && ((((size_t)m * N + n) & 7) == 0)) {   // 16-byte aligned: two stores
        *(u32x4_v *)o = (u32x4_v){b[0], b[1], b[2], b[3]};
        *(u32x4_v *)(o + 8) = (u32x4_v){b[4], b[5], b[6], b[7]};
      } else {   // the ragged end of a row, or N % 8 != 0
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (n + e < N) o[e] = (uint16_t)(b[e / 2] >> (16 * (e & 1)));
      }
    }
  }
}

template <bool BLOCKWISE>
static void go_fp8(int stages, dim3 grid, const uint8_t *Aq, const float *a_scale, const uint8_t *Wq,
                   const float *w_scale, uint16_t *out, float *partial, int M, int N, int K, int nsplit, int Np,
                   hipStream_t st) {
  if (stages == 2)
    fp8_gemm_kernel<BLOCKWISE, 2><<<grid, 256, 0, st>>>(Aq, a_scale, Wq, w_scale, out, partial, M, N, K, nsplit, Np);
  else
    fp8_gemm_kernel<BLOCKWISE, 3><<<grid, 256, 0, st>>>(Aq, a_scale, Wq, w_scale, out, partial, M, N, K, nsplit, Np);
}

// nsplit > 1: the K steps are split into nsplit slices (grid z) that write
// float32 partials [nsplit][M][Np] to `partial`, then the fixed-order reduce
// writes `out`.
hipError_t launch_fp8_gemm(int scaling, const uint8_t *Aq, const float *a_scale, const uint8_t *Wq,
                           const float *w_scale, uint16_t *out, float *partial, int M, int N, int K, int nsplit,
                           int Np, int cus, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (scaling == 0 && nsplit == 1 && fp8_big_tiles(M, N, K, cus))
    return launch_fp8_gemm_big(Aq, a_scale, Wq, w_scale, out, M, N, K, st);
  const dim3 grid((N + kF8Tile - 1) / kF8Tile, (M + kF8Tile - 1) / kF8Tile, nsplit);
  const int stages = (long long)grid.x * grid.y * nsplit >= 2LL * cus ? 2 : 3;
  if (scaling == 1)
    go_fp8<true>(stages, grid, Aq, a_scale, Wq, w_scale, out, partial, M, N, K, nsplit, Np, st);
  else
    go_fp8<false>(stages, grid, Aq, a_scale, Wq, w_scale, out, partial, M, N, K, nsplit, Np, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit <= 1) return e;
  return launch_reduce(O_BF16, partial, out, M, N, Np, nsplit, st);
}

}  // namespace qg
