// Small-M MFMA path of the group-quantized GEMM (bf16 activations, int4
// weights, bf16 scales, optional int4 zero-points, groups of 128), for the
// band of M where the product is still bound by the weight bytes but a
// vector-ALU GEMV runs out of arithmetic (the small-M specialisation of the
// page "quantization-and-fused-kernels" (arganzheng.life), section 三.3,
// item 6, and the roofline argument of its section 三.2).
//
// Structure: the weights stream once, as in the GEMV path, and the dot
// products run on v_mfma_f32_16x16x32_bf16 with M padded to MB blocks of 16
// rows:
//   - a workgroup (4 waves) covers one 64-column tile of the packed layout
//     and a K-slice of whole groups (slice z of nsplit, the z-split of the
//     page "04 · 分组量化 GEMM 内核" (developer.aliyun.com), section 3.3);
//     each wave takes a contiguous share of the slice's groups;
//   - per group, each lane loads 16 bytes of packed words per k-step (4
//     adjacent columns x 8 k; a wave reads 1 KiB of contiguous memory) and
//     turns each word into four bf16 pairs of the exact integers q - z:
//     each code goes into the mantissa of fp16 1024.0 (fp16 magic number,
//     section 二.4 of the first page), v_fma_mix_f32 widens each half to
//     float32 and subtracts 1024 + z (or, for the code one nibble higher,
//     scales by 1/16 and subtracts 64 + z), and v_cvt_pk_bf16_f32 packs two
//     results; every step is exact (|q - z| <= 15 needs 4 bits). MFMA column
//     j of tile f is physical column 4j + f of the 64-column tile;
//   - activation fragments are read from global memory as bf16, unchanged
//     (rows past M read as zeros); each product a * (q - z) is exact in the
//     MFMA's float32 accumulator, which sums the group's 128 of them;
//   - per group the scale is applied in float32: acc += s * P. No biased sum
//     is formed, so a column whose codes all equal its zero-point gives
//     exactly zero;
//   - the 4 waves' results are added in wave order (waves 1..3 through LDS),
//     then written to the output (nsplit == 1) or to float32 partials that a
//     second kernel adds in the order z = 0..nsplit-1.
// Grouped (MoE) mode: blockIdx.z is a block of 16 MB routed rows of one
// expert (the align step's sorted_ids); row i of the block gathers the
// activations of token sorted_ids[.] / topk (padding rows read zeros), the
// expert's weights, scales and zero-points are offset by its index, and the
// row is written to output row sorted_ids[.].
#include "common.h"

namespace qg {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_s;
typedef __attribute__((ext_vector_type(4))) float f32x4_s;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_s;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_s;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_s;
typedef __attribute__((ext_vector_type(2))) float f32x2_s;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_s;

constexpr int kWaves = 4;
constexpr int kBufWord3s = 0x00020000;
constexpr int kStreamPolicy = 2;    // non-temporal
// groups of weights in registers: kDepth - 1 in flight while one is computed
constexpr int kDepth = 2;

__device__ __forceinline__ uint32_t magic_pair() {  // fp16 1024.0 in both halves
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  f32x2_s v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_s));
}

// float32 1.0 in a register the compiler cannot see through, so that x * 1 +
// c stays one v_fma_mix_f32 instead of a conversion and an add
__device__ __forceinline__ float opaque_one() {
  float one;
  asm volatile("v_mov_b32 %0, 1.0" : "=v"(one));
  return one;
}

// The eight codes of a packed word (layout version 2: codes 2i and 2i + 1 at
// bits 4i and 4i + 16) as bf16 q - z, in k order. c0 = -(1024 + z), c1 =
// -(64 + z).
__device__ __forceinline__ bf16x8_s dequant(uint32_t w, uint32_t magic, float one, float c0, float c1) {
  const uint32_t t = w >> 8;
  const f16x2_s h0 = __builtin_bit_cast(f16x2_s, (w & 0x000F000Fu) | magic);  // 1024 + q0, 1024 + q1
  const f16x2_s h1 = __builtin_bit_cast(f16x2_s, (w & 0x00F000F0u) | magic);  // 1024 + 16 q2, 1024 + 16 q3
  const f16x2_s h2 = __builtin_bit_cast(f16x2_s, (t & 0x000F000Fu) | magic);  // q4, q5
  const f16x2_s h3 = __builtin_bit_cast(f16x2_s, (t & 0x00F000F0u) | magic);  // q6, q7
  u32x4_s x;
  x[0] = bf16x2_bits(__builtin_fmaf((float)h0[0], one, c0), __builtin_fmaf((float)h0[1], one, c0));
  x[1] = bf16x2_bits(__builtin_fmaf((float)h1[0], 0.0625f, c1), __builtin_fmaf((float)h1[1], 0.0625f, c1));
  x[2] = bf16x2_bits(__builtin_fmaf((float)h2[0], one, c0), __builtin_fmaf((float)h2[1], one, c0));
  x[3] = bf16x2_bits(__builtin_fmaf((float)h3[0], 0.0625f, c1), __builtin_fmaf((float)h3[1], 0.0625f, c1));
  return __builtin_bit_cast(bf16x8_s, x);
}

}  // namespace

template <int MB, int OF, bool ZP, bool GR>
__global__ __launch_bounds__(kWaves * kWave) void gemm_small_kernel(SmallArgs a) {
  extern __shared__ __align__(16) unsigned char s_red[];   // [waves - 1][MB * 16][64] float32

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int tile = blockIdx.x;
  const int z = blockIdx.y;
  const int R = a.K / 8;

  int gb, gcount, wg0, wgc;
  split_range(a.ngroups, a.nsplit, z, gb, gcount);
  split_range(gcount, kWaves, wave, wg0, wgc);

  // grouped row blocks: this block's expert, or nothing to do
  const uint32_t *Wb = a.W;
  const uint16_t *Sb = a.S;
  const uint32_t *Zb = a.Z;
  const int r0 = GR ? blockIdx.z * 16 * MB : 0;   // first routed row of the block
  if constexpr (GR) {
    if (r0 >= *a.num_post_pad) return;
    const int e = a.tile_experts[blockIdx.z];
    if (e < 0) return;
    Wb += (size_t)e * a.w_expert_words;
    Sb += (size_t)e * a.s_expert_elems;
    if constexpr (ZP) Zb += (size_t)e * a.z_expert_words;
  }
  // output row of block row `row` (>= M: not written)
  auto out_row = [&](int row) { return GR ? a.sorted_ids[r0 + row] : row; };

  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(Wb + (size_t)tile * R * kTileCols), (short)0, R * kTileCols * 4, kBufWord3s);
  const int w_voff = (lk * kTileCols + 4 * li) * 4;
  // scales and zero-points of the lane's 4 columns (N % 8 == 0: all 4 are
  // in or all out; a lane past N reads column 0's and its results are
  // dropped)
  const int ncol = tile * kTileCols + 4 * li;
  // canonical column of the scales and zero-points (a gate-up packed
  // product holds gate and up columns in the tile's halves)
  const int lcol = a.gu_d > 0 ? gate_up_column(ncol, a.gu_d, a.N) : ncol;
  const int scol = lcol < a.N ? lcol : 0;
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)Sb, (short)0, a.ngroups * a.N * 2, kBufWord3s);
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)Zb, (short)0, ZP ? a.ngroups * (a.N >> 3) * 4 : 0, kBufWord3s);
  // activations: fragment (fm, s) of lane (li, lk) is row 16 fm + li,
  // k = 128 g + 32 s + 8 lk .. +7; rows past M read zeros (range check of
  // the VGPR offset; the group offset in the SGPR operand stays in the row)
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.A, (short)0, (GR ? a.arows : a.M) * a.K * 2, kBufWord3s);
  // byte offset of each fragment row's activations (a padding row of a
  // grouped block gets an out-of-range offset: zeros, no memory access)
  int a_off[MB];
#pragma unroll
  for (int fm = 0; fm < MB; ++fm) {
    if constexpr (GR) {
      const int slot = out_row(16 * fm + li);
      a_off[fm] = slot < a.M ? (slot / a.topk) * a.K * 2 : (int)0x80000000u;
    } else {
      a_off[fm] = (16 * fm + li) * a.K * 2;
    }
  }

  const uint32_t magic = magic_pair();
  f32x4_s acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_s){0.f, 0.f, 0.f, 0.f};

  // One group's loads. The weights (from HBM) are issued kDepth - 1 groups
  // ahead of the computation, the activations, scales and zero-points (from
  // L2) one group ahead. A group past the wave's range re-reads the wave's
  // last one, or the matrix's last one for a wave without groups: valid
  // addresses, results unused.
  struct WeightLoads {
    u32x4_s w[4];
  };
  struct GroupLoads {
    bf16x8_s af[MB][4];
    u32x2_s sv;
    uint32_t zw;
  };
  auto group_of = [&](int gi) { return min(gb + wg0 + (gi < wgc ? gi : (wgc > 0 ? wgc - 1 : 0)), a.ngroups - 1); };
  auto issue_w = [&](int gi, WeightLoads &L) {
    const int g = group_of(gi);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      L.w[s] = __builtin_bit_cast(u32x4_s, __builtin_amdgcn_raw_buffer_load_b128(
                                               w_rsrc, w_voff, (g * 16 + 4 * s) * kTileCols * 4, kStreamPolicy));
  };
  auto issue = [&](int gi, GroupLoads &L) {
    const int g = group_of(gi);
#pragma unroll
    for (int fm = 0; fm < MB; ++fm)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        L.af[fm][s] = __builtin_bit_cast(
            bf16x8_s, __builtin_amdgcn_raw_buffer_load_b128(
                          a_rsrc, a_off[fm] | ((32 * s + 8 * lk) * 2), g * 256, 0));
    L.sv = __builtin_bit_cast(u32x2_s, __builtin_amdgcn_raw_buffer_load_b64(s_rsrc, scol * 2, g * a.N * 2, 0));
    L.zw = 0x88888888u;
    if constexpr (ZP)
      L.zw = __builtin_amdgcn_raw_buffer_load_b32(z_rsrc, (scol >> 3) * 4, g * (a.N >> 3) * 4, 0) >>
             (4 * (scol & 7));
  };
  const float one = opaque_one();
  auto compute = [&](const WeightLoads &W, const GroupLoads &L) {
    // column 4 li + fn of the lane: zero-point nibble fn of zw, scale sc[fn]
    float c0[4], c1[4];
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
      const float zf = (float)((L.zw >> (4 * fn)) & 0xFu);
      c0[fn] = -1024.f - zf;
      c1[fn] = -64.f - zf;
    }
    f32x4_s P[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) P[i][j] = (f32x4_s){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_s bfr[4];
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) bfr[fn] = dequant(W.w[s][fn], magic, one, c0[fn], c1[fn]);
#pragma unroll
      for (int fm = 0; fm < MB; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
          P[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(L.af[fm][s], bfr[fn], P[fm][fn], 0, 0, 0);
    }
    const float sc[4] = {__uint_as_float(L.sv[0] << 16), __uint_as_float(L.sv[0] & 0xFFFF0000u),
                         __uint_as_float(L.sv[1] << 16), __uint_as_float(L.sv[1] & 0xFFFF0000u)};
#pragma unroll
    for (int fm = 0; fm < MB; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[fm][fn][r] = __builtin_fmaf(sc[fn], P[fm][fn][r], acc[fm][fn][r]);
  };

  // group j sits in weight slot j % kDepth and activation slot j % 2; the
  // loop is unrolled so that every slot index is a constant (no register
  // copies, which would wait for loads in flight)
  constexpr int kUnroll = kDepth % 2 == 0 ? kDepth : 2 * kDepth;
  WeightLoads wr[kDepth];
  GroupLoads ar[2];
  // the loads in flight at the loop head are issued in the loop's own order
  // (weights of group j, activations of group j, weights of group j + 1,
  // ...), so the compiler's wait analysis sees the same state on both edges
  issue_w(0, wr[0]);
  issue(0, ar[0]);
#pragma unroll
  for (int d = 1; d < kDepth - 1; ++d) issue_w(d, wr[d]);
  __builtin_amdgcn_sched_barrier(0);
  // (the last group leaves both loops at once: a jump back to the loop head
  // from there would merge different sets of loads in flight, and the
  // compiler would then wait for all of them at the head)
  for (int gi = 0; gi < wgc; gi += kUnroll) {
#pragma unroll
    for (int d = 0; d < kUnroll; ++d) {
      if (gi + d >= wgc) goto groups_done;
      // activations first: the wait for a group's activations (counted in
      // issue order) then leaves the later groups' weights in flight
      issue(gi + d + 1, ar[(d + 1) % 2]);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(gi + d + kDepth - 1, wr[(d + kDepth - 1) % kDepth]);
      __builtin_amdgcn_sched_barrier(0);
      compute(wr[d % kDepth], ar[d % 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
groups_done:

  // ---- the 4 waves' results, added in wave order: waves 1..3 hand theirs
  // to wave 0 through LDS (element (16 fm + 4 lk + r, 4 li + fn) of wave w at
  // s_red[(((w - 1) * MB + fm) * 16 + 4 lk + r) * 64 + 4 li + fn]) ----
  float *red = (float *)s_red;
  if (wave > 0) {
#pragma unroll
    for (int fm = 0; fm < MB; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(f32x4_s *)&red[(((wave - 1) * MB + fm) * 16 + 4 * lk + r) * 64 + 4 * li] =
            (f32x4_s){acc[fm][0][r], acc[fm][1][r], acc[fm][2][r], acc[fm][3][r]};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if (wave > 0) return;

  const int n = tile * kTileCols + 4 * li;
#pragma unroll
  for (int fm = 0; fm < MB; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = out_row(16 * fm + 4 * lk + r);
      f32x4_s v = (f32x4_s){acc[fm][0][r], acc[fm][1][r], acc[fm][2][r], acc[fm][3][r]};
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += *(const f32x4_s *)&red[(((w - 1) * MB + fm) * 16 + 4 * lk + r) * 64 + 4 * li];
      if (a.gu_d > 0 && a.nsplit == 1) {
        // gate-up packed product: lane li < 8 holds gate columns 4 li .. +3
        // of the tile, lane li + 8 (same row) their up columns; SwiGLU's gate
        // step gives output columns 32 tile + 4 li .. +3 of [M][gu_d]
        f32x4_s u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = __shfl_xor(v[c], 8);
        const int nout = 32 * tile + 4 * li;
        if (row >= a.M || li >= 8 || nout >= a.gu_d) continue;
        f32x4_s g;
#pragma unroll
        for (int c = 0; c < 4; ++c) g[c] = silu_f32(v[c]) * u[c];
        const size_t o = (size_t)row * a.gu_d + nout;
        if constexpr (OF == O_BF16)
          *(u32x2_s *)((uint16_t *)a.out + o) = (u32x2_s){bf16x2_bits(g[0], g[1]), bf16x2_bits(g[2], g[3])};
        else
          *(f32x4_s *)((float *)a.out + o) = g;
        continue;
      }
      if (row >= a.M) continue;
      if (a.nsplit > 1) {
        *(f32x4_s *)&a.partial[((size_t)z * a.M + row) * a.Np + n] = v;
      } else if (n < a.N) {
        const size_t o = (size_t)row * a.N + n;
        if constexpr (OF == O_BF16)
          *(u32x2_s *)((uint16_t *)a.out + o) = (u32x2_s){bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
        else
          *(f32x4_s *)((float *)a.out + o) = v;
      }
    }
}

template <int MB, int OF, bool ZP, bool GR>
static hipError_t go_small(const SmallArgs &a, dim3 grid, hipStream_t st) {
  const size_t lds = (size_t)(kWaves - 1) * MB * 16 * 64 * 4;
  gemm_small_kernel<MB, OF, ZP, GR><<<grid, kWaves * kWave, lds, st>>>(a);
  return hipGetLastError();
}

template <int OF, bool ZP, bool GR>
static hipError_t go_small_mb(int mb, const SmallArgs &a, dim3 grid, hipStream_t st) {
  switch (mb) {
    case 1: return go_small<1, OF, ZP, GR>(a, grid, st);
    case 2: return go_small<2, OF, ZP, GR>(a, grid, st);
    case 3: return go_small<3, OF, ZP, GR>(a, grid, st);
    case 4: return go_small<4, OF, ZP, GR>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

// The dispatcher sends only bf16 activations, G == 128, N % 8 == 0 and
// M <= 64 here (mb = ceil(M / 16) row blocks of 16).
hipError_t launch_gemm_small(int ofmt, bool zp, int mb, const SmallArgs &a, dim3 grid, hipStream_t st) {
  if (a.N % 8 != 0 || a.K % 128 != 0 || mb < 1 || mb > 4 || a.M > 16 * mb) return hipErrorInvalidValue;
  if (ofmt == O_BF16)
    return zp ? go_small_mb<O_BF16, true, false>(mb, a, grid, st) : go_small_mb<O_BF16, false, false>(mb, a, grid, st);
  return zp ? go_small_mb<O_F32, true, false>(mb, a, grid, st) : go_small_mb<O_F32, false, false>(mb, a, grid, st);
}

// Grouped (MoE) blocks of 16 mb routed rows; grid (Np / 64, nsplit, row blocks).
hipError_t launch_gemm_small_grouped(int ofmt, bool zp, int mb, const SmallArgs &a, dim3 grid, hipStream_t st) {
  if (a.N % 8 != 0 || a.K % 128 != 0 || (mb != 1 && mb != 2 && mb != 4)) return hipErrorInvalidValue;
  if (ofmt == O_BF16)
    return zp ? go_small_mb<O_BF16, true, true>(mb, a, grid, st) : go_small_mb<O_BF16, false, true>(mb, a, grid, st);
  return zp ? go_small_mb<O_F32, true, true>(mb, a, grid, st) : go_small_mb<O_F32, false, true>(mb, a, grid, st);
}

}  // namespace qg
