// FP8 (E4M3) W8A8 GEMM, per-token x per-channel scaling, for products large
// enough to give every compute unit a 256 x 256 tile: the same computation
// as the 128 x 128 kernel (page "quantization-and-fused-kernels"
// (arganzheng.life), section 四.2: float32 sum over K of a w, then the weight
// scale, then the activation scale), with twice the products per byte
// copied into LDS.
//
//   - Workgroup tile 256 x 256, 4 waves (one per SIMD) of 128 x 128 = 4 x 4
//     tiles of v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales), 256 float32
//     accumulators per lane (they live in the accumulation registers; this
//     file is built without the flag that forces matrix results into
//     ordinary VGPRs).
//   - K advances in chunks of 128 bytes, each taken as two half-steps of 64
//     (one instruction per tile per half-step), in the same K order as the
//     128 x 128 kernel, so the two kernels give bitwise equal results.
//   - A chunk's operand tiles (256 rows x 128 bytes each, 64 KiB) are copied
//     by buffer loads straight into LDS, whole 128-byte rows (cache lines) per
//     request, into a ring of 2 stages: a chunk's copies are issued as soon
//     as its stage is free, two half-steps before it is needed. A half-step's
//     fragments are read into registers during the previous half-step,
//     between its matrix instructions (two register sets), so a stage is free
//     once its second half-step's fragments are in registers.
//   - The 16-byte pieces of a row are XOR-swizzled with bits 1..4 of the row,
//     so that the 16 lanes of a fragment read (16 rows, one piece each, for
//     the activation rows and for the weight rows in the instruction's row
//     order) hit 16 different 4-bank groups.
//   - A lane holds one output row and 16 adjacent output columns of each tile
//     (weight rows in the order 16 ((i / 4) % 2) + 4 (i / 8) + i % 4); the
//     epilogue writes them with two 16-byte stores.
#include "common.h"

#include <type_traits>

namespace qg {

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_b;
typedef __attribute__((ext_vector_type(8))) int i32x8_b;
typedef __attribute__((ext_vector_type(16))) float f32x16_b;
typedef __attribute__((ext_vector_type(4))) float f32x4_b;
typedef __attribute__((ext_vector_type(2))) float f32x2_b;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_b;
typedef __attribute__((address_space(3))) void lds_void_b;

constexpr int kBufWord3 = 0x00020000;    // raw buffer: 32-bit data, no swizzle
constexpr int kDead = (int)0x80000000u;  // out-of-range buffer offset: zero result, no access
constexpr int kBT = 256;                 // tile rows (activations) and columns (weights)
constexpr int kBK = 128;                 // K bytes per chunk
constexpr int kBOp = kBT * kBK;          // 32 KiB: one operand's chunk
constexpr int kBStage = 2 * kBOp;        // activations, then weights
constexpr int kBStages = 2;

// physical 16-byte slot of logical piece p (0..7) of a 128-byte row: p ^ swz(row)
__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) | ((((row >> 3) ^ (row >> 4)) & 1) << 2); }

}  // namespace

__global__ __launch_bounds__(256, 1) void fp8_gemm_big_kernel(const uint8_t *__restrict__ Aq,
                                                             const float *__restrict__ a_scale,
                                                             const uint8_t *__restrict__ Wq,
                                                             const float *__restrict__ w_scale,
                                                             uint16_t *__restrict__ out, int M, int N, int K) {
  __shared__ __align__(16) unsigned char s_ring[kBStages * kBStage];   // 128 KiB
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wr = wave >> 1, wc = wave & 1;
  // Tile order: workgroups go to the 8 dies (XCDs, each with its own L2) in
  // turn by launch order; the launch order is remapped so that each die gets
  // a compact block of tiles (4 row tiles by tiles / 32 columns) whose
  // activation rows and weight columns its L2 then serves.
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
  const int m0 = ty * kBT, n0 = tx * kBT;
  const int nchunks = K / kBK;

  // operand resources start at the tile's first row; rows past M (or N) fall
  // outside num_records and read zeros
  const int a_rows = M - m0 < kBT ? M - m0 : kBT;
  const int b_rows = N - n0 < kBT ? N - n0 : kBT;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(Aq + (size_t)m0 * K), (short)0, a_rows * K, kBufWord3);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(Wq + (size_t)n0 * K), (short)0, b_rows * K, kBufWord3);

  // Copy j (0..7) of wave w moves LDS bytes 1 KiB * (4 j + w) of an operand
  // chunk: rows 8 (4 j + w) + lane / 8, physical slot lane % 8 holding
  // logical piece (lane % 8) ^ swz(row); swz(row) is the same for every j.
  const int crow = 8 * wave + (lane >> 3);
  const int c_voff = crow * K + 16 * ((lane & 7) ^ swz(crow));   // + 32 K j; + 128 chunk (SGPR)
  // copy c of a chunk: c = 0..7 activations, 8..15 weights (j = c % 8)
  auto copy_one = [&](int chunk, int stage, int c, int dead) {
    unsigned char *sb = s_ring + stage * kBStage + (c >> 3) * kBOp + 1024 * (4 * (c & 7) + wave);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c < 8 ? a_rsrc : b_rsrc, (lds_void_b *)sb, 16,
                                             (c_voff + 32 * K * (c & 7)) | dead, chunk * kBK, 0, 0);
  };

  // Fragment of a 32-row tile for half-step e of a chunk: row l32 of the
  // tile (activations) or row wperm (weights), the 32 bytes
  // k = 64 e + 32 (lane / 32) .. +31, i.e. logical pieces 4 e + 2 hl and the
  // next. Tiles 32 rows apart have the same swizzle.
  const int wperm = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
  const int arow = 128 * wr + l32, brow = 128 * wc + wperm;
  int a_off[2][2], b_off[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      a_off[e][q] = arow * kBK + 16 * ((4 * e + 2 * hl + q) ^ swz(arow));
      b_off[e][q] = kBOp + brow * kBK + 16 * ((4 * e + 2 * hl + q) ^ swz(brow));
    }

  struct Frags {
    i32x8_b a[4], b[4];
  };
  auto frag = [&](const unsigned char *sb, int o0, int o1, int t) {
    const u32x4_b lo = *(const u32x4_b *)(sb + o0 + t * 32 * kBK);
    const u32x4_b hi = *(const u32x4_b *)(sb + o1 + t * 32 * kBK);
    return (i32x8_b){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  f32x16_b acc[4][4];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[fm][fn][e] = 0.f;

  // One half-step: 16 slots, each one matrix instruction on C (tile q / 4,
  // q % 4), then the next half-step's fragment reads from stage `sbn`, half
  // `en`, in the slots kReadAt names (early: they have landed by the next
  // wait), and, when `copies`, one copy of chunk `cn` into stage `stc` per
  // slot: the weights' 8 first, then the activations' (the weights stream
  // from HBM, the activations are mostly served by the caches; weights
  // first measured about 2% faster at M = N = K = 4096). With one wave per
  // SIMD the order is kept as written, so that no wait or queue stall sits
  // between two matrix instructions.
  constexpr int kReadAt[16] = {0, 4, 1, 5, 2, 6, 3, 7, -1, -1, -1, -1, -1, -1, -1, -1};   // fragment (b: + 4)
  auto half = [&](const Frags &C, Frags &Nx, const unsigned char *sbn, auto en_c, bool copies, int cn, int stc,
                  int dead) __attribute__((always_inline)) {
    constexpr int en = decltype(en_c)::value;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int fm = q >> 2, fn = q & 3;
      acc[fm][fn] =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(C.b[fn], C.a[fm], acc[fm][fn], 0, 0, 0, 127, 0, 127);
      const int f = kReadAt[q];
      if (f >= 4) Nx.b[f - 4] = frag(sbn, b_off[en][0], b_off[en][1], f - 4);
      else if (f >= 0) Nx.a[f] = frag(sbn, a_off[en][0], a_off[en][1], f);
      if (copies) copy_one(cn, stc, q < 8 ? 8 + q : q - 8, dead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Chunk c: half-step 2c computes on the fragments read during the previous
  // half-step and reads half-step 2c + 1's (same stage); half-step 2c + 1
  // first waits until chunk c + 1 is in LDS (no copy is then in flight) and
  // every wave has read chunk c's stage (its last fragments are in
  // registers), then issues chunk c + 2's copies into that stage and reads
  // half-step 2c + 2's fragments from chunk c + 1's stage.
  for (int p = 0; p < kBStages; ++p)
#pragma unroll
    for (int c = 0; c < 16; ++c) copy_one(p, p, c, p < nchunks ? 0 : kDead);
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  Frags fx, fy;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    fx.a[t] = frag(s_ring, a_off[0][0], a_off[0][1], t);
    fx.b[t] = frag(s_ring, b_off[0][0], b_off[0][1], t);
  }
  for (int c = 0; c < nchunks; ++c) {
    const int st = c & 1;
    half(fx, fy, s_ring + st * kBStage, std::integral_constant<int, 1>{}, false, 0, 0, 0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    half(fy, fx, s_ring + (st ^ 1) * kBStage, std::integral_constant<int, 0>{}, true, c + 2, st,
         c + 2 < nchunks ? 0 : kDead);
  }
  // the copies past the last chunk (zeros into stages no one reads) land
  // before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: tile (fm, fn) element e is row 128 wr + 32 fm + l32,
  // column 128 wc + 32 fn + 16 (lane / 32) + e; out = a_scale * (w_scale *
  // sum) ----
  float as[4];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
    const int m = m0 + 128 * wr + 32 * fm + l32;
    as[fm] = m < M ? a_scale[m] : 0.f;
  }
#pragma unroll
  for (int fn = 0; fn < 4; ++fn) {
    const int n = n0 + 128 * wc + 32 * fn + 16 * hl;
    if (n >= N) continue;
    float ws[16];
    if (n + 16 <= N) {   // 64-byte aligned: n is a multiple of 16
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4_b w4 = *(const f32x4_b *)(w_scale + n + 4 * e4);
#pragma unroll
        for (int e = 0; e < 4; ++e) ws[4 * e4 + e] = w4[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) ws[e] = n + e < N ? w_scale[n + e] : 0.f;
    }
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const int m = m0 + 128 * wr + 32 * fm + l32;
      if (m >= M) continue;
      uint32_t b[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const f32x2_b pr = {as[fm] * (ws[2 * e2] * acc[fm][fn][2 * e2]),
                            as[fm] * (ws[2 * e2 + 1] * acc[fm][fn][2 * e2 + 1])};
        b[e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_b));
      }
      uint16_t *o = out + (size_t)m * N + n;
      if (n + 16 <= N && ((((size_t)m * N + n) & 7) == 0)) {   // 16-byte aligned: two stores
        *(u32x4_b *)o = (u32x4_b){b[0], b[1], b[2], b[3]};
        *(u32x4_b *)(o + 8) = (u32x4_b){b[4], b[5], b[6], b[7]};
      } else {   // the ragged end of a row, or N % 8 != 0
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (n + e < N) o[e] = (uint16_t)(b[e / 2] >> (16 * (e & 1)));
      }
    }
  }
}

bool fp8_big_tiles(int M, int N, int K, int cus) {
  const long long tiles = (long long)((M + kBT - 1) / kBT) * ((N + kBT - 1) / kBT);
  return tiles >= cus && (long long)kBT * K + kBK <= 0x7fffffffLL;
}

hipError_t launch_fp8_gemm_big(const uint8_t *Aq, const float *a_scale, const uint8_t *Wq, const float *w_scale,
                               uint16_t *out, int M, int N, int K, hipStream_t st) {
  const dim3 grid((N + kBT - 1) / kBT, (M + kBT - 1) / kBT);
  fp8_gemm_big_kernel<<<grid, 256, 0, st>>>(Aq, a_scale, Wq, w_scale, out, M, N, K);
  return hipGetLastError();
}

}  // namespace qg
