// C ABI of the group-quantized GEMM (declared in include/qgemm.h):
// argument validation, dispatch by M, K-split sizing, workspace sizing and
// launches on the caller's stream. No device memory is allocated here and no
// call synchronizes the host.
//
// A call enqueues one kernel, or two when K is split: the split kernel writes
// float32 partials to the workspace and a reduction kernel adds them in the
// fixed order z = 0..nsplit-1 (the kernel boundary orders the two; no
// device-wide fences or atomics are used). The tiled MFMA path adds a
// pre-pass that writes the activations as fp16 (scaled by a power of two per
// row), the row exponents and float32 scales to the workspace. Precisions 7 and 8
// quantize float32 activations to int8 codes and per-group scales inside the
// int8 GEMV's prologue (into LDS, no extra launch) for M <= 4, and with a
// pre-pass into the workspace above that.
//
// Dispatch follows the roofline argument of the page
// "quantization-and-fused-kernels" (arganzheng.life), section 三.2: at small
// M the product is bound by the weight bytes, so the weights stream once:
// through the vector-ALU GEMV path at M = 1 (and for fp32 / int8 activations
// or groups of 32 up to M = 8), through the small-M MFMA path for bf16
// activations at 2 <= M <= 64 (measured faster than the GEMV from M = 2 and
// than the tiled GEMM up to M = 64); at larger M the product is bound by
// arithmetic and bf16 activations go to the tiled MFMA GEMM. The K-split (nsplit) and its fixed-order
// reduction follow the z-split of the page "04 · 分组量化 GEMM 内核"
// (developer.aliyun.com), section 3.3: a pure function of the shape and the
// device's compute-unit count, so repeated calls (and captured graphs) take
// the same partition and give bitwise identical results.
#include <limits.h>

#include <atomic>

#include "../../include/qgemm.h"
#include "common.h"

using namespace qg;

namespace {

struct Formats {
  int w, a, s, o;
  bool dq = false;  // float32 activations quantized to int8 per group inside the call
};

bool prec_formats(int prec, Formats &f) {
  switch (prec) {
    case QG_W4_A_BF16: f = {W4, A_BF16, S_BF16, O_BF16}; return true;
    case QG_W4_A_F32: f = {W4, A_F32, S_F32, O_F32}; return true;
    case QG_W8_A_F32: f = {W8, A_F32, S_F32, O_F32}; return true;
    case QG_W4_A_I8: f = {W4, A_I8, S_F32, O_F32}; return true;
    case QG_W8_A_I8: f = {W8, A_I8, S_F32, O_F32}; return true;
    case QG_W4_A_BF16_OF32: f = {W4, A_BF16, S_BF16, O_F32}; return true;
    case QG_W4_A_F32_DQ8: f = {W4, A_I8, S_F32, O_F32, true}; return true;
    case QG_W8_A_F32_DQ8: f = {W8, A_I8, S_F32, O_F32, true}; return true;
    default: return false;
  }
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device (cached); 256 (MI355X) when no device
// can be queried, so that planning also works on a host without a GPU.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// hipGetLastError reports the last error of any runtime call on this thread,
// and it stays pending until read. Each entry point reads and drops such an
// error, left by some earlier call that is not ours, right before its first
// launch, so that the check after its own launches sees only their errors.
// A fault of the device persists and is still reported.
void drop_pending_error() { (void)hipGetLastError(); }

size_t padded_cols(int N) { return ((size_t)N + kColAlign - 1) / kColAlign * kColAlign; }

constexpr size_t kPartialCap = 256ull << 20;  // bytes of float32 partials at most
constexpr int kSmallMaxM = 64;                // rows the small-M MFMA path takes (4 blocks of 16)
constexpr int kSmallI8MinM = 9;               // int8 activations: fewer rows stay on the vector-ALU GEMV
constexpr size_t kGemvLdsCap = 60 * 1024;     // dynamic LDS per workgroup (static LDS comes on top)
constexpr int kMoeMaxExperts = 1024;          // experts the align step's LDS counters hold
constexpr int kDqFuseMaxM = 4;                // in-call int8 quantization fused into the GEMV up to this M

struct Plan {
  int path = QG_PATH_GEMV;
  int nsplit = 1;
  int mb = 1, mblocks = 1;
  int tiles_x = 1, tiles_y = 1;
  int units = 1;          // groups (GEMV) or 128-k chunks (GEMM) along K
  size_t lds = 0;
  bool dq_fused = false;  // precisions 7, 8: quantized in the GEMV's prologue, or
  size_t codes = 0;       //   by a pre-pass into the workspace: bytes of int8 codes,
  size_t ascale = 0;      //   then of their float32 scales, at its start
  size_t prep = 0;        // MFMA path: bytes of the pre-pass's outputs (after the above)
  size_t ws = 0;
};

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// MFMA path: the pre-pass's fp16 activations [M][K], row exponents [M] and
// float32 scales [K/128][Np], each rounded up to 256 bytes.
size_t gemm_a16_bytes(int M, int K) { return round256((size_t)M * K * 2); }
size_t gemm_rexp_bytes(int M) { return round256((size_t)M * 4); }
size_t gemm_s32_bytes(int N, int K) { return round256((size_t)(K / kGemmKC) * padded_cols(N) * 4); }

size_t gemv_lds(const Formats &f, int mb, int G, int ngroups, int nsplit) {
  const int kpw = f.w == W4 ? 8 : 4;
  const int ab = f.a == A_I8 ? kpw : (f.a == A_BF16 ? 2 * kpw : 4 * kpw);
  const int gmax = (ngroups + nsplit - 1) / nsplit;
  const size_t rows = (size_t)gmax * (G / kpw);
  const size_t stage = ((size_t)mb * rows + 1) * (ab + 4);  // staged rows + a spare slot
  const size_t red = (size_t)gemv_waves(mb) * mb * kTileCols * 4;
  size_t b = stage > red ? stage : red;
  return (b + 15) / 16 * 16;
}

// Balanced split: the smallest nsplit giving the same per-slice count.
int balance(int units, int nsplit) {
  if (nsplit < 1) nsplit = 1;
  if (nsplit > units) nsplit = units;
  const int per = (units + nsplit - 1) / nsplit;
  return (units + per - 1) / per;
}

int make_plan(int M, int N, int K, int G, const Formats &f, int force_path, int force_nsplit, Plan &p) {
  const int cus = device_cus();
  const size_t Np = padded_cols(N);
  const bool gemm_ok = f.a == A_BF16 && G == 128 && K % kGemmKC == 0 && N % 8 == 0 && M <= 65535 &&
                       (size_t)M * K * 2 <= (size_t)INT_MAX &&
                       (size_t)(K / kGemmKC) * Np * 4 <= (size_t)INT_MAX;
  // int8 activations (given, or quantized by the pre-pass) take the integer
  // MFMA kernel from kSmallI8MinM rows on
  const bool small_i8 = f.a == A_I8;
  const bool small_ok = small_i8 ? ((G == 32 || G == 128) && K % 128 == 0 && N % 4 == 0 && M <= kSmallMaxM &&
                                    (size_t)M * K <= (size_t)INT_MAX)
                                 : (f.a == A_BF16 && G == 128 && N % 8 == 0 && M <= kSmallMaxM &&
                                    (size_t)M * K * 2 <= (size_t)INT_MAX);
  int path = force_path;
  if (path == QG_PATH_AUTO)
    path = (M >= (small_i8 ? kSmallI8MinM : 2) && small_ok) ? QG_PATH_SMALL
           : (M > 8 && gemm_ok)                             ? QG_PATH_GEMM
                                                            : QG_PATH_GEMV;
  if ((path == QG_PATH_GEMM && !gemm_ok) || (path == QG_PATH_SMALL && !small_ok)) return QG_EUNSUPPORTED;
  if (path != QG_PATH_GEMV && path != QG_PATH_GEMM && path != QG_PATH_SMALL) return QG_EINVAL;
  p.path = path;

  long long base;
  if (path == QG_PATH_GEMV) {
    p.mb = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    p.mblocks = (M + p.mb - 1) / p.mb;
    p.tiles_x = (int)(Np / kTileCols);
    p.tiles_y = p.mblocks;
    p.units = K / G;
  } else if (path == QG_PATH_SMALL) {
    p.mb = (M + 15) / 16;
    p.tiles_x = (int)(Np / kTileCols);
    p.tiles_y = 1;
    p.units = K / 128;
  } else {
    p.tiles_x = (int)(Np / kGemmBN);
    p.tiles_y = (M + kGemmBM - 1) / kGemmBM;
    p.units = K / kGemmKC;
  }
  base = (long long)p.tiles_x * p.tiles_y;  // workgroups without a K-split

  // K-split: only when the tiles alone leave compute units idle; then aim at
  // two workgroups per compute unit for the GEMV, one for the MFMA paths
  // (the tiled GEMM's 3-stage LDS ring fits one workgroup per compute unit,
  // and the small-M path's partials grow with M). Measured on MI355X, K = N = 4096:
  // M = 256 26.1 us at nsplit 4 vs 31.4 us at 8; M = 512 31.2 us at 2 vs
  // 38.7 us at 4.
  // The GEMV and the small-M MFMA path split only when the tiles leave at
  // least half the compute units idle (the partials and the reduce cost more
  // than the extra workgroups recover once most units are busy). At 176
  // tiles (K = 2048, N = 11264) no split ran: GEMV M = 1, int8 activations,
  // q4_0 6.1 vs 9.1 us (3 slices), q8_0 7.7 vs 9.9 us, float32 activations
  // 9.2 vs 9.7 and 10.1 vs 11.3 us; integer MFMA, M = 32, 12.4 vs 15.3 us (2
  // slices). At 64 tiles (K = N = 4096, bf16, M = 16 / 64) 4 slices ran 8.5
  // / 15.6 vs 11.2 / 22.9 us unsplit. The tiled GEMM splits below one tile
  // per unit (M = 512, 128 tiles: 31.2 us at 2 slices), into at most one
  // workgroup per unit: its 3-stage ring holds one workgroup per unit, so a
  // slice count that overshoots runs a second round of workgroups (M = 384,
  // 96 tiles: 3 slices 39.5 us, 2 slices 31.1 us; M = 96 .. 512 the rounded
  // down count is the fastest or within 5% of it).
  const long long target = path == QG_PATH_GEMV ? 2LL * cus : cus;
  const long long full = path == QG_PATH_GEMM ? cus : (cus + 1) / 2;
  int ns;
  if (force_nsplit > 0)
    ns = force_nsplit;
  else if (base >= full)
    ns = 1;
  else if (path == QG_PATH_GEMM)
    ns = (int)(cus / base);
  else
    ns = (int)((target + base - 1) / base);
  ns = balance(p.units, ns);
  if (path == QG_PATH_GEMV)
    while (ns < p.units && gemv_lds(f, p.mb, G, p.units, ns) > kGemvLdsCap) ns = balance(p.units, ns + 1);
  if (force_nsplit <= 0)
    while (ns > 1 && (size_t)ns * M * Np * 4 > kPartialCap) {
      const int lower = balance(p.units, ns - 1);
      if (path == QG_PATH_GEMV && gemv_lds(f, p.mb, G, p.units, lower) > kGemvLdsCap) break;
      ns = lower;
    }
  if (path == QG_PATH_GEMV) {
    if (gemv_lds(f, p.mb, G, p.units, ns) > kGemvLdsCap) return QG_EUNSUPPORTED;
    p.lds = gemv_lds(f, p.mb, G, p.units, ns);
  }
  p.nsplit = ns;
  p.prep = path == QG_PATH_GEMM ? gemm_a16_bytes(M, K) + gemm_rexp_bytes(M) + gemm_s32_bytes(N, K) : 0;
  if (f.dq) {
    // Each workgroup quantizes the rows and groups it stages; that repeats
    // the work once per column tile, so beyond a few rows one pre-pass that
    // writes the codes and scales to the workspace is faster (measured on
    // MI355X, K = 2048, N = 11264: M = 1 9.5 vs 10.9 us, M = 32 27.9 vs
    // 20.9 us). Both compute the same codes.
    p.dq_fused = M <= kDqFuseMaxM;
    if (!p.dq_fused) {
      p.codes = round256((size_t)M * K);
      p.ascale = round256((size_t)M * (K / G) * 4);
    }
  }
  p.ws = p.codes + p.ascale + p.prep + (p.nsplit > 1 ? (size_t)p.nsplit * M * Np * 4 : 0);
  return QG_OK;
}

// Shape checks shared by every entry point. Returns a status code.
int check_shape(int M, int N, int K, int G, int prec, int has_zp, Formats &f) {
  if (!prec_formats(prec, f)) return QG_EUNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0) return QG_EINVAL;
  if (G != 32 && G != 128) return QG_EUNSUPPORTED;
  if (K % G != 0) return QG_EINVAL;
  if (has_zp && (f.w != W4 || N % 8 != 0)) return QG_EUNSUPPORTED;
  if (padded_cols(N) > (size_t)INT_MAX) return QG_EUNSUPPORTED;
  // grid limits: K-rows of the repack and row blocks of the GEMV
  if ((f.w == W4 ? K / 8 : K / 4) > 65535) return QG_EUNSUPPORTED;
  if ((M + 7) / 8 > 65535) return QG_EUNSUPPORTED;
  // buffer resources address scales, zero-points and one weight tile with
  // 32-bit byte offsets
  if ((size_t)(K / G) * N * 4 > (size_t)INT_MAX || (size_t)K * kTileCols > (size_t)INT_MAX) return QG_EUNSUPPORTED;
  return QG_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

int qgemm_layout_version(void) { return 2; }

size_t qgemm_packed_bytes(int K, int N, int prec) {
  Formats f;
  if (!prec_formats(prec, f) || K <= 0 || N <= 0) return 0;
  if (f.w == W4 ? K % 8 : K % 4) return 0;
  const size_t rows = f.w == W4 ? (size_t)K / 8 : (size_t)K / 4;
  return rows * padded_cols(N) * 4;
}

int qgemm_pack(const void *w_canonical, void *w_packed, int K, int N, int prec, void *stream) {
  Formats f;
  if (!prec_formats(prec, f)) return QG_EUNSUPPORTED;
  if (K <= 0 || N <= 0 || !w_canonical || !w_packed) return QG_EINVAL;
  if (f.w == W4 ? K % 8 : K % 4) return QG_EINVAL;
  if ((f.w == W4 ? K / 8 : K / 4) > 65535 || padded_cols(N) > (size_t)INT_MAX) return QG_EUNSUPPORTED;
  if (!aligned16(w_canonical) || !aligned16(w_packed)) return QG_EALIGN;
  drop_pending_error();
  const hipError_t e = launch_pack(f.w, w_canonical, (uint32_t *)w_packed, K, N, (int)padded_cols(N), 0,
                                   (hipStream_t)stream);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

int qgemm_plan(int M, int N, int K, int group, int prec, int force_path, int force_nsplit, int *path,
               int *nsplit, size_t *workspace_bytes) {
  Formats f;
  int st = check_shape(M, N, K, group, prec, 0, f);
  if (st != QG_OK) return st;
  Plan p;
  st = make_plan(M > 0 ? M : 1, N, K, group, f, force_path, force_nsplit, p);
  if (st != QG_OK) return st;
  if (path) *path = p.path;
  if (nsplit) *nsplit = p.nsplit;
  if (workspace_bytes) *workspace_bytes = M > 0 ? p.ws : 0;
  return QG_OK;
}

size_t qgemm_workspace_bytes(int M, int N, int K, int group, int prec) {
  size_t ws = 0;
  if (qgemm_plan(M, N, K, group, prec, QG_PATH_AUTO, 0, nullptr, nullptr, &ws) != QG_OK) return 0;
  return ws;
}

// Whether t256 tiles of 128 x 256 finish sooner than t128 tiles of 128 x 128,
// each kernel taking one tile per compute unit at a time: a round of the wide
// tiles costs about 1.6 rounds of the narrow ones (256 tiles of each at K =
// N = 4096: 71.6 against 44.8 us), so ties go to the narrow tiles.
static bool wide_rounds_cheaper(long long t128, long long t256, int cus) {
  const long long r128 = (t128 + cus - 1) / cus, r256 = (t256 + cus - 1) / cus;
  return 8 * r256 < 5 * r128;
}

// The product of qgemm_run_ex; gu_d > 0: a gate-up packed product of N =
// 2 gu_d columns whose SwiGLU gate step is applied in the epilogue (out is
// [M][gu_d]; bf16 activations on the GEMV or small-M path only).
static int run_common(int M, int N, int K, int group, int prec, int has_zp, const void *A, const void *a_scales,
                      const void *w_packed, const void *scales, const void *zeros, void *out, void *workspace,
                      size_t workspace_bytes, void *stream, int force_path, int force_nsplit, int gu_d) {
  Formats f;
  int st = check_shape(M, N, K, group, prec, has_zp, f);
  if (st != QG_OK) return st;
  if (M == 0) return QG_OK;
  if (!A || !w_packed || !scales || !out) return QG_EINVAL;
  const bool given_scales = f.a == A_I8 && !f.dq;
  if (given_scales && !a_scales) return QG_EINVAL;
  if (has_zp && !zeros) return QG_EINVAL;
  if (!aligned16(A) || !aligned16(w_packed) || !aligned16(scales) || !aligned16(out) ||
      (given_scales && !aligned16(a_scales)) || (has_zp && !aligned16(zeros)))
    return QG_EALIGN;
  Plan p;
  st = make_plan(M, N, K, group, f, force_path, force_nsplit, p);
  if (st != QG_OK) return st;
  if (gu_d > 0 && (p.path == QG_PATH_GEMM || f.a != A_BF16)) return QG_EUNSUPPORTED;
  if (p.ws > 0) {
    if (!workspace || workspace_bytes < p.ws) return QG_EWORKSPACE;
    if (!aligned16(workspace)) return QG_EALIGN;
  }
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  float *partial = p.nsplit > 1 ? (float *)(ws + p.codes + p.ascale + p.prep) : nullptr;
  const int Np = (int)padded_cols(N);
  drop_pending_error();
  hipError_t e = hipSuccess;
  if (f.dq && !p.dq_fused) {
    // the product then reads the codes and scales this writes
    e = launch_quant((const float *)A, (int8_t *)ws, (float *)(ws + p.codes), M, K, group, s);
    if (e != hipSuccess) return QG_EHIP;
    A = ws;
    a_scales = ws + p.codes;
  }
  if (p.path == QG_PATH_GEMV) {
    GemvArgs a;
    a.A = A;
    a.a_scale = (const float *)a_scales;
    a.W = (const uint32_t *)w_packed;
    a.S = scales;
    a.Z = has_zp ? (const uint32_t *)zeros : nullptr;
    a.out = out;
    a.partial = partial;
    a.M = M; a.N = N; a.K = K; a.G = group; a.Np = Np;
    a.ngroups = K / group;
    a.nsplit = p.nsplit;
    a.gu_d = gu_d;
    const dim3 grid(p.tiles_x, p.mblocks, p.nsplit);
    e = f.a == A_I8 ? launch_gemv_i8(f.w, has_zp != 0, p.dq_fused, p.mb, a, grid, p.lds, s)
                    : launch_gemv(f.w, f.a, f.s, f.o, has_zp != 0, p.mb, a, grid, p.lds, s);
  } else if (p.path == QG_PATH_SMALL && f.a == A_I8) {
    SmallI8Args a;
    a.A = (const int8_t *)A;
    a.a_scale = (const float *)a_scales;
    a.W = (const uint32_t *)w_packed;
    a.S = (const float *)scales;
    a.Z = has_zp ? (const uint32_t *)zeros : nullptr;
    a.out = (float *)out;
    a.partial = partial;
    a.M = M; a.N = N; a.K = K; a.G = group; a.Np = Np;
    a.nsplit = p.nsplit;
    e = launch_gemm_small_i8(f.w, has_zp != 0, p.mb, a, dim3(p.tiles_x, p.nsplit), s);
  } else if (p.path == QG_PATH_SMALL) {
    SmallArgs a;
    a.A = (const uint16_t *)A;
    a.W = (const uint32_t *)w_packed;
    a.S = (const uint16_t *)scales;
    a.Z = has_zp ? (const uint32_t *)zeros : nullptr;
    a.out = out;
    a.partial = partial;
    a.M = M; a.N = N; a.K = K; a.Np = Np;
    a.ngroups = K / 128;
    a.nsplit = p.nsplit;
    a.gu_d = gu_d;
    e = launch_gemm_small(f.o, has_zp != 0, p.mb, a, dim3(p.tiles_x, p.nsplit), s);
  } else {
    GemmArgs a;
    a.A = (const uint16_t *)A;
    a.W = (const uint32_t *)w_packed;
    a.S = (const uint16_t *)scales;
    a.Z = has_zp ? (const uint32_t *)zeros : nullptr;
    a.out = out;
    a.partial = partial;
    char *pp = ws + p.codes + p.ascale;
    a.A16 = (uint16_t *)pp;
    a.rexp = (int *)(pp + gemm_a16_bytes(M, K));
    a.S32 = (float *)(pp + gemm_a16_bytes(M, K) + gemm_rexp_bytes(M));
    a.M = M; a.N = N; a.K = K; a.Np = Np;
    a.nchunks = K / kGemmKC;
    a.nsplit = p.nsplit;
    const bool wide = p.nsplit == 1 && Np % 256 == 0 &&
                      wide_rounds_cheaper((long long)p.tiles_x * p.tiles_y, (long long)(Np / 256) * p.tiles_y,
                                          device_cus());
    e = launch_gemm(f.o, has_zp != 0, a, dim3(p.tiles_x, p.tiles_y, p.nsplit), wide, s);
  }
  if (e == hipSuccess && p.nsplit > 1)
    e = gu_d > 0 ? launch_reduce_gate_up(f.o, partial, out, M, gu_d, Np, p.nsplit, s)
                 : launch_reduce(f.o, partial, out, M, N, Np, p.nsplit, s);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

int qgemm_run_ex(int M, int N, int K, int group, int prec, int has_zp, const void *A,
                 const void *a_scales, const void *w_packed, const void *scales, const void *zeros,
                 void *out, void *workspace, size_t workspace_bytes, void *stream, int force_path,
                 int force_nsplit) {
  return run_common(M, N, K, group, prec, has_zp, A, a_scales, w_packed, scales, zeros, out, workspace,
                    workspace_bytes, stream, force_path, force_nsplit, 0);
}

// ---- fused gate_up product with SwiGLU's gate step ----

static bool gate_up_prec(int prec) { return prec == QG_W4_A_BF16 || prec == QG_W4_A_BF16_OF32; }

int qgemm_pack_gate_up(const void *w_canonical, void *w_packed, int K, int d, int prec, void *stream) {
  if (!gate_up_prec(prec)) return QG_EUNSUPPORTED;
  if (K <= 0 || d <= 0 || !w_canonical || !w_packed) return QG_EINVAL;
  if (K % 8 != 0 || d % 32 != 0) return QG_EINVAL;
  if (d > INT_MAX / 2 || K / 8 > 65535 || padded_cols(2 * d) > (size_t)INT_MAX) return QG_EUNSUPPORTED;
  if (!aligned16(w_canonical) || !aligned16(w_packed)) return QG_EALIGN;
  drop_pending_error();
  const hipError_t e = launch_pack(W4, w_canonical, (uint32_t *)w_packed, K, 2 * d, (int)padded_cols(2 * d), d,
                                   (hipStream_t)stream);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

int qgemm_gate_up_plan(int M, int d, int K, int group, int prec, int force_path, int force_nsplit, int *path,
                       int *nsplit, size_t *workspace_bytes) {
  if (!gate_up_prec(prec)) return QG_EUNSUPPORTED;
  if (d <= 0 || d % 32 != 0) return QG_EINVAL;
  if (d > INT_MAX / 2) return QG_EUNSUPPORTED;
  int pth = 0;
  const int st = qgemm_plan(M, 2 * d, K, group, prec, force_path, force_nsplit, &pth, nsplit, workspace_bytes);
  if (st != QG_OK) return st;
  if (pth == QG_PATH_GEMM) return QG_EUNSUPPORTED;
  if (path) *path = pth;
  return QG_OK;
}

size_t qgemm_gate_up_workspace_bytes(int M, int d, int K, int group, int prec) {
  size_t ws = 0;
  if (qgemm_gate_up_plan(M, d, K, group, prec, QG_PATH_AUTO, 0, nullptr, nullptr, &ws) != QG_OK) return 0;
  return ws;
}

int qgemm_run_gate_up_silu_ex(int M, int d, int K, int group, int prec, int has_zp, const void *A,
                              const void *w_packed, const void *scales, const void *zeros, void *out,
                              void *workspace, size_t workspace_bytes, void *stream, int force_path,
                              int force_nsplit) {
  if (!gate_up_prec(prec)) return QG_EUNSUPPORTED;
  if (d <= 0 || d % 32 != 0) return QG_EINVAL;
  if (d > INT_MAX / 2) return QG_EUNSUPPORTED;
  return run_common(M, 2 * d, K, group, prec, has_zp, A, nullptr, w_packed, scales, zeros, out, workspace,
                    workspace_bytes, stream, force_path, force_nsplit, d);
}

int qgemm_run_gate_up_silu(int M, int d, int K, int group, int prec, int has_zp, const void *A,
                           const void *w_packed, const void *scales, const void *zeros, void *out, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return qgemm_run_gate_up_silu_ex(M, d, K, group, prec, has_zp, A, w_packed, scales, zeros, out, workspace,
                                   workspace_bytes, stream, QG_PATH_AUTO, 0);
}

int qgemm_run(int M, int N, int K, int group, int prec, int has_zp, const void *A,
              const void *a_scales, const void *w_packed, const void *scales, const void *zeros,
              void *out, void *workspace, size_t workspace_bytes, void *stream) {
  return qgemm_run_ex(M, N, K, group, prec, has_zp, A, a_scales, w_packed, scales, zeros, out, workspace,
                      workspace_bytes, stream, QG_PATH_AUTO, 0);
}

}  // extern "C"

// Workspace of qgemm_run_noalloc: one copy of this array per GPU, placed in
// the code object's global memory when the library's code is loaded on that
// device and held until the process ends. Host code never uses the array's
// name as an address (on the host it names a stand-in): each device's
// address comes from hipGetSymbolAddress, taken once with that device
// current.
static __device__ __align__(256) unsigned char scratch[QG_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<void *> g_scratch[kMaxDevices];

// This device's copy of `scratch`, or null when its address cannot be had.
void *scratch_address(int dev) {
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void *q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
    (void)hipGetLastError();
    return nullptr;
  }
  // threads that race here all store the same address
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" {

int qgemm_run_noalloc(int M, int N, int K, int group, int prec, int has_zp, const void *A, const void *a_scales,
                      const void *w_packed, const void *scales, const void *zeros, void *out, void *stream) {
  Formats f;
  int st = check_shape(M, N, K, group, prec, has_zp, f);
  if (st != QG_OK) return st;
  if (M == 0) return QG_OK;
  Plan p;
  st = make_plan(M, N, K, group, f, QG_PATH_AUTO, 0, p);
  if (st != QG_OK) return st;
  if (p.ws > (size_t)QG_NOALLOC_SCRATCH_BYTES) return QG_EWORKSPACE;
  void *ws = nullptr;
  if (p.ws > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
      (void)hipGetLastError();
      return QG_EHIP;
    }
    ws = scratch_address(dev);
    if (!ws) return QG_EHIP;
  }
  return qgemm_run_ex(M, N, K, group, prec, has_zp, A, a_scales, w_packed, scales, zeros, out, ws,
                      ws ? (size_t)QG_NOALLOC_SCRATCH_BYTES : 0, stream, QG_PATH_AUTO, 0);
}

int qgemm_quantize_activations(const void *A, int M, int K, int group, void *Aq, void *a_scales,
                               void *stream) {
  if (M < 0 || K <= 0) return QG_EINVAL;
  if (group != 32 && group != 128) return QG_EUNSUPPORTED;
  if (K % group != 0) return QG_EINVAL;
  if ((size_t)M * K / 1024 > (size_t)INT_MAX) return QG_EUNSUPPORTED;  // grid of 256 x 4 elements
  if (M == 0) return QG_OK;
  if (!A || !Aq || !a_scales) return QG_EINVAL;
  if (!aligned16(A) || !aligned16(Aq) || !aligned16(a_scales)) return QG_EALIGN;
  drop_pending_error();
  const hipError_t e = launch_quant((const float *)A, (int8_t *)Aq, (float *)a_scales, M, K, group,
                                    (hipStream_t)stream);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

int qgemm_dequantize(const void *w_packed, const void *scales, const void *zeros, int K, int N, int group,
                     int prec, int has_zp, void *out, void *stream) {
  if (prec != QG_W4_A_BF16 && prec != QG_W4_A_BF16_OF32) return QG_EUNSUPPORTED;
  if (group != 32 && group != 128) return QG_EUNSUPPORTED;
  if (K <= 0 || N <= 0 || K % group != 0) return QG_EINVAL;
  if (K / 8 > 65535 || padded_cols(N) > (size_t)INT_MAX) return QG_EUNSUPPORTED;
  if (has_zp && N % 8 != 0) return QG_EUNSUPPORTED;
  if (!w_packed || !scales || !out || (has_zp && !zeros)) return QG_EINVAL;
  if (!aligned16(w_packed) || !aligned16(scales) || !aligned16(out) || (has_zp && !aligned16(zeros)))
    return QG_EALIGN;
  drop_pending_error();
  const hipError_t e = launch_dequant_w4((const uint32_t *)w_packed, (const uint16_t *)scales,
                                         has_zp ? (const uint32_t *)zeros : nullptr, (uint16_t *)out, K, N, group,
                                         (hipStream_t)stream);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

bool moe_block_ok(int block) {
  return block == 1 || block == 2 || block == 4 || block == 8 || block == 16 || block == 32 || block == 64;
}

int qgemm_moe_max_tiles(int numel, int E, int block) {
  if (numel < 0 || E < 1 || E > kMoeMaxExperts || !moe_block_ok(block)) return 0;
  const long long t = ((long long)numel + (long long)E * (block - 1)) / block;
  return t > 65535 ? 0 : (int)(t > 0 ? t : 1);
}

int qgemm_moe_align(const int *topk_ids, int numel, int E, int block, int *sorted_ids, int *tile_experts,
                    int *num_post_pad, void *stream) {
  if (numel < 0) return QG_EINVAL;
  const int max_tiles = qgemm_moe_max_tiles(numel, E, block);
  if (max_tiles == 0) return QG_EUNSUPPORTED;
  if (!sorted_ids || !tile_experts || !num_post_pad || (numel > 0 && !topk_ids)) return QG_EINVAL;
  if ((numel > 0 && !aligned16(topk_ids)) || !aligned16(sorted_ids) || !aligned16(tile_experts) ||
      !aligned16(num_post_pad))
    return QG_EALIGN;
  drop_pending_error();
  const hipError_t e = launch_moe_align(topk_ids, numel, E, block, max_tiles, sorted_ids, tile_experts,
                                        num_post_pad, (hipStream_t)stream);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

namespace {

// Plan of the grouped GEMV: one row block per possible tile, a K-split when
// the column tiles times the tiles that are surely used (numel / block)
// leave compute units idle; the same rules as the dense GEMV.
// Blocks of 1..8 rows run on the grouped GEMV, blocks of 16, 32 or 64 rows
// on the grouped small-M MFMA path (groups of 128, N % 8 == 0).
int moe_plan(int numel, int N, int K, int G, const Formats &f, int E, int block, int force_nsplit, Plan &p) {
  const int cus = device_cus();
  const size_t Np = padded_cols(N);
  const bool mfma = block >= 16;
  if (mfma && (G != 128 || N % 8 != 0)) return QG_EUNSUPPORTED;
  p.path = mfma ? QG_PATH_SMALL : QG_PATH_GEMV;
  p.mb = mfma ? block / 16 : block;
  p.mblocks = qgemm_moe_max_tiles(numel, E, block);
  p.tiles_x = (int)(Np / kTileCols);
  p.units = K / G;
  const long long used = (numel + block - 1) / block;
  const long long base = (long long)p.tiles_x * (used > 0 ? used : 1);
  const long long target = mfma ? cus : 2LL * cus;
  int ns = force_nsplit > 0 ? force_nsplit : (base >= cus ? 1 : (int)((target + base - 1) / base));
  ns = balance(p.units, ns);
  if (!mfma)
    while (ns < p.units && gemv_lds(f, p.mb, G, p.units, ns) > kGemvLdsCap) ns = balance(p.units, ns + 1);
  if (force_nsplit <= 0)
    while (ns > 1 && (size_t)ns * numel * Np * 4 > kPartialCap) {
      const int lower = balance(p.units, ns - 1);
      if (!mfma && gemv_lds(f, p.mb, G, p.units, lower) > kGemvLdsCap) break;
      ns = lower;
    }
  if (!mfma) {
    if (gemv_lds(f, p.mb, G, p.units, ns) > kGemvLdsCap) return QG_EUNSUPPORTED;
    p.lds = gemv_lds(f, p.mb, G, p.units, ns);
  }
  p.nsplit = ns;
  p.ws = ns > 1 ? (size_t)ns * numel * Np * 4 : 0;
  return QG_OK;
}

int check_moe(int T, int topk, int N, int K, int G, int prec, int has_zp, int E, int block, Formats &f) {
  if (prec != QG_W4_A_BF16 && prec != QG_W4_A_BF16_OF32) return QG_EUNSUPPORTED;
  if (T < 0 || topk < 1) return QG_EINVAL;
  if ((long long)T * topk > INT_MAX / 2) return QG_EUNSUPPORTED;
  const int numel = T * topk;
  if (qgemm_moe_max_tiles(numel, E, block) == 0) return QG_EUNSUPPORTED;
  // the MFMA blocks address the T activation rows with 32-bit byte offsets
  if (block >= 16 && (size_t)T * K * 2 > (size_t)INT_MAX) return QG_EUNSUPPORTED;
  return check_shape(numel > 0 ? numel : 1, N, K, G, prec, has_zp, f);
}

}  // namespace

int qgemm_moe_default_block(int T, int topk, int E, int group, int N) {
  if (T < 1 || topk < 1 || E < 1) return 1;
  if (T == 1 || group != 128 || N % 8 != 0) return T == 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8));
  // one 16-row MFMA block holds every row of an expert when T <= 16 (a
  // token's experts are distinct); beyond, size the block for about twice
  // the average rows per expert
  if (T <= 16) return 16;
  const long long twice_avg = 2LL * T * topk / E;
  return twice_avg <= 16 ? 16 : (twice_avg <= 32 ? 32 : 64);
}

size_t qgemm_moe_workspace_bytes(int T, int topk, int N, int K, int group, int prec, int E, int block) {
  Formats f;
  if (check_moe(T, topk, N, K, group, prec, 0, E, block, f) != QG_OK || T == 0) return 0;
  Plan p;
  if (moe_plan(T * topk, N, K, group, f, E, block, 0, p) != QG_OK) return 0;
  return p.ws;
}

// The grouped product of qgemm_moe_run; gu_d > 0: each expert's weight is a
// gate-up packed product of N = 2 gu_d columns whose SwiGLU gate step is
// applied in the epilogue (out is [T * topk][gu_d]).
static int moe_run_common(int T, int topk, int N, int K, int group, int prec, int has_zp, int E, int block,
                          const void *A, const void *w_packed, const void *scales, const void *zeros,
                          const int *sorted_ids, const int *tile_experts, const int *num_post_pad, void *out,
                          void *workspace, size_t workspace_bytes, void *stream, int gu_d) {
  Formats f;
  int st = check_moe(T, topk, N, K, group, prec, has_zp, E, block, f);
  if (st != QG_OK) return st;
  if (T == 0) return QG_OK;
  if (!A || !w_packed || !scales || !out || !sorted_ids || !tile_experts || !num_post_pad) return QG_EINVAL;
  if (has_zp && !zeros) return QG_EINVAL;
  if (!aligned16(A) || !aligned16(w_packed) || !aligned16(scales) || !aligned16(out) || !aligned16(sorted_ids) ||
      !aligned16(tile_experts) || !aligned16(num_post_pad) || (has_zp && !aligned16(zeros)))
    return QG_EALIGN;
  const int numel = T * topk;
  Plan p;
  st = moe_plan(numel, N, K, group, f, E, block, 0, p);
  if (st != QG_OK) return st;
  if (p.ws > 0) {
    if (!workspace || workspace_bytes < p.ws) return QG_EWORKSPACE;
    if (!aligned16(workspace)) return QG_EALIGN;
  }
  hipStream_t s = (hipStream_t)stream;
  float *partial = p.nsplit > 1 ? (float *)workspace : nullptr;
  const int Np = (int)padded_cols(N);
  drop_pending_error();
  hipError_t e;
  if (p.path == QG_PATH_SMALL) {
    SmallArgs a = {};
    a.A = (const uint16_t *)A;
    a.W = (const uint32_t *)w_packed;
    a.S = (const uint16_t *)scales;
    a.Z = has_zp ? (const uint32_t *)zeros : nullptr;
    a.out = out;
    a.partial = partial;
    a.M = numel; a.N = N; a.K = K; a.Np = Np;
    a.ngroups = K / 128;
    a.nsplit = p.nsplit;
    a.sorted_ids = sorted_ids;
    a.tile_experts = tile_experts;
    a.num_post_pad = num_post_pad;
    a.topk = topk;
    a.arows = T;
    a.w_expert_words = qgemm_packed_bytes(K, N, prec) / 4;
    a.s_expert_elems = (size_t)(K / 128) * N;
    a.z_expert_words = (size_t)(K / 128) * (N / 8);
    a.gu_d = gu_d;
    e = launch_gemm_small_grouped(f.o, has_zp != 0, p.mb, a, dim3(p.tiles_x, p.nsplit, p.mblocks), s);
  } else {
    GemvArgs a = {};
    a.A = A;
    a.W = (const uint32_t *)w_packed;
    a.S = scales;
    a.Z = has_zp ? (const uint32_t *)zeros : nullptr;
    a.out = out;
    a.partial = partial;
    a.M = numel; a.N = N; a.K = K; a.G = group; a.Np = Np;
    a.ngroups = K / group;
    a.nsplit = p.nsplit;
    a.sorted_ids = sorted_ids;
    a.tile_experts = tile_experts;
    a.num_post_pad = num_post_pad;
    a.topk = topk;
    a.w_expert_words = qgemm_packed_bytes(K, N, prec) / 4;
    a.s_expert_bytes = (size_t)(K / group) * N * 2;
    a.z_expert_words = (size_t)(K / group) * (N / 8);
    a.gu_d = gu_d;
    e = launch_gemv_grouped(f.o, has_zp != 0, p.mb, a, dim3(p.tiles_x, p.mblocks, p.nsplit), p.lds, s);
  }
  if (e == hipSuccess && p.nsplit > 1)
    e = gu_d > 0 ? launch_reduce_gate_up(f.o, partial, out, numel, gu_d, Np, p.nsplit, s)
                 : launch_reduce(f.o, partial, out, numel, N, Np, p.nsplit, s);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

int qgemm_moe_run(int T, int topk, int N, int K, int group, int prec, int has_zp, int E, int block, const void *A,
                  const void *w_packed, const void *scales, const void *zeros, const int *sorted_ids,
                  const int *tile_experts, const int *num_post_pad, void *out, void *workspace,
                  size_t workspace_bytes, void *stream) {
  return moe_run_common(T, topk, N, K, group, prec, has_zp, E, block, A, w_packed, scales, zeros, sorted_ids,
                        tile_experts, num_post_pad, out, workspace, workspace_bytes, stream, 0);
}

int qgemm_moe_run_gate_up_silu(int T, int topk, int d, int K, int group, int prec, int has_zp, int E, int block,
                               const void *A, const void *w_packed, const void *scales, const void *zeros,
                               const int *sorted_ids, const int *tile_experts, const int *num_post_pad, void *out,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (d <= 0 || d % 32 != 0) return QG_EINVAL;
  if (d > INT_MAX / 2) return QG_EUNSUPPORTED;
  return moe_run_common(T, topk, 2 * d, K, group, prec, has_zp, E, block, A, w_packed, scales, zeros, sorted_ids,
                        tile_experts, num_post_pad, out, workspace, workspace_bytes, stream, d);
}

int qgemm_fp8_quantize(const void *A, int M, int K, int block, void *Aq, void *a_scales, void *stream) {
  if (M < 0 || K <= 0) return QG_EINVAL;
  if (block != QG_FP8_PER_TOKEN && block != 128) return QG_EUNSUPPORTED;
  if (K % (block ? block : 8) != 0) return QG_EINVAL;
  if ((size_t)M * K / 2048 > (size_t)INT_MAX) return QG_EUNSUPPORTED;  // grid of 256 x 8 elements
  if (M == 0) return QG_OK;
  if (!A || !Aq || !a_scales) return QG_EINVAL;
  if (!aligned16(A) || !aligned16(Aq) || !aligned16(a_scales)) return QG_EALIGN;
  drop_pending_error();
  const hipError_t e = launch_fp8_quant((const uint16_t *)A, (uint8_t *)Aq, (float *)a_scales, M, K, block,
                                        (hipStream_t)stream);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

// FP8 GEMM plan: workgroup tiles of 128 x 128 over (N, M); with fewer tiles
// than compute units the K steps are split into slices, at most one round of
// one workgroup per unit (the 3-stage ring holds one workgroup per unit), as
// for the tiled W4 GEMM, and evened out over the steps. Partials [nsplit][M]
// [Np] with Np = N rounded up to the tile.
static int fp8_check(int M, int N, int K, int scaling) {
  if (M < 0 || N <= 0 || K <= 0) return QG_EINVAL;
  if (scaling != QG_FP8_PER_TOKEN && scaling != QG_FP8_BLOCKWISE) return QG_EUNSUPPORTED;
  if (K % 128 != 0) return QG_EINVAL;
  if (scaling == QG_FP8_BLOCKWISE && N % 128 != 0) return QG_EUNSUPPORTED;
  // buffer resources address 128 rows of K bytes, and 128 rows of K / 128 scales,
  // with 32-bit offsets; the grid has ceil(M / 128) rows of workgroups
  if ((size_t)128 * K > (size_t)INT_MAX || (M + 127) / 128 > 65535) return QG_EUNSUPPORTED;
  if ((size_t)(N + 127) / 128 * 128 > (size_t)INT_MAX) return QG_EUNSUPPORTED;
  return QG_OK;
}

static int fp8_nsplit(int M, int N, int K, int force_nsplit, int cus) {
  const int nsteps = K / 128;
  const long long tiles = (long long)((N + 127) / 128) * ((M + 127) / 128);
  const size_t Np = (size_t)(N + 127) / 128 * 128;
  // at most max(4, 128 / M) slices: past that the partials' traffic costs
  // more than the extra workgroups recover (K = N = 4096, forced sweeps: M = 16
  // best at 8 slices, 10.5 us vs 11.0 at 4; M = 32, 64, 128 best at 3-4, 6-8%
  // ahead of 8)
  const int cap = M > 0 && 128 / M > 4 ? 128 / M : 4;
  int ns = force_nsplit > 0 ? force_nsplit : (tiles >= cus ? 1 : (int)std::min<long long>(cus / tiles, cap));
  ns = balance(nsteps, ns);
  if (force_nsplit <= 0)
    while (ns > 1 && (size_t)ns * M * Np * 4 > kPartialCap) ns = balance(nsteps, ns - 1);
  return ns;
}

size_t qgemm_fp8_workspace_bytes(int M, int N, int K, int scaling) {
  if (fp8_check(M, N, K, scaling) != QG_OK || M == 0) return 0;
  const int ns = fp8_nsplit(M, N, K, 0, device_cus());
  return ns > 1 ? (size_t)ns * M * ((size_t)(N + 127) / 128 * 128) * 4 : 0;
}

int qgemm_fp8_gemm_ex(int M, int N, int K, int scaling, const void *Aq, const void *a_scales, const void *Wq,
                      const void *w_scales, void *out, void *workspace, size_t workspace_bytes, int force_nsplit,
                      void *stream) {
  const int chk = fp8_check(M, N, K, scaling);
  if (chk != QG_OK) return chk;
  if (force_nsplit < 0) return QG_EINVAL;
  if (M == 0) return QG_OK;
  if (!Aq || !a_scales || !Wq || !w_scales || !out) return QG_EINVAL;
  if (!aligned16(Aq) || !aligned16(a_scales) || !aligned16(Wq) || !aligned16(w_scales) || !aligned16(out))
    return QG_EALIGN;
  const int cus = device_cus();
  const int ns = fp8_nsplit(M, N, K, force_nsplit, cus);
  const int Np = (N + 127) / 128 * 128;
  if (ns > 1) {
    if (!workspace || workspace_bytes < (size_t)ns * M * Np * 4) return QG_EWORKSPACE;
    if (!aligned16(workspace)) return QG_EALIGN;
  }
  drop_pending_error();
  const hipError_t e = launch_fp8_gemm(scaling, (const uint8_t *)Aq, (const float *)a_scales, (const uint8_t *)Wq,
                                       (const float *)w_scales, (uint16_t *)out, (float *)workspace, M, N, K, ns, Np,
                                       cus, (hipStream_t)stream);
  return e == hipSuccess ? QG_OK : QG_EHIP;
}

int qgemm_fp8_gemm(int M, int N, int K, int scaling, const void *Aq, const void *a_scales, const void *Wq,
                   const void *w_scales, void *out, void *stream) {
  return qgemm_fp8_gemm_ex(M, N, K, scaling, Aq, a_scales, Wq, w_scales, out, nullptr, 0, 1, stream);
}

int qgemm_stream_read(const void *src, size_t bytes, void *out, int blocks, void *stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0 || bytes >= (size_t)INT_MAX || blocks < 1 || blocks > 65535)
    return QG_EINVAL;
  if (!aligned16(src) || ((uintptr_t)out & 3u) != 0) return QG_EALIGN;
  drop_pending_error();
  return launch_stream_read(src, bytes, (uint32_t *)out, blocks, (hipStream_t)stream) == hipSuccess ? QG_OK
                                                                                                    : QG_EHIP;
}

const char *qgemm_strerror(int status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_EINVAL: return "invalid argument (null pointer, bad size, or K not a multiple of the group)";
    case QG_EUNSUPPORTED: return "unsupported combination (group size, precision, zero-points or limits)";
    case QG_EWORKSPACE: return "workspace missing or smaller than qgemm_workspace_bytes()";
    case QG_EALIGN: return "pointer not 16-byte aligned";
    case QG_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
