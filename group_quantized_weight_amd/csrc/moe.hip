// Routing metadata for the grouped (MoE) GEMV: the align step of the fused
// MoE pipeline on the page "quantization-and-fused-kernels"
// (arganzheng.life), section 六.3. From the expert of every routed slot
// (topk_ids, slot i = token * topk + j) it writes
//   sorted_ids:   the slots grouped by expert, each expert's segment padded
//                 to a multiple of `block` rows with the sentinel numel;
//   tile_experts: the expert of each block of `block` rows (-1 past the end);
//   num_post_pad: the padded row count.
// It is a counting sort in one workgroup: per-expert counts (LDS atomics),
// an exclusive sum of the padded counts (lane shifts within each wave, then
// over the waves), then each slot takes the next free position of its
// expert's segment. As on the page, the order of slots
// within an expert follows the atomics' arrival; the grouped GEMV computes
// every row on its own, so its output does not depend on that order. Slots
// whose expert is outside [0, E) are skipped (their output rows are left
// unspecified).
#include "common.h"

namespace qg {

// Slots each thread keeps in registers between the counting and the placing
// pass (slot i is held by thread i % 1024 while i < 1024 * kAlignKeep; later
// slots are read again).
constexpr int kAlignKeep = 8;

__global__ __launch_bounds__(1024) void moe_align_kernel(const int *__restrict__ topk_ids, int numel, int E, int block,
                                                        int max_tiles, int *__restrict__ sorted_ids,
                                                        int *__restrict__ tile_experts, int *__restrict__ num_post_pad) {
  extern __shared__ int sh[];
  int *cnt = sh;             // [E]
  int *off = sh + E;         // [E + 1] padded segment starts
  int *cur = off + E + 1;    // [E] next free position per expert
  __shared__ int s_wave[16]; // inclusive sums of the 16 waves' padded counts
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += nt) {
    cnt[e] = 0;
    cur[e] = 0;
  }
  __syncthreads();
  int ek[kAlignKeep];
#pragma unroll
  for (int r = 0; r < kAlignKeep; ++r) {
    const int i = tid + r * nt;
    ek[r] = i < numel ? topk_ids[i] : -1;
  }
#pragma unroll
  for (int r = 0; r < kAlignKeep; ++r)
    if (ek[r] >= 0 && ek[r] < E) atomicAdd(&cnt[ek[r]], 1);
  for (int i = tid + kAlignKeep * nt; i < numel; i += nt) {
    const int e = topk_ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive sum of the padded counts (E <= 1024: thread e holds expert e):
  // inclusive sums within a wave by lane shifts; above 64 experts, then over
  // the waves
  auto wave_scan = [&](int x) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    return x;
  };
  auto publish = [&](int v, int incl) {
    if (tid < E) off[tid] = incl - v;
    if (tid == E - 1) {
      off[E] = incl;
      *num_post_pad = incl;
    }
  };
  if (E <= 64) {
    if (wv == 0) {
      const int v = tid < E ? (cnt[tid] + block - 1) / block * block : 0;
      publish(v, wave_scan(v));
    }
  } else {
    const int v = tid < E ? (cnt[tid] + block - 1) / block * block : 0;
    const int x = wave_scan(v);
    if (lane == 63) s_wave[wv] = x;
    __syncthreads();
    if (wv == 0) {
      int w = lane < 16 ? s_wave[lane] : 0;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int y = __shfl_up(w, d);
        if (lane >= d) w += y;
      }
      if (lane < 16) s_wave[lane] = w;
    }
    __syncthreads();
    publish(v, x + (wv > 0 ? s_wave[wv - 1] : 0));
  }
  __syncthreads();
  const int total = off[E];
  for (int p = tid; p < max_tiles * block; p += nt) sorted_ids[p] = numel;
  for (int t = tid; t < max_tiles; t += nt) {
    int e = -1;
    if (t * block < total) {  // the expert whose segment holds row t * block: off[e] <= x < off[e + 1]
      const int xr = t * block;
      int lo = 0, hi = E;     // first j in [0, E] with off[j] > xr is in (lo, hi]
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (off[mid] <= xr)
          lo = mid;
        else
          hi = mid - 1;
      }
      e = lo;
    }
    tile_experts[t] = e;
  }
  __syncthreads();  // the sentinel fill above is ordered before the placement below
#pragma unroll
  for (int r = 0; r < kAlignKeep; ++r) {
    const int e = ek[r];
    if (e >= 0 && e < E) sorted_ids[off[e] + atomicAdd(&cur[e], 1)] = tid + r * nt;
  }
  for (int i = tid + kAlignKeep * nt; i < numel; i += nt) {
    const int e = topk_ids[i];
    if (e >= 0 && e < E) sorted_ids[off[e] + atomicAdd(&cur[e], 1)] = i;
  }
}

hipError_t launch_moe_align(const int *topk_ids, int numel, int E, int block, int max_tiles, int *sorted_ids,
                            int *tile_experts, int *num_post_pad, hipStream_t st) {
  moe_align_kernel<<<1, 1024, (size_t)(3 * E + 1) * sizeof(int), st>>>(topk_ids, numel, E, block, max_tiles,
                                                                       sorted_ids, tile_experts, num_post_pad);
  return hipGetLastError();
}

}  // namespace qg
