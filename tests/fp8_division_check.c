/* The FP8 quantization divides bf16 activations by one float32 scale per
 * row or block, sc = RN(amax / 448), with a shortcut for finite sc >= 2^-100:
 * r = RN(1 / sc), q = RN(x r), RN(q + RN(x - sc q) r) (Markstein's
 * correction step; the inner fma leaves the residual exact). The codes must
 * equal those of the correctly rounded quotient RN(x / sc). This program
 * checks that for every bf16 magnitude amax whose scale takes the shortcut
 * and every bf16 x with |x| <= amax: both quotients, clamped to +-448 and
 * rounded to E4M3 (3 fraction bits, subnormal step 2^-9, ties to even), give
 * the same value. Prints the counts; exit status 1 on any difference.
 * Build with -ffp-contract=off (no fused operations beyond the fmaf calls). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bf16(uint32_t h) {
  const uint32_t u = h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* E4M3 value of v after clamping to +-448, round to nearest even */
static double e4m3(float v) {
  double a = fabs((double)v);
  if (a > 448.0) a = 448.0;
  if (a == 0.0) return 0.0;
  const int e = (int)floor(log2(a));
  const double step = ldexp(1.0, e - 3 < -9 ? -9 : e - 3);
  double r = nearbyint(a / step) * step;
  if (r > 448.0) r = 448.0;
  return v < 0 ? -r : r;
}

int main(void) {
  long long checked = 0, differ = 0, scales = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : checked, differ, scales)
  for (int ha = 1; ha < 0x7F80; ++ha) {
    const float amax = from_bf16((uint32_t)ha);
    const float sc = amax / 448.f;
    if (!(sc >= 0x1p-100f) || !isfinite(sc)) continue;
    const float r = 1.0f / sc;
    ++scales;
    for (uint32_t hx = 0; hx < 0x10000; ++hx) {
      const float x = from_bf16(hx);
      if (!isfinite(x) || fabsf(x) > amax) continue;
      const float q = x * r;
      const float got = fmaf(fmaf(-sc, q, x), r, q);
      ++checked;
      if (e4m3(got) != e4m3(x / sc)) ++differ;
    }
  }
  printf("scales %lld, values %lld, differing codes %lld\n", scales, checked, differ);
  return differ != 0;
}
