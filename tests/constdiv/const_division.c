/* Host check of the quantizers' division by a constant D: q0 = fl(x c) with
 * c = fl(1/D), the residual fl(x - q0 D) by a fused multiply-add (exact), then
 * q = fl(q0 + r c) by another.  Each listed binade of non-negative binary32 x
 * is checked whole against fl(x / D), computed as the binary64 quotient
 * rounded to binary32 (no double-rounding error: x / D is never a binary32
 * midpoint nor within 2^-53 of one, since 1/D has a periodic binary
 * expansion).  Binades 0 (subnormals) to 40 cover every x whose residual
 * can be subnormal; above that every step scales exactly with x, so one
 * binade stands for all, and the top binade checks the overflow end.
 * Usage: const_division D...; prints one line per D, exit status 1 on any
 * mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_to_f(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(int argc, char** argv) {
  int fail = 0;
  for (int i = 1; i < argc; ++i) {
    const float d = (float)atof(argv[i]);
    const float c = 1.0f / d;
    unsigned long long checked = 0, bad = 0;
    for (uint32_t e = 0; e < 255; ++e) {
      if (e > 32 && e != 127 && e != 254) continue;
#pragma omp parallel for reduction(+ : checked, bad)
      for (uint32_t m = 0; m < (1u << 23); ++m) {
        const float x = bits_to_f(e << 23 | m);
        const float q0 = x * c;
        const float r = fmaf(-q0, d, x);
        const float q = fmaf(r, c, q0);
        const float ref = (float)((double)x / (double)d);
        bad += memcmp(&q, &ref, 4) != 0;
        ++checked;
      }
    }
    printf("D %g: %llu values, %llu mismatches\n", d, checked, bad);
    fail |= bad != 0;
  }
  return fail;
}
