/* Checks, on the host, the arithmetic identity the quantize kernels use in place of an IEEE fp32
 * division x / s:  r = RN(1/s);  q0 = RN(x*r);  e = fma(q0, s, -x);  q = fma(-e, r, q0)
 * (the residual is negated so that x = -0 keeps its sign).
 * For every finite BF16 x (all 65536 bit patterns) with |x| <= amax and for many scales s drawn like the quantizer's
 * (s = max(RN(amax / fmt_max), fp32(1e-12)) with amax a random finite BF16 or FP32 magnitude), it
 * compares q with x / s bit for bit, and also with random FP32 x in [-amax, amax].
 * A mismatch is only allowed where both quotients are below 2^-60 in magnitude with the same sign:
 * that happens only for |x| < ~2^-100 (the FMA residual is then not exact), and since s >= 1e-12 such
 * quotients are far below 2^-17, the smallest FP8 rounding boundary, so both encode to the same
 * signed zero.  Any other mismatch is reported and fails the run.
 * Usage: division_identity <n_scales> <seed>.  Prints "checked <n> mismatches <m> tiny <t>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)(st >> 11); }
static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t b_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(int argc, char** argv) {
  long nscales = argc > 1 ? atol(argv[1]) : 1000;
  st = argc > 2 ? strtoull(argv[2], 0, 10) * 2654435761ull + 1 : 88172645463325252ull;
  const float floor_ = f_of(0x2B8CBCCCu);
  const float fmaxs[2] = {448.0f, 57344.0f};
  long checked = 0, bad = 0, tiny = 0;
  for (long i = 0; i < nscales; ++i) {
    float fmx = fmaxs[i & 1];
    float amax;
    do {
      uint32_t b = (i % 3 == 0) ? ((rnd() & 0x7FFFu) << 16) : (rnd() & 0x7FFFFFFFu);
      amax = f_of(b);
    } while (!isfinite(amax));
    volatile float s = amax / fmx;
    if (s < floor_) s = floor_;
    volatile float r = 1.0f / s;
    for (uint32_t xb = 0; xb < 65536u + 4096u; ++xb) {
      float x;
      if (xb < 65536u) {
        x = f_of(xb << 16);
        if (!isfinite(x) || fabsf(x) > amax) continue;
      } else {
        x = f_of((rnd() & 0x7FFFFFFFu) | ((rnd() & 1u) << 31));
        if (!isfinite(x) || fabsf(x) > amax) continue;
      }
      volatile float ref = x / s;
      volatile float q0 = x * r;
      volatile float e = fmaf(q0, s, -x);
      volatile float q = fmaf(-e, r, q0);
      ++checked;
      if (b_of(q) != b_of(ref)) {
        if (fabsf(ref) < 0x1p-60f && fabsf(q) < 0x1p-60f && signbit(q) == signbit(ref)) { ++tiny; continue; }
        if (bad < 10) fprintf(stderr, "mismatch x=%a s=%a ref=%a got=%a\n", x, (float)s, (float)ref, (float)q);
        ++bad;
      }
    }
  }
  printf("checked %ld mismatches %ld tiny %ld\n", checked, bad, tiny);
  return bad != 0;
}
