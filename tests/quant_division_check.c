// Host check of the FP8 activation quantiser's division (quant_dev.h,
// quant_act_unit): the activation side of blockwise FP8 ("[Moe] Fix
// flashinfer_trtllm silently dropping swiglu_limit clamped SwiGLU
// activation", sglang PR #39920, "Modifications") divides each bf16 value x
// of a 128-column group by sc = amax / 448 (fp32, correctly rounded) and
// rounds the quotient to e4m3. The kernel forms the quotient as
//   r = RN(1 / sc), q0 = RN(x r), e = RN(fma(-q0, sc, x)), q = RN(fma(e, r, q0))
// when sc >= 2^-64 and x = 0 or |x| >= 2^-64, and divides otherwise.
// Exhaustively over every positive finite bf16 amax and every bf16 x in
// [0, amax] on that path (the sign is symmetric), q must equal the correctly
// rounded x / sc whenever that is normal, and the e4m3 code (after the +-448
// clamp, round to nearest even) must be the same always. Exit status 0 on
// success. Compiled with -ffp-contract=off so that each operation rounds.
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
static float bf(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static double e4m3(double v) {               // RNE to e4m3fn magnitude, v >= 0, v <= 448
  if (v == 0) return 0;
  int e; frexp(v, &e); e -= 1;               // v in [2^e, 2^(e+1))
  double step = e >= -6 ? ldexp(1.0, e - 3) : ldexp(1.0, -9);
  return rint(v / step) * step;
}
int main(void) {
  const float LIM = 0x1p-64f, XLIM = 0x1p-64f;   // the kernel's limits
  long checked = 0, badq = 0, badc = 0, slow = 0;
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {
    float a = bf(ab);
    volatile float sc = a / 448.0f;
    if (!(sc >= LIM)) { ++slow; continue; }
    float r = 1.0f / sc;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      float x = bf(xb);
      if (xb != 0 && !(x >= XLIM)) continue;
      float q0 = x * r;
      float e = fmaf(-q0, sc, x);
      float q = fmaf(e, r, q0);
      float ref = (float)((double)x / (double)sc);
      ++checked;
      if (memcmp(&q, &ref, 4) != 0 && ref >= 0x1p-126f) {
        if (badq < 5) printf("normal-quotient mismatch a=%a x=%a q=%a ref=%a\n", a, x, q, ref);
        ++badq;
      }
      double cq = e4m3(fmin(q, 448.0f)), cr = e4m3(fmin(ref, 448.0f));
      if (cq != cr) { if (badc < 5) printf("code mismatch a=%a x=%a\n", a, x); ++badc; }
    }
  }
  printf("checked %ld pairs: %ld normal-quotient mismatches, %ld code mismatches; %ld amax values below the limit\n",
         checked, badq, badc, slow);
  return (badq || badc) != 0;
}
