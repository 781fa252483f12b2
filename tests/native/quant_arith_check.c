// Exhaustive CPU check of the fused kernel's activation-quotient recipe.
//
// The kernel forms s = RN(amax / 448) as s0 = amax RN(1/448) corrected once with the exact
// remainder, s = fma(fma(-s0, 448, amax), RN(1/448), s0); this program checks that it equals the
// IEEE division for every bf16 amax.
// The kernel forms x / s as q = fma(x, yh, x yl) with a two-term reciprocal:
// yh = 1 / s rounded toward zero (RN(1 / s), stepped down one unit when the residual
// e = fma(-s, yh, 1) is negative) and yl = e yh >= 0, after rescaling x and s by 2^64 when
// 0 < s < 2^-64.
// For every positive bf16 amax and every bf16 x with |x| <= amax (both signs), this program checks
// that the e4m3 code (round to nearest even, saturating at 448) of that q equals the code of the
// correctly rounded IEEE division x / s.  It counts fp32 quotient mismatches separately (they may
// exist far below the e4m3 range) and exits non-zero on any code mismatch.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float bf(uint16_t b) { uint32_t u = (uint32_t)b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint8_t enc(float v) {
  const uint8_t sg = signbit(v) ? 0x80 : 0;
  const double a = fabs((double)v);
  if (a >= 464.0) return sg | 0x7E;
  if (a < 0x1p-6) {
    const long n = lrint(a * 512.0);  // ties to even (default rounding mode)
    return sg | (uint8_t)n;           // n == 8 is the smallest normal, code 0x08
  }
  int e;
  frexp(a, &e);                        // a = f 2^e, f in [0.5, 1)
  const double m = a / ldexp(1.0, e - 1) - 1.0;  // [0, 1)
  long mant = lrint(m * 8.0);
  int ex = e - 1;
  if (mant == 8) { mant = 0; ++ex; }
  int code = ((ex + 7) << 3) | (int)mant;
  if (code > 0x7E) code = 0x7E;
  return sg | (uint8_t)code;
}
int main(void) {
  long long checked = 0, bad = 0, fbad = 0, sbad = 0;
  #pragma omp parallel for reduction(+:checked,bad,fbad,sbad) schedule(dynamic)
  for (int ab = 1; ab < 0x7F80; ++ab) {
    const float am = bf((uint16_t)ab);
    const float s0 = am * (1.0f / 448.0f);
    const float s = fmaf(fmaf(-s0, 448.0f, am), 1.0f / 448.0f, s0);
    if (s != am / 448.0f) { printf("scale differs from the division: am=%a\n", am); ++sbad; }
    const float k = (s > 0.0f && s < 0x1p-64f) ? 0x1p64f : 1.0f;
    const float sk = s * k;
    float yh = 1.0f / sk;
    float e = fmaf(-sk, yh, 1.0f);
    if (e < 0.0f) {
      uint32_t u; memcpy(&u, &yh, 4); --u; memcpy(&yh, &u, 4);
      e = fmaf(-sk, yh, 1.0f);
    }
    const float yl = e * yh;
    for (int xb = 0; xb <= ab; ++xb) {
      for (int sg = 0; sg < 2; ++sg) {
        const float x = sg ? -bf((uint16_t)xb) : bf((uint16_t)xb);
        const float f = x * k;
        const float q = fmaf(f, yh, f * yl);
        const float ref = x / s;
        ++checked;
        if (q != ref || signbit(q) != signbit(ref)) ++fbad;
        if (enc(q) != enc(ref)) { if (bad < 5) printf("am=%a x=%a q=%a ref=%a\n", am, x, q, ref); ++bad; }
      }
    }
  }
  printf("pairs %lld, fp32 quotient mismatches %lld, e4m3 code mismatches %lld, scale mismatches %lld\n",
         checked, fbad, bad, sbad);
  return bad != 0 || sbad != 0;
}
