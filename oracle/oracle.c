/*
 * oracle.c -- plain, slow CPU reference for the small-M FP8 block-scale GEMM with fused
 * activation quantisation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load or call it.  It shares no
 * code, header, table or constant with the HIP library, and includes nothing from it.
 *
 * Sources (cited by page title and section):
 *   [P1] sglang "[AMD] Small-M FP8 block-scale GEMM with fused activation quant for gfx950
 *        (Qwen3.5)", section Modifications: bf16 activations are quantised to fp8 in 1x128
 *        groups with a per-group scale; the fp8 weight carries one fp32 scale per 128x128
 *        block (weight_scale_inv, shape [N/128, K/128]); each 128-wide K block's partial sum
 *        is multiplied by x_scale * w_scale in fp32; the output is bf16.
 *   [P4] sglang "[Perf] [AMD] dsv4: optional e8m0 mxscale GEMM for dense 128x128 fp8
 *        linears", sections Motivation / Modifications and the commit message: power-of-two
 *        128x128 weight scales stored as e8m0 bytes and a ue8m0 per-1x128 activation quant.
 *   The e4m3fn format itself (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 *   infinities, S.1111.111 = NaN, max 448) is the OCP 8-bit floating point format the
 *   pages' "fp8"/"float8_e4m3fn" names.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - group scale  sx = RN32(amax / 448), one IEEE fp32 division; quotient q = RN32(x / sx),
 *     one IEEE fp32 division per element; then nearest e4m3, ties to even mantissa;
 *   - values beyond 448 saturate to +-448; the sign of zero and of underflowing values is kept;
 *   - an all-zero group has scale 0 and signed-zero codes;
 *   - e8m0 activation scale: smallest power of two 2^E with amax <= 448 * 2^E ("rounded up"),
 *     E clamped to [-127, 127], byte E + 127; an all-zero group gets E = -127;
 *   - e8m0 weight scale: 2^E with E = log2(amax / 448) rounded to the nearest integer
 *     ("forced to 2^round(log2(amax/448))"), clamped to [-127, 127]; codes saturate at 448;
 *   - the product is accumulated exactly enough (fp64) and rounded once to bf16, ties to even.
 *
 * Build:  gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC oracle.c -o liboracle.so
 * (no FTZ/DAZ, no contraction: every float operation below is a single IEEE-754 operation).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------ */
/* Scalar codecs                                                                               */
/* ------------------------------------------------------------------------------------------ */

/* bf16 bit pattern -> its exact fp32 value (bf16 is the top half of an fp32). */
float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* e4m3fn byte -> exact value (OCP FP8 E4M3): subnormal m * 2^-9, normal (1 + m/8) * 2^(e-7). */
double oracle_e4m3_decode(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 0xF, m = b & 0x7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? (double)m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -mag : mag;
}

/* Values of the non-negative finite codes 0x00..0x7E, ascending (code order == value order). */
static double pos_value(int code) { return oracle_e4m3_decode((uint8_t)code); }

/* Finite value -> e4m3fn byte: nearest representable value, ties to the even code (mantissa
 * LSB 0), magnitudes at or above 448 saturate to 448, and the sign bit of the input is kept
 * (so -0.0 and negative values that round to zero give 0x80).  Input must not be NaN. */
uint8_t oracle_e4m3_encode(double f) {
  uint8_t sign = signbit(f) ? 0x80 : 0x00;
  double a = fabs(f);
  if (a >= 448.0) return sign | 0x7E;
  /* binary search for the largest code lo with value(lo) <= a; value(0x7E) = 448 > a */
  int lo = 0, hi = 0x7E;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (pos_value(mid) <= a) lo = mid; else hi = mid;
  }
  double dlo = a - pos_value(lo), dhi = pos_value(hi) - a;
  int code;
  if (dlo < dhi) code = lo;
  else if (dhi < dlo) code = hi;
  else code = (lo % 2 == 0) ? lo : hi;
  return sign | (uint8_t)code;
}

/* fp64 value -> nearest bf16 (8 significant bits, exponent range of fp32), ties to even. */
uint16_t oracle_bf16_from_double(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
  double a = fabs(v);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else if (a < ldexp(1.0, -126)) {
    r = nearbyint(ldexp(a, 133)) * ldexp(1.0, -133);        /* subnormal grid 2^-133 */
  } else {
    int e;
    frexp(a, &e);                                           /* a in [2^(e-1), 2^e) */
    r = nearbyint(ldexp(a, 8 - e)) * ldexp(1.0, e - 8);     /* 8 significant bits */
  }
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80;           /* overflow to infinity */
  float rf = (float)r;                                       /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &rf, 4);
  return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------------------------ */
/* Activation quantisation, 1x128 groups along K  [P1 Modifications; P4 commit message]        */
/* ------------------------------------------------------------------------------------------ */

/* fp32 group scales.  x: bf16 [M, ldx] row-major; q: e4m3 [M, ldq]; sx: fp32 [M, K/128]. */
void oracle_quant_act_fp32(const uint16_t* x, int64_t ldx, int M, int K,
                           uint8_t* q, int64_t ldq, float* sx) {
  int G = K / 128;
  for (int m = 0; m < M; ++m) {
    for (int g = 0; g < G; ++g) {
      const uint16_t* xg = x + (int64_t)m * ldx + 128 * g;
      uint8_t* qg = q + (int64_t)m * ldq + 128 * g;
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i) {
        float a = fabsf(oracle_bf16_to_f32(xg[i]));
        if (a > amax) amax = a;
      }
      float s = amax / 448.0f;                    /* one IEEE fp32 division */
      sx[(int64_t)m * G + g] = s;
      for (int i = 0; i < 128; ++i) {
        float xv = oracle_bf16_to_f32(xg[i]);
        if (amax == 0.0f) {
          qg[i] = signbit(xv) ? 0x80 : 0x00;
        } else {
          float quo = xv / s;                     /* one IEEE fp32 division */
          qg[i] = oracle_e4m3_encode((double)quo);
        }
      }
    }
  }
}

/* Smallest E with amax <= 448 * 2^E, clamped to [-127, 127]; amax == 0 gives -127. */
int oracle_e8m0_ceil_exponent(double amax) {
  if (amax == 0.0) return -127;
  int E = -127;
  while (E < 127 && amax > ldexp(448.0, E)) ++E;
  return E;
}

/* ue8m0 group scales: sx byte = E + 127, q = enc(x * 2^-E) (the scaling is exact). */
void oracle_quant_act_e8m0(const uint16_t* x, int64_t ldx, int M, int K,
                           uint8_t* q, int64_t ldq, uint8_t* sx) {
  int G = K / 128;
  for (int m = 0; m < M; ++m) {
    for (int g = 0; g < G; ++g) {
      const uint16_t* xg = x + (int64_t)m * ldx + 128 * g;
      uint8_t* qg = q + (int64_t)m * ldq + 128 * g;
      double amax = 0.0;
      for (int i = 0; i < 128; ++i) {
        double a = fabs((double)oracle_bf16_to_f32(xg[i]));
        if (a > amax) amax = a;
      }
      int E = oracle_e8m0_ceil_exponent(amax);
      sx[(int64_t)m * G + g] = (uint8_t)(E + 127);
      for (int i = 0; i < 128; ++i)
        qg[i] = oracle_e4m3_encode(ldexp((double)oracle_bf16_to_f32(xg[i]), -E));
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Weight quantisation, 128x128 blocks (load-time step that produces the GEMM's inputs)        */
/* ------------------------------------------------------------------------------------------ */

static float block_amax_f32(const float* w, int64_t ldw, int nb, int kb) {
  float amax = 0.0f;
  for (int r = 0; r < 128; ++r)
    for (int c = 0; c < 128; ++c) {
      float a = fabsf(w[(int64_t)(128 * nb + r) * ldw + 128 * kb + c]);
      if (a > amax) amax = a;
    }
  return amax;
}

/* fp32 block scales: sw = RN32(amax / 448), w8 = enc(RN32(w / sw)); w: fp32 [N, ldw]. */
void oracle_quant_weight_fp32(const float* w, int64_t ldw, int N, int K, uint8_t* w8, float* sw) {
  int NB = N / 128, KB = K / 128;
  /* blocks are independent: threads split them, each block's arithmetic is unchanged */
#pragma omp parallel for collapse(2) schedule(static)
  for (int nb = 0; nb < NB; ++nb)
    for (int kb = 0; kb < KB; ++kb) {
      float amax = block_amax_f32(w, ldw, nb, kb);
      float s = amax / 448.0f;
      sw[(int64_t)nb * KB + kb] = s;
      for (int r = 0; r < 128; ++r)
        for (int c = 0; c < 128; ++c) {
          int64_t n = 128 * nb + r, k = 128 * kb + c;
          float v = w[n * ldw + k];
          w8[n * K + k] = (amax == 0.0f) ? (signbit(v) ? 0x80 : 0x00)
                                          : oracle_e4m3_encode((double)(v / s));
        }
    }
}

/* E = log2(amax/448) rounded to nearest: with 448*2^F <= amax < 448*2^(F+1), take F when
 * amax < 448 * 2^(F+1/2), i.e. amax^2 < 448^2 * 2^(2F+1) (exact in fp64), else F+1.  The
 * midpoint is irrational, so there are no ties.  Clamped to [-127, 127]; amax == 0 -> -127. */
int oracle_e8m0_round_exponent(double amax) {
  if (amax == 0.0) return -127;
  /* outside the search range the clamp decides: no fp32 amax lies below 448 * 2^-300, and an
   * infinite one clamps to the top (a NaN amax has no exponent: treated like zero) */
  if (!(amax >= ldexp(448.0, -300))) return -127;
  if (isinf(amax)) return 127;
  int F = -300;
  while (!(ldexp(448.0, F) <= amax && amax < ldexp(448.0, F + 1))) ++F;
  int E = (amax * amax < 448.0 * 448.0 * ldexp(1.0, 2 * F + 1)) ? F : F + 1;
  if (E < -127) E = -127;
  if (E > 127) E = 127;
  return E;
}

/* e8m0 block scales: byte E + 127, w8 = enc(w * 2^-E), saturating at 448. */
void oracle_quant_weight_e8m0(const float* w, int64_t ldw, int N, int K, uint8_t* w8, uint8_t* sw) {
  int NB = N / 128, KB = K / 128;
#pragma omp parallel for collapse(2) schedule(static)
  for (int nb = 0; nb < NB; ++nb)
    for (int kb = 0; kb < KB; ++kb) {
      int E = oracle_e8m0_round_exponent((double)block_amax_f32(w, ldw, nb, kb));
      sw[(int64_t)nb * KB + kb] = (uint8_t)(E + 127);
      for (int r = 0; r < 128; ++r)
        for (int c = 0; c < 128; ++c) {
          int64_t n = 128 * nb + r, k = 128 * kb + c;
          w8[n * K + k] = oracle_e4m3_encode(ldexp((double)w[n * ldw + k], -E));
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* GEMM: Y[m,n] = sum_k dec(q[m,k]) * sx[m,k/128] * dec(w8[n,k]) * sw[n/128,k/128]  [P1]     */
/* ------------------------------------------------------------------------------------------ */

/* Columns [n0, n1) of the fp64 reference, written to ref[m * N + n].  threads <= 0: all. */
void oracle_gemm_fp32(const uint8_t* q, int64_t ldq, const float* sx, const uint8_t* w8,
                      const float* sw, int M, int N, int K, int n0, int n1, double* ref,
                      int threads) {
  int G = K / 128;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(static)
#endif
  for (int n = n0; n < n1; ++n) {
    for (int m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        double a = oracle_e4m3_decode(q[(int64_t)m * ldq + k]) * (double)sx[(int64_t)m * G + k / 128];
        double b = oracle_e4m3_decode(w8[(int64_t)n * K + k]) * (double)sw[(int64_t)(n / 128) * G + k / 128];
        acc += a * b;
      }
      ref[(int64_t)m * N + n] = acc;
    }
  }
  (void)threads;
}

/* Same with power-of-two scales given as e8m0 bytes (value 2^(byte - 127)). */
void oracle_gemm_e8m0(const uint8_t* q, int64_t ldq, const uint8_t* sx, const uint8_t* w8,
                      const uint8_t* sw, int M, int N, int K, int n0, int n1, double* ref,
                      int threads) {
  int G = K / 128;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(static)
#endif
  for (int n = n0; n < n1; ++n) {
    for (int m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        double a = oracle_e4m3_decode(q[(int64_t)m * ldq + k]) * ldexp(1.0, (int)sx[(int64_t)m * G + k / 128] - 127);
        double b = oracle_e4m3_decode(w8[(int64_t)n * K + k]) * ldexp(1.0, (int)sw[(int64_t)(n / 128) * G + k / 128] - 127);
        acc += a * b;
      }
      ref[(int64_t)m * N + n] = acc;
    }
  }
  (void)threads;
}

/* Round an fp64 [count] array to bf16 bit patterns. */
void oracle_round_bf16(const double* ref, int64_t count, uint16_t* y) {
  for (int64_t i = 0; i < count; ++i) y[i] = oracle_bf16_from_double(ref[i]);
}

/* Whole path for columns [n0, n1): quantise X (fp32 or e8m0 scales), GEMM, round to bf16.
 * q_work: M*K bytes, sx_work: M*K/128 fp32 or bytes; y: bf16 [M, N]; ref: fp64 [M, N]. */
void oracle_quant_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w8, const void* sw,
                       int M, int N, int K, int n0, int n1, int e8m0, uint8_t* q_work,
                       void* sx_work, double* ref, uint16_t* y, int threads) {
  if (e8m0) {
    oracle_quant_act_e8m0(x, ldx, M, K, q_work, K, (uint8_t*)sx_work);
    oracle_gemm_e8m0(q_work, K, (const uint8_t*)sx_work, w8, (const uint8_t*)sw, M, N, K, n0, n1,
                     ref, threads);
  } else {
    oracle_quant_act_fp32(x, ldx, M, K, q_work, K, (float*)sx_work);
    oracle_gemm_fp32(q_work, K, (const float*)sx_work, w8, (const float*)sw, M, N, K, n0, n1, ref,
                     threads);
  }
  for (int m = 0; m < M; ++m)
    for (int n = n0; n < n1; ++n)
      y[(int64_t)m * N + n] = oracle_bf16_from_double(ref[(int64_t)m * N + n]);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
