// smallm_fp8bs.hip -- HIP kernels and C ABI for the small-M FP8 block-scale GEMM with fused
// activation quantisation on MI355X (gfx950 / CDNA4).
//
//   Y[m, n] (bf16) = sum_k q(X)[m, k] * sx[m, k/128] * W8[n, k] * sw[n/128, k/128]
//
// What is computed follows the sglang page "[AMD] Small-M FP8 block-scale GEMM with fused
// activation quant for gfx950 (Qwen3.5)", section Modifications (1x128 activation groups with a
// per-group scale and fp8 bytes, one streaming pass over the fp8 weight, one fp8 MFMA per
// 128-wide K block, x_scale * w_scale applied to each block partial in fp32, a cross-wave LDS
// reduction to bf16), and "[Perf] [AMD] dsv4: optional e8m0 mxscale GEMM for dense 128x128 fp8
// linears" (power-of-two scales stored as e8m0 bytes, ue8m0 1x128 activation quant).  The code
// is written for gfx950 only.  Design points of this implementation:
//
//  * Packed weight layout: the columns are dealt to workgroups (one per CU for the pages' shapes),
//    each owning NA (0 or 1) group of 16 columns and a remainder group of CB (0, 2, 4 or 8)
//    columns, stored contiguously.  A 16-column x 128-K block is one 2 KiB fragment in the lane
//    order of the B operand of v_mfma_scale_f32_16x16x128_f8f6f4 (lane l = 16 c + j holds column
//    j and K bytes [32 c, 32 c + 32): bytes 0..15 in the fragment's first KiB, 16..31 in its
//    second), so a wave fetches it with two coalesced 16-byte non-temporal loads per lane.  A
//    remainder fragment packs SB = 16 / CB consecutive K blocks of the CB columns the same way.
//  * Work split: a workgroup owns its columns and all of K; K is cut into up to 8 ranges, each
//    with an MFMA wave (weight stream + MFMAs) and a quantising wave (activation loads, 1x128
//    group amax over a DPP quad of lanes, e4m3 codes and scales staged in LDS) that meet only
//    through LDS flags.  The ranges' partial sums meet once in LDS and are reduced in a fixed
//    order to bf16.
//  * Quantisation is bit-exact with q = e4m3_rne(RN(x / s)), s = RN(amax / 448): the quotient
//    is formed with a two-term reciprocal of s (a multiply and an FMA per element, after an
//    exact 2^64 rescaling of a group whose scale is below 2^-64), proven on the CPU to give the
//    code of the correctly rounded division for every pair of bf16 amax and x; the fp8 encoding
//    is the hardware round-to-nearest-even conversion, exact below 464.
//  * Deterministic reduction: per-range fp32 partials are summed through LDS in a fixed order.
//
// Build flags (see the package's build module): --offload-arch=gfx950 -O3 -ffp-contract=off,
// no fast-math, fp32 denormals kept, packed-fp32 instructions disabled.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "../../include/smallm_fp8bs.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kRowStride = 144;              // LDS row pitch of the staged e4m3 rows (128 + 16 pad)

// ---------------------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Smallest E with amax <= 448 * 2^E for a bf16 amax given as its 16-bit pattern (sign clear),
// clamped to [-127, 127].  With amax = (1 + man/128) * 2^(ef-127): 448 = 1.75 * 2^8, so
// E = ef - 135 when man/128 <= 0.75, else ef - 134.  Zero and subnormal amax give -127.
__device__ __forceinline__ int e8m0_ceil_exponent_bf16(uint32_t amax16) {
  const int ef = (int)((amax16 >> 7) & 0xFF);
  const int man = (int)(amax16 & 0x7F);
  if (ef == 0) return -127;
  const int E = ef - 135 + (man > 0x60 ? 1 : 0);
  return E < -127 ? -127 : E;
}

// Nearest-integer log2(amax / 448) for a block amax (fp32), clamped to [-127, 127].  With
// amax = ma * 2^ea, ma in [1, 2): E = ea - 8, except ea - 9 when ma < 1.75 / sqrt(2), i.e.
// ma^2 < 1.53125 (exact in fp64).  All-zero block: -127.
__device__ __forceinline__ int e8m0_round_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int ex;
  const float fr = frexpf(amax, &ex);
  const double ma = 2.0 * (double)fr;
  int E = (ex - 1) - 8 - ((ma * ma < 1.53125) ? 1 : 0);
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// x / s for the 32 elements as described below, then e4m3 with round to nearest even, four at a
// time; RESCALE multiplies x by k first.
template <bool RESCALE>
__device__ __forceinline__ void quant32_codes(const float (&xf)[32], float yh, float yl, float k,
                                              uint32_t (&w)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float f = xf[4 * j + t];
      if (RESCALE) f *= k;
      q[t] = __builtin_fmaf(f, yh, f * yl);
    }
    // the first conversion's other half is overwritten by the second, so any register serves as
    // its old value (q[0]'s own: no copy of a zero)
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], __float_as_int(q[0]), false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
    w[j] = (uint32_t)p;
  }
}

// The same from the packed bf16 pairs, widening each value where it is used.
template <bool RESCALE>
__device__ __forceinline__ void quant32_codes_packed(const u32x4 (&xv)[4], float yh, float yl, float k,
                                                     uint32_t (&w)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t d = xv[(2 * j + (t >> 1)) >> 2][(2 * j + (t >> 1)) & 3];
      float f = __uint_as_float((t & 1) ? (d & 0xFFFF0000u) : (d << 16));
      if (RESCALE) f *= k;
      q[t] = __builtin_fmaf(f, yh, f * yl);
    }
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], __float_as_int(q[0]), false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
    w[j] = (uint32_t)p;
  }
}

// max(m, |a|, |b|) in one instruction (the absolute values are source modifiers)
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(a), "v"(b), "v"(m));
  return r;
}

// Quantise 32 consecutive bf16 of one 1x128 group (this lane's quarter; the group is spread
// over a DPP quad) with an fp32 group scale.  Returns the scale, writes 32 e4m3 bytes.
//
// Group amax, two forms with the same result on finite input: WIDE widens the 32 bf16 values to
// fp32 once (exact) for both the amax (a three-input max over magnitudes, two elements per
// instruction) and the quotients, which takes fewer instructions but holds 32 more registers
// while the scale is formed; otherwise the amax is taken on the bf16 bit patterns (with the sign
// cleared, integer order is magnitude order) and each value is widened where it is used.  Either
// way the magnitudes are non-negative, so the integer order of their bit patterns is their order
// across the quad.
//
// x / s is formed with a two-term reciprocal, 1/s ~ yh + yl: yh is 1/s rounded toward zero (the
// correctly rounded reciprocal, stepped down one unit when the residual 1 - s yh comes out
// negative) and yl = (1 - s yh) yh >= 0 its remainder, so that q = fma(x, yh, x yl) costs a
// multiply and an FMA per element and keeps the sign of a zero x.  A group scale below 2^-64 is
// first rescaled by 2^64 (x 2^64 / (s 2^64) is the same quotient; both products are exact,
// |x| <= 448 s keeping x 2^64 below 448) so that 1/s stays finite.  Over every pair of bf16 amax
// and bf16 x with |x| <= amax, the e4m3 code of q equals that of the correctly rounded division
// RN(x / s): q differs from RN(x / s) only by quotients that no e4m3 rounding boundary separates.
template <bool WIDE>
__device__ __forceinline__ float quant32_fp32(const u32x4 (&xv)[4], u32x4 (&qv)[2]) {
  float xf[32];
  float am;
  if constexpr (WIDE) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t d = xv[i >> 2][i & 3];
      xf[2 * i] = __uint_as_float(d << 16);
      xf[2 * i + 1] = __uint_as_float(d & 0xFFFF0000u);
    }
    float mf = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mf = max3_abs(mf, xf[2 * i], xf[2 * i + 1]);
    am = __uint_as_float(quad_max_u32(__float_as_uint(mf)));
  } else {
    u16x2 mx = u16x2{0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, xv[i >> 2][i & 3] & 0x7FFF7FFFu));
    am = __uint_as_float(quad_max_u32(max((uint32_t)mx[0], (uint32_t)mx[1])) << 16);
  }
  // the correctly rounded fp32 quotient amax / 448, as a multiply by RN(1 / 448) and one
  // correction with the exact remainder (equal to the IEEE division for every bf16 amax, the
  // subnormal ones included, with fp32 denormals kept)
  const float s0 = am * (1.0f / 448.0f);
  const float s = __builtin_fmaf(__builtin_fmaf(-s0, 448.0f, am), 1.0f / 448.0f, s0);
  const bool tiny = s > 0.0f && s < 0x1p-64f;       // (an all-zero group needs no rescaling)
  const float k = tiny ? 0x1p64f : 1.0f;                // rescaling of a tiny group
  const float sk = s * k;
  float yh = (am > 0.0f) ? 1.0f / sk : 0.0f;            // correctly rounded reciprocal
  float e = __builtin_fmaf(-sk, yh, 1.0f);               // its residual, exact
  if (e < 0.0f) {                                        // rounded up: one unit toward zero
    yh = __uint_as_float(__float_as_uint(yh) - 1u);
    e = __builtin_fmaf(-sk, yh, 1.0f);
  }
  const float yl = e * yh;                               // all-zero group: yh = yl = 0
  uint32_t w[8];
  // the rescaling multiply only runs when some group of the wave needs it (a wave-wide vote)
  if constexpr (WIDE) {
    if (__builtin_amdgcn_ballot_w64(tiny) != 0) quant32_codes<true>(xf, yh, yl, k, w);
    else quant32_codes<false>(xf, yh, yl, k, w);
  } else {
    if (__builtin_amdgcn_ballot_w64(tiny) != 0) quant32_codes_packed<true>(xv, yh, yl, k, w);
    else quant32_codes_packed<false>(xv, yh, yl, k, w);
  }
  qv[0] = u32x4{w[0], w[1], w[2], w[3]};
  qv[1] = u32x4{w[4], w[5], w[6], w[7]};
  return s;
}

// Same group with a ue8m0 scale; returns the scale byte E + 127.
__device__ __forceinline__ uint32_t quant32_e8m0(const u32x4 (&xv)[4], u32x4 (&qv)[2]) {
  u16x2 mx = u16x2{0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t d = xv[i >> 2][i & 3] & 0x7FFF7FFFu;
    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, d));
  }
  uint32_t am = max((uint32_t)mx[0], (uint32_t)mx[1]);
  am = quad_max_u32(am);
  const int E = e8m0_ceil_exponent_bf16(am);
  uint32_t w[8];
  if (E > -127) {
    // x * 2^-E in the conversion itself: the scale operand contributes only its exponent.
    const float scale = __uint_as_float((uint32_t)(E + 127) << 23);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t d0 = xv[(2 * j) >> 2][(2 * j) & 3];
      const uint32_t d1 = xv[(2 * j + 1) >> 2][(2 * j + 1) & 3];
      v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s{0, 0}, __builtin_bit_cast(v2bf, d0), scale, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, d1), scale, true);
      w[j] = __builtin_bit_cast(uint32_t, r);
    }
  } else {
    // E = -127 (all-zero or tiny group): exact scaling by 2^127 in fp32, then convert.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t d = xv[(2 * j + h) >> 2][(2 * j + h) & 3];
        v[2 * h] = ldexpf(__uint_as_float(d << 16), 127);
        v[2 * h + 1] = ldexpf(__uint_as_float(d & 0xFFFF0000u), 127);
      }
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], p, true);
      w[j] = (uint32_t)p;
    }
  }
  qv[0] = u32x4{w[0], w[1], w[2], w[3]};
  qv[1] = u32x4{w[4], w[5], w[6], w[7]};
  return (uint32_t)(E + 127);
}

// ---------------------------------------------------------------------------------------------
// weight quantisation (load time): one workgroup per 128x128 block, 2 threads per row
// ---------------------------------------------------------------------------------------------

template <bool E8M0>
__global__ __launch_bounds__(256) void quant_weight_kernel(const float* __restrict__ w, int64_t ldw,
                                                           uint8_t* __restrict__ w8, void* __restrict__ sw,
                                                           int K) {
  __shared__ float part[4];
  const int nb = blockIdx.x, kb = blockIdx.y, KB = K >> 7;
  const int tid = threadIdx.x, r = tid >> 1, half = tid & 1;
  const float* src = w + (int64_t)(nb * 128 + r) * ldw + kb * 128 + half * 64;
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 t = *(const float4*)(src + 4 * i);
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) am = fmaxf(am, fabsf(v[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  if ((tid & 63) == 0) part[tid >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  uint32_t out[16];
  if (!E8M0) {
    const float s = am / 448.0f;
    if (tid == 0) ((float*)sw)[nb * KB + kb] = s;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float q[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) q[h] = (am > 0.0f) ? v[4 * j + h] / s : v[4 * j + h];
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
      out[j] = (uint32_t)p;
    }
  } else {
    const int E = e8m0_round_exponent(am);
    if (tid == 0) ((uint8_t*)sw)[nb * KB + kb] = (uint8_t)(E + 127);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float q[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) q[h] = fminf(fmaxf(ldexpf(v[4 * j + h], -E), -448.0f), 448.0f);
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
      out[j] = (uint32_t)p;
    }
  }
  u32x4* dst = (u32x4*)(w8 + (int64_t)(nb * 128 + r) * K + kb * 128 + half * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
}

// ---------------------------------------------------------------------------------------------
// weight (un)packing: one thread per 16-byte chunk of the packed layout
// ---------------------------------------------------------------------------------------------
//
// Packed layout.  The N columns are dealt to NWG workgroups; workgroup w owns
//   * NA (0 or 1) group of 16 columns, [16 w, 16 w + 16), stored as K / 128 fragments of 2 KiB in
//     K order (one fragment per 128-wide K block: the B operand of one 16x16x128 MFMA), and
//   * a remainder group of CB columns (0, 2, 4 or 8), [16 NA NWG + CB w, + CB), stored as
//     K / (128 SB) fragments of CB * SB * 128 bytes, each holding SB consecutive K blocks of the
//     CB columns side by side (B column j = c SB + s is column c in K block s of the fragment).
// Workgroup w's bytes are contiguous, at w * (16 NA + CB) * K: the 16-column fragments first.  In a
// fragment with NB B columns (16, or CB * SB), lane l = 16 chunk + j (j < NB) holds K bytes
// [32 chunk, 32 chunk + 32) of B column j: bytes 0..15 at (chunk NB + j) * 16 and bytes 16..31
// at NB * 64 + (chunk NB + j) * 16, so a wave fetches a fragment with two loads that each cover
// NB * 64 contiguous bytes.  The remainder group lets every workgroup stream the same number of
// bytes (one workgroup per CU) while keeping most fragments free of the padding that chaining
// several K blocks in one MFMA would cost.

struct PackGeom {
  int na, cb, sb, nwg;
};

template <bool PACK>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   int K, PackGeom g, int64_t chunks) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= chunks) return;
  const int KB = K >> 7;
  const int64_t region = (int64_t)(16 * g.na + g.cb) * K;  // bytes per workgroup
  const int64_t w = (o * 16) / region;
  const int64_t off = o * 16 - w * region;
  const int64_t abytes = (int64_t)g.na * KB * 2048;
  int64_t n, k;
  if (off < abytes) {
    const int64_t kb = off >> 11;
    const int within = (int)(off & 2047), half = within >> 10, lane = (within & 1023) >> 4;
    n = 16 * w + (lane & 15);
    k = kb * 128 + (lane >> 4) * 32 + half * 16;
  } else {
    const int nb = g.cb * g.sb, fb = nb * 128;
    const int64_t ob = off - abytes;
    const int64_t f = ob / fb;
    const int within = (int)(ob - f * fb), half = within / (fb >> 1), idx = (within % (fb >> 1)) >> 4;
    const int chunk = idx / nb, j = idx % nb;
    n = (int64_t)16 * g.na * g.nwg + (int64_t)g.cb * w + j / g.sb;
    k = (f * g.sb + j % g.sb) * 128 + chunk * 32 + half * 16;
  }
  if (PACK)
    *(u32x4*)(dst + o * 16) = *(const u32x4*)(src + n * K + k);
  else
    *(u32x4*)(dst + n * K + k) = *(const u32x4*)(src + o * 16);
}

// ---------------------------------------------------------------------------------------------
// standalone activation quantisation: a DPP quad of lanes per 1x128 group
// ---------------------------------------------------------------------------------------------

template <bool E8M0>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        void* __restrict__ sx, int M, int K) {
  const int KB = K >> 7;
  const int g = blockIdx.x * 64 + (threadIdx.x >> 2);
  const int c = threadIdx.x & 3;
  const bool valid = g < M * KB;
  const int m = valid ? g / KB : 0, kb = valid ? g % KB : 0;
  u32x4 xv[4];
  const u32x4* xp = (const u32x4*)(x + (int64_t)m * ldx + kb * 128 + c * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] = valid ? xp[i] : u32x4{0, 0, 0, 0};
  u32x4 qv[2];
  if (!E8M0) {
    const float s = quant32_fp32<false>(xv, qv);
    if (valid && c == 0) ((float*)sx)[(int64_t)m * KB + kb] = s;
  } else {
    const uint32_t e = quant32_e8m0(xv, qv);
    if (valid && c == 0) ((uint8_t*)sx)[(int64_t)m * KB + kb] = (uint8_t)e;
  }
  if (valid) {
    u32x4* qp = (u32x4*)(q + (int64_t)m * ldq + kb * 128 + c * 32);
    qp[0] = qv[0];
    qp[1] = qv[1];
  }
}

// ---------------------------------------------------------------------------------------------
// producer: RMSNorm of a row, then the 1x128 quantisation of its bf16 output
// ---------------------------------------------------------------------------------------------

constexpr int kRmsChunks = 2;  // 32 values per lane and chunk: rows of up to 2 * 32 * 256 values

// Knuth's TwoSum: a + b = t + e exactly, t = RN(a + b).
__device__ __forceinline__ void two_sum(double a, double b, double& t, double& e) {
  t = a + b;
  const double bp = t - a;
  e = (a - (t - bp)) + (b - bp);
}

// (s, c) += (s2, c2) as unevaluated sums; symmetric in its two operands.
__device__ __forceinline__ void dd_add(double& s, double& c, double s2, double c2) {
  double t, e;
  two_sum(s, s2, t, e);
  s = t;
  c = (c + c2) + e;
}

// An fp64 value from another lane of the same row of 16 (DPP), as two 32-bit moves.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

template <int CTRL>
__device__ __forceinline__ void dd_add_dpp(double& s, double& c) {
  const double s2 = dpp_f64<CTRL>(s), c2 = dpp_f64<CTRL>(c);
  dd_add(s, c, s2, c2);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ float next_up_pos(float f) { return __uint_as_float(__float_as_uint(f) + 1u); }
__device__ __forceinline__ float next_dn_pos(float f) {
  return f > 0.0f ? __uint_as_float(__float_as_uint(f) - 1u) : 0.0f;
}

// RN32((S + C) / H) for a non-negative double-double S + C: the fp64 candidate, then compared with
// the midpoints to its fp32 neighbours exactly (mid * H is exact in fp64 and, being within a
// factor of two of S, so is mid * H - S; subtracting C keeps the sign), ties to even.
__device__ __forceinline__ float rn32_dd_over(double S, double C, int H) {
  float f = (float)((S + C) / (double)H);
  if (!(f <= 3.40282347e38f)) return f;  // beyond the fp32 range: +inf
  const double dh = (double)H;
  const float up = next_up_pos(f), dn = next_dn_pos(f);
  const double du = __builtin_fma(0.5 * ((double)f + (double)up), dh, -S) - C;
  const double dl = __builtin_fma(0.5 * ((double)f + (double)dn), dh, -S) - C;
  const bool odd = (__float_as_uint(f) & 1u) != 0;
  if (du < 0.0 || (du == 0.0 && odd)) return up;
  if (f > 0.0f && (dl > 0.0 || (dl == 0.0 && odd))) return dn;
  return f;
}

// RN32(1 / sqrt(v)) for a positive fp32 v, correctly rounded: the fp64 candidate, then the
// midpoint m to each fp32 neighbour is tested exactly through the sign of m^2 v - 1 (m^2 is exact
// in fp64, the FMA rounds once).  1 / sqrt(v) is never a midpoint, so there are no ties.
__device__ __forceinline__ float rsqrt_rn32(float v) {
  if (!(v <= 3.40282347e38f)) return 0.0f;
  float r = (float)(1.0 / __builtin_sqrt((double)v));
  const double mu = 0.5 * ((double)r + (double)next_up_pos(r));
  const double ml = 0.5 * ((double)r + (double)next_dn_pos(r));
  if (__builtin_fma(mu * mu, (double)v, -1.0) < 0.0) return next_up_pos(r);
  if (__builtin_fma(ml * ml, (double)v, -1.0) > 0.0) return next_dn_pos(r);
  return r;
}

// One workgroup per row; lane l of the row holds values 32 l .. 32 l + 31 (a DPP quad per 1x128
// group).  Mean square: exact squares summed in fp64 per lane, then across lanes and waves as
// double-double sums in a fixed order, rounded once to fp32.  y = RN32(RN32(x r) w) rounded to
// bf16; q and sx are then exactly those of the standalone quantisation of y.  y and q may be
// null (not written); with q null, sx is not written either.
template <bool E8M0>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ w, float eps,
    uint16_t* __restrict__ y, int64_t ldy, uint8_t* __restrict__ q, int64_t ldq,
    void* __restrict__ sx, int H) {
  __shared__ double red[2][4];
  const int m = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int nt = blockDim.x, nw = nt >> 6;
  const int nl = H >> 5;
  const uint16_t* xr = x + (int64_t)m * ldx;
  u32x4 xv[kRmsChunks][4], wv[kRmsChunks][4];
#pragma unroll
  for (int k = 0; k < kRmsChunks; ++k) {  // the row and the weight, both loaded up front
    const int l = tid + k * nt;
    const bool valid = l < nl;
    const u32x4* xp = (const u32x4*)(xr + (int64_t)(valid ? l : 0) * 32);
    const u32x4* wp = (const u32x4*)(w + (valid ? l : 0) * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[k][i] = valid ? xp[i] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[k][i] = valid ? wp[i] : u32x4{0, 0, 0, 0};
  }
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kRmsChunks; ++k) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t d = xv[k][i >> 2][i & 3];
      const double a = (double)__uint_as_float(d << 16), b = (double)__uint_as_float(d & 0xFFFF0000u);
      s = __builtin_fma(a, a, s);
      s = __builtin_fma(b, b, s);
    }
  }
  // within each row of 16 lanes by DPP (lane pairs 1, 2, then the half and full row mirrors:
  // every lane of the row ends with the same sum), the four rows from lanes 0, 16, 32, 48 in a
  // fixed order, then across the waves through LDS
  double c = 0.0;
  dd_add_dpp<0xB1>(s, c);   // quad_perm [1, 0, 3, 2]
  dd_add_dpp<0x4E>(s, c);   // quad_perm [2, 3, 0, 1]
  dd_add_dpp<0x141>(s, c);  // row_half_mirror
  dd_add_dpp<0x140>(s, c);  // row_mirror
  double ws = readlane_f64(s, 0), wc = readlane_f64(c, 0);
  dd_add(ws, wc, readlane_f64(s, 16), readlane_f64(c, 16));
  dd_add(ws, wc, readlane_f64(s, 32), readlane_f64(c, 32));
  dd_add(ws, wc, readlane_f64(s, 48), readlane_f64(c, 48));
  if ((tid & 63) == 0) { red[0][wave] = ws; red[1][wave] = wc; }
  __syncthreads();
  double S = red[0][0], C = red[1][0];
  for (int i = 1; i < nw; ++i) dd_add(S, C, red[0][i], red[1][i]);
  const float ms = rn32_dd_over(S, C, H);
  const float r = rsqrt_rn32(ms + eps);

#pragma unroll
  for (int k = 0; k < kRmsChunks; ++k) {
    const int l = tid + k * nt;
    if (k * nt >= nl) break;  // no lane of this chunk holds values (uniform)
    const bool valid = l < nl;
    u32x4 yv[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t d = xv[k][i >> 2][i & 3], e = wv[k][i >> 2][i & 3];
      const float y0 = (__uint_as_float(d << 16) * r) * __uint_as_float(e << 16);
      const float y1 = (__uint_as_float(d & 0xFFFF0000u) * r) * __uint_as_float(e & 0xFFFF0000u);
      // fp32 -> bf16 with round to nearest even, both halves in one conversion
      yv[i >> 2][i & 3] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){y0, y1}, v2bf));
    }
    if (y != nullptr && valid) {
      u32x4* yp = (u32x4*)(y + (int64_t)m * ldy + l * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) yp[i] = yv[i];
    }
    if (q != nullptr) {
      // every lane of the wave takes part in the group reductions; invalid quads are whole groups
      u32x4 qv[2];
      const int g = l >> 2, KB = H >> 7;
      if (!E8M0) {
        const float sc = quant32_fp32<false>(yv, qv);
        if (valid && (l & 3) == 0) ((float*)sx)[(int64_t)m * KB + g] = sc;
      } else {
        const uint32_t e = quant32_e8m0(yv, qv);
        if (valid && (l & 3) == 0) ((uint8_t*)sx)[(int64_t)m * KB + g] = (uint8_t)e;
      }
      if (valid) {
        u32x4* qp = (u32x4*)(q + (int64_t)m * ldq + l * 32);
        qp[0] = qv[0];
        qp[1] = qv[1];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// the GEMM (fused quant or pre-quantised input; fp32 or e8m0 scales)
// ---------------------------------------------------------------------------------------------

enum Mode { kFusedF32 = 0, kFusedE8 = 1, kPreqF32 = 2, kPreqE8 = 3 };

constexpr int kMaxWaves = 8;  // K ranges per workgroup (an MFMA wave and a quantising wave each)

template <int MT, int RC, int MODE>
struct GemmCfg {
  static constexpr bool kE8 = (MODE & 1) != 0;
  static constexpr bool kPreq = (MODE & 2) != 0;
  static constexpr int kMP = 16 * MT;                    // rows per workgroup (M padded to the MFMA)
  static constexpr int kPasses = MT * RC;                // 16-group passes of a full round
  static constexpr int kStq = RC * kMP * kRowStride;     // one wave's staged e4m3 rows
  static constexpr int kSts = RC * kMP * 4;              // their scales (fp32, or e8m0 bytes)
  static constexpr int kRed = 2 * MT * 4 * 64 * 4;       // one wave's partial sums (both groups)
  static constexpr int kWave = ((kStq + kSts > kRed ? kStq + kSts : kRed) + 15) / 16 * 16;
  // up to 8 K ranges of two waves each (1024 threads), for one or two 16-row tiles
  static constexpr int kRanges = kMaxWaves;
  static constexpr int kSmem = kRanges * kWave;
};

// A wave-uniform fp32 value loaded through the scalar cache.
__device__ __forceinline__ float sload_f32(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

__device__ __forceinline__ float dpp_f32_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_f32_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
}

// LDS-only release / acquire between the waves of a workgroup: only LDS accesses are ordered, so
// the fences wait for the LDS counter alone, never for loads in flight from memory.
__device__ __forceinline__ void lds_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local"); }
__device__ __forceinline__ void lds_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local"); }
__device__ __forceinline__ void flag_set(uint32_t* f, uint32_t v) {
  lds_release();
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t flag_wait(uint32_t* f, uint32_t v) {
  uint32_t x;
  while ((x = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < v) __builtin_amdgcn_s_sleep(1);
  lds_acquire();
  return x;  // the count observed (at least v)
}

// One workgroup per column share of the packed layout (one per CU for the pages' shapes).  K is
// split into NW ranges of R blocks.  Each range has two waves, an MFMA wave (wave r) and a
// quantising wave (wave NW + r), and both walk it in rounds of RC blocks:
//   * the quantising wave loads the activation rows of the round's K blocks (bf16, or
//     pre-quantised bytes and scales), quantises them (a DPP quad of lanes per 1x128 group, 16
//     groups per pass, row-major over the round's K blocks, so one pass covers 16 / RC rows),
//     stages the e4m3 bytes and scales in the range's part of LDS and raises the range's flag.  It
//     runs at a higher wave priority, so that its VALU work issues ahead of the MFMA waves' on its
//     SIMD;
//   * the MFMA wave issues the round's weight block scales (scalar loads) and fragments
//     (non-temporal 16-byte buffer loads, the remainder fragments first), waits for the flag, and
//     consumes each fragment as soon as its loads have landed: a 16-column fragment is one
//     16x16x128 MFMA per M tile; a remainder fragment (CB columns x SB K blocks) is SB MFMAs, the B
//     operand masked so that MFMA s only sees the B columns of K block s (exact: the other columns
//     contribute zero).
// The two waves of a range meet only through its flags (ready: the round is staged; consumed: the
// staging area may be reused), so the weight stream never waits for the quantiser and the
// quantiser never waits for weight loads to be issued.  fp32 scales: each K block's partial is
// multiplied by x_scale * w_scale into the accumulator; e8m0 scales are the MFMA's own scale
// operands.  The MFMA waves' partial sums meet once in LDS, summed in range order.
template <int MT, int MODE, int NA, bool HASB, int SB, int RC>
__global__ __launch_bounds__(1024) void smallm_gemm_kernel(
    const void* __restrict__ a_src, int64_t lda, const void* __restrict__ sa_src,
    const uint8_t* __restrict__ wp, const void* __restrict__ sw, uint16_t* __restrict__ y,
    int64_t ldy, int M, int K, int R, int CB, int NWG, uint8_t* __restrict__ q_dbg,
    void* __restrict__ sx_dbg) {
  using Cfg = GemmCfg<MT, RC, MODE>;
  constexpr int MP = Cfg::kMP;
  constexpr int NPASS = Cfg::kPasses;
  constexpr int NV = Cfg::kPreq ? 2 : 4;  // 16-byte activation loads per lane and pass
  constexpr int rowb = Cfg::kPreq ? 1 : 2;  // bytes per activation element
  constexpr int NFB = HASB ? RC / SB : 1;  // remainder fragments per round
  static_assert(!HASB || (RC % SB == 0), "a round holds whole remainder fragments");
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::kSmem];
  __shared__ uint32_t ready[kMaxWaves], consumed[kMaxWaves];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NW = blockDim.x >> 7;  // K ranges (two waves each)
  const int KB = K >> 7;
  const int wg = blockIdx.x;
  const int m0 = blockIdx.y * MP;
  const int Mc = min(M - m0, MP);
  const bool mfma_wave = wave < NW;
  const int rg = mfma_wave ? wave : wave - NW;  // this wave's K range
  uint8_t* stq = smem + rg * Cfg::kWave;
  float* sts_f = (float*)(stq + Cfg::kStq);
  uint8_t* sts_b = stq + Cfg::kStq;
  const int kw0 = rg * R;
  const int kw1 = min(kw0 + R, KB);
  const int cols = 16 * NA + CB;

  if (tid < kMaxWaves) {
    ready[tid] = 0;
    consumed[tid] = 0;
  }
  __syncthreads();  // the flags are cleared (before any load is issued)

  if (mfma_wave) {
    // ---- MFMA wave: the weight stream of the range and its MFMAs ----
    v4f accA[MT], accA2[MT], accB[MT], accB2[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accA[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      accA2[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      accB[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      accB2[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const uint8_t* wreg = wp + (int64_t)wg * cols * K;
    const uint32_t abytes = (uint32_t)(NA * KB) * 2048u;
    const int NB = HASB ? CB * SB : 16;       // B columns of a remainder fragment
    const uint32_t fbytes = (uint32_t)NB * 128u;
    const uint32_t bbytes = HASB ? (uint32_t)(KB / SB) * fbytes : 0u;
    const __amdgpu_buffer_rsrc_t wrA = __builtin_amdgcn_make_buffer_rsrc((void*)wreg, 0, (int)abytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrB = __builtin_amdgcn_make_buffer_rsrc((void*)(wreg + abytes), 0, (int)bbytes, 0x00020000);
    const int nbA = (16 * wg) >> 7;                      // 128-column block of the 16-column group
    const int nbB = (16 * NA * NWG + CB * wg) >> 7;      // and of the remainder group
    const uint32_t swbytes = Cfg::kE8 ? (uint32_t)((cols * NWG / 128) * KB) : 0u;  // the whole [N/128, K/128] array
    const __amdgpu_buffer_rsrc_t swr = __builtin_amdgcn_make_buffer_rsrc((void*)sw, 0, (int)swbytes, 0x00020000);
    uint32_t rd = 0;
    for (int kr = kw0; kr < kw1; kr += RC, ++rd) {
      // the lane index, formed afresh in every round where the compiler cannot see through it, so
      // that lane-derived addresses are computed inside the round instead of held in registers
      // across it (a spill reload would wait for every load in flight)
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int nk = min(RC, kw1 - kr);   // K blocks of this round; the others are zero fragments
      const int jl = ln & 15;             // B column of this lane
      const int sl = jl & (SB - 1);       // its K block within a remainder fragment
      const bool bcol = jl < NB;
      const uint32_t boff = (uint32_t)(((ln >> 4) * NB + jl) * 16);
      // weight block scales of the round's K blocks, first in the queue (index clamped into the row:
      // blocks past the range multiply zero weights)
      float swA[RC], swB[RC];
      int ewA[RC], ewB[RC];
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        const int kb = min(kr + i, KB - 1);
        if (!Cfg::kE8) {
          swA[i] = NA ? sload_f32((const float*)sw + nbA * KB + kb) : 0.0f;
          swB[i] = HASB ? sload_f32((const float*)sw + nbB * KB + kb) : 0.0f;
        } else {
          ewA[i] = NA ? __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_raw_buffer_load_b8(swr, (uint32_t)(nbA * KB + kb), 0, 0)) : 0;
          ewB[i] = HASB ? __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_raw_buffer_load_b8(swr, (uint32_t)(nbB * KB + kb), 0, 0)) : 0;
        }
      }
      // the remainder fragments first: every K block of the round has an MFMA on them
      u32x4 wa[RC][2], wb[NFB][2];
#pragma unroll
      for (int f = 0; f < NFB; ++f) {
        if (HASB) {
          const uint32_t off = (f * SB < nk && bcol) ? (uint32_t)((kr / SB) + f) * fbytes + boff : bbytes;
          wb[f][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrB, off, 0, 2));
          wb[f][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrB, off + (fbytes >> 1), 0, 2));
        }
      }
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        if (NA) {
          const uint32_t off = (i < nk) ? (uint32_t)(kr + i) * 2048u + (uint32_t)ln * 16u : abytes;
          wa[i][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrA, off, 0, 2));
          wa[i][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrA, off + 1024u, 0, 2));
        }
      }
      flag_wait(&ready[rg], rd + 1);  // the round's activations are staged
      // A remainder fragment's MFMA for its K block s sees only the B columns of that block (the
      // others are masked to zero), so in the fp32 modes its result is scaled like a 16-column
      // fragment's: lanes of other K blocks hold exact zeros and add nothing.
      auto tile = [&](int i, int mt, v8i& at, v4f& sx4, int& sa) {
        const int row = mt * 16 + jl;
        const u32x4* ap = (const u32x4*)(stq + (i * MP + row) * kRowStride + (ln >> 4) * 32);
        const u32x4 a0 = ap[0], a1 = ap[1];
        at = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        if (Cfg::kE8) sa = (int)sts_b[i * MP + row];
        else sx4 = *(const v4f*)(sts_f + i * MP + mt * 16 + 4 * (ln >> 4));
      };
      // K block by K block: each activation tile is read from LDS once and feeds the remainder
      // fragment's MFMA (the fragments issued first) and the 16-column fragment's
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        if (MT == 2) {  // one K block's tiles live at a time
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
        v8i b = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        if (HASB) {
          const int f = i / SB, s = i % SB;
          b = __builtin_bit_cast(v8i, __builtin_shufflevector(wb[f][0], wb[f][1], 0, 1, 2, 3, 4, 5, 6, 7));
          if (SB > 1) {
            const uint32_t bmask = (sl == s) ? 0xFFFFFFFFu : 0u;  // lanes of K block s
#pragma unroll
            for (int d = 0; d < 8; ++d) b[d] = (int)((uint32_t)b[d] & bmask);
          }
        }
        v8i a16 = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        if (NA) a16 = __builtin_bit_cast(v8i, __builtin_shufflevector(wa[i][0], wa[i][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          v8i at;
          v4f sx4;
          int sa;
          tile(i, mt, at, sx4, sa);
          if (HASB) {
            if (Cfg::kE8) {
              v4f& acc = (i & 1) ? accB2[mt] : accB[mt];
              acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at, b, acc, 0, 0, 0, sa, 0, ewB[i]);
            } else {
              const v4f fb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at, b, v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                              0, 0, 0, 127, 0, 127);
              const float sc = swB[i];
#pragma unroll
              for (int e = 0; e < 4; ++e) accB[mt][e] = __builtin_fmaf(sx4[e] * sc, fb[e], accB[mt][e]);
            }
          }
          if (NA) {
            if (Cfg::kE8) {
              v4f& acc = (i & 1) ? accA2[mt] : accA[mt];
              acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at, a16, acc, 0, 0, 0, sa, 0, ewA[i]);
            } else {
              const v4f fa = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at, a16, v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                              0, 0, 0, 127, 0, 127);
              const float sc = swA[i];
#pragma unroll
              for (int e = 0; e < 4; ++e) accA[mt][e] = __builtin_fmaf(sx4[e] * sc, fa[e], accA[mt][e]);
            }
          }
          if (MT == 2 && !Cfg::kE8) {
            // two tiles: the block's scaled partials join the accumulators here, in the MFMAs' own
            // block (deferring them past the round's last MFMA would hold every MFMA result of
            // the round, more than a wave's 128 registers)
            asm volatile("" : "+v"(accA[mt]), "+v"(accB[mt]));
          }
        }
      }
      if (kr + RC < kw1) flag_set(&consumed[rg], rd + 1);  // the staging area may take the next round
    }
    // ---- the partial sums into the range's LDS (no longer read) ----
    float* red = (float*)stq;
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    lds_release();
    lds_acquire();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v4f pa = accA[mt];
      if (Cfg::kE8) pa += accA2[mt];
      v4f pb = accB[mt];
      if (Cfg::kE8) pb += accB2[mt];
      if (HASB && SB > 1) {
        // the SB K-block partials of a remainder column sit in SB neighbouring lanes: fold them into
        // the first, in a fixed order
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[e] += dpp_f32_xor1(pb[e]);
          if (SB > 2) pb[e] += dpp_f32_xor2(pb[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (NA) red[((0 * MT + mt) * 4 + e) * 64 + lane] = pa[e];
        if (HASB) red[((1 * MT + mt) * 4 + e) * 64 + lane] = pb[e];
      }
    }
  } else {
    // ---- quantising wave: the activations of the range, staged round by round ----
    __builtin_amdgcn_s_setprio(3);
    const uint32_t xbytes = (uint32_t)((int64_t)(Mc - 1) * lda * rowb + (int64_t)K * rowb);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)a_src + (int64_t)m0 * lda * rowb), 0, (int)xbytes, 0x00020000);
    const uint32_t sbytes_x = (uint32_t)(Mc * KB) * (Cfg::kE8 ? 1u : 4u);
    const __amdgpu_buffer_rsrc_t sxr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)sa_src + (int64_t)m0 * KB * (Cfg::kE8 ? 1 : 4)), 0, (int)sbytes_x, 0x00020000);
    // Which 32 values of its group lane c of a quad holds.  bf16 rows with one 16-row tile:
    // lane c's load i takes elements 32 i + 8 c + [0, 8), so each load instruction reads 64
    // contiguous bytes of every group (half of one 128-byte line, where lane-contiguous quarters
    // touch two lines); the quantiser is indifferent to the order, and the staged row gets the
    // lane's codes back in place.  Otherwise lane c holds the contiguous values 32 c + [0, 32):
    // pre-quantised rows take one line per group anyway, and the two-tile loop measured no
    // better interleaved.
    constexpr bool kInter = !Cfg::kPreq && MT == 1;
    constexpr int lane_elem = kInter ? 8 : 32;
    constexpr uint32_t load_step = kInter ? 64u : 16u;
    auto stage = [&](uint8_t* row, int c, const u32x4 (&qv)[2]) {
      if constexpr (!kInter) {
        u32x4* dp = (u32x4*)(row + c * 32);
        dp[0] = qv[0];
        dp[1] = qv[1];
      } else {
        // the lane's codes in element order: bytes 8 i + [0, 8) belong at 32 i + 8 c + [0, 8)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4& h = qv[i >> 1];
          *(uint2*)(row + 32 * i + 8 * c) = (i & 1) ? uint2{h[2], h[3]} : uint2{h[0], h[1]};
        }
      }
    };
    uint32_t rd = 0;
    for (int kr = kw0; kr < kw1; kr += RC, ++rd) {
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int nk = min(RC, kw1 - kr);   // K blocks of this round; the others are staged as zeros
      const int G = Mc * RC;              // groups of the round (row-major over its K blocks)
      const int grp = ln >> 2, c = ln & 3;
      u32x4 xv[NPASS][NV];
      uint32_t xs[NPASS];
      // activation loads of passes [P0, P1)
      auto load_act = [&](int P0, int P1) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          if (p < P0 || p >= P1) continue;
          if (p * 16 < G) {
            const int g = p * 16 + grp;
            const int m = g / RC, kbl = g & (RC - 1);
            const bool valid = g < G && kbl < nk;
            const uint32_t off = valid ? (uint32_t)(((int64_t)m * lda + (kr + kbl) * 128 + c * lane_elem) * rowb) : xbytes;
#pragma unroll
            for (int i = 0; i < NV; ++i)
              xv[p][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off + load_step * i, 0, 0));
            if (Cfg::kPreq) {
              const uint32_t so = valid ? (uint32_t)(m * KB + kr + kbl) * (Cfg::kE8 ? 1u : 4u) : sbytes_x;
              xs[p] = Cfg::kE8 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(sxr, so, 0, 0)
                               : __builtin_amdgcn_raw_buffer_load_b32(sxr, so, 0, 0);
            }
          }
        }
      };
      // quantisation (or staging) of passes [P0, P1) into the range's LDS
      auto quant_act = [&](int P0, int P1) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          if (p < P0 || p >= P1) continue;
          if (p * 16 < G) {
            const int g = p * 16 + grp;
            const int m = g / RC, kbl = g & (RC - 1);
            u32x4 qv[2];
            float sc = 0.0f;
            uint32_t eb = 0;
            if constexpr (!Cfg::kPreq) {
              if constexpr (Cfg::kE8) eb = quant32_e8m0(xv[p], qv);
              else sc = quant32_fp32<false>(xv[p], qv);  // one tile: every pass's loads are held at once
            } else {
              qv[0] = xv[p][0];
              qv[1] = xv[p][1];
              if (Cfg::kE8) eb = xs[p];
              else sc = __uint_as_float(xs[p]);
            }
            // K blocks past the range (a short last round) are staged too: their loads returned
            // zeros, so the MFMAs on them see zero codes and scales instead of stale LDS
            if (g < G) {
              stage(stq + (kbl * MP + m) * kRowStride, c, qv);
              if (c == 0) {
                if (Cfg::kE8) sts_b[kbl * MP + m] = (uint8_t)eb;
                else sts_f[kbl * MP + m] = sc;
              }
            }
          }
        }
      };
      if constexpr (MT == 1) {
        // one 16-row tile: every pass loaded up front
        load_act(0, NPASS);
        if (rd > 0) flag_wait(&consumed[rg], rd);  // the MFMA wave has read the previous round
        quant_act(0, NPASS);
      } else {
        // two tiles: a loop with two passes in flight, each pass loaded while the one before it is
        // quantised (the passes of a round would not fit in registers at once); passes past the
        // round read zeros past the end of the buffer and are not staged
        const int np = (G + 15) >> 4;
        u32x4 xa[NV], xb[NV];
        uint32_t sa_ = 0, sb_ = 0;
        auto load1 = [&](int p, u32x4 (&v)[NV], uint32_t& sv) {
          const int g = p * 16 + grp;
          const int m = g / RC, kbl = g & (RC - 1);
          const bool valid = g < G && kbl < nk;
          const uint32_t off = valid ? (uint32_t)(((int64_t)m * lda + (kr + kbl) * 128 + c * lane_elem) * rowb) : xbytes;
#pragma unroll
          for (int i = 0; i < NV; ++i)
            v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off + load_step * i, 0, 0));
          if (Cfg::kPreq) {
            const uint32_t so = valid ? (uint32_t)(m * KB + kr + kbl) * (Cfg::kE8 ? 1u : 4u) : sbytes_x;
            sv = Cfg::kE8 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(sxr, so, 0, 0)
                          : __builtin_amdgcn_raw_buffer_load_b32(sxr, so, 0, 0);
          }
        };
        auto quant1 = [&](int p, u32x4 (&v)[NV], uint32_t sv) {
          const int g = p * 16 + grp;
          const int m = g / RC, kbl = g & (RC - 1);
          u32x4 qv[2];
          float sc = 0.0f;
          uint32_t eb = 0;
          if constexpr (!Cfg::kPreq) {
            if constexpr (Cfg::kE8) eb = quant32_e8m0(v, qv);
            else sc = quant32_fp32<true>(v, qv);  // two tiles: two passes in flight
          } else {
            qv[0] = v[0];
            qv[1] = v[1];
            if (Cfg::kE8) eb = sv;
            else sc = __uint_as_float(sv);
          }
          if (g < G) {
            stage(stq + (kbl * MP + m) * kRowStride, c, qv);
            if (c == 0) {
              if (Cfg::kE8) sts_b[kbl * MP + m] = (uint8_t)eb;
              else sts_f[kbl * MP + m] = sc;
            }
          }
        };
        load1(0, xa, sa_);
        load1(1, xb, sb_);
        if (rd > 0) flag_wait(&consumed[rg], rd);  // the MFMA wave has read the previous round
        for (int p = 0; p < np; p += 2) {
          quant1(p, xa, sa_);
          load1(p + 2, xa, sa_);
          if (p + 1 < np) quant1(p + 1, xb, sb_);
          load1(p + 3, xb, sb_);
        }
      }
      if (!Cfg::kPreq && wg == 0 && (q_dbg != nullptr || sx_dbg != nullptr)) {
        // debug copies of the bytes and scales this round used (workgroup 0 only), from the staging area
        lds_release();
        lds_acquire();
        for (int t = ln; t < Mc * nk * 8; t += 64) {
          const int row = t / (nk * 8), rem = t - row * nk * 8, kbl = rem >> 3, part = rem & 7;
          if (q_dbg != nullptr)
            *(u32x4*)(q_dbg + (int64_t)(m0 + row) * K + (kr + kbl) * 128 + part * 16) =
                *(const u32x4*)(stq + (kbl * MP + row) * kRowStride + part * 16);
          if (sx_dbg != nullptr && part == 0) {
            if (Cfg::kE8) ((uint8_t*)sx_dbg)[(int64_t)(m0 + row) * KB + kr + kbl] = sts_b[kbl * MP + row];
            else ((float*)sx_dbg)[(int64_t)(m0 + row) * KB + kr + kbl] = sts_f[kbl * MP + row];
          }
        }
      }
      flag_set(&ready[rg], rd + 1);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  __syncthreads();
  // thread t: row t / 32 and column t % 32 of the region (at most 24 columns); every slot is read
  // and those of absent ranges are replaced by -0 (x + -0 == x) without a branch
  const int na16 = 16 * NA;
  static_assert(16 * NA + 8 <= 32, "a region has at most 32 columns");
  for (int t = tid; t < MP * 32; t += blockDim.x) {
    const int row = t >> 5, ci = t & 31;
    if (row >= Mc || ci >= cols) continue;
    const int mt = row >> 4, r = row & 15, e = r & 3;
    const bool inA = ci < na16;
    const int part = inA ? 0 : 1;
    const int li = (r >> 2) * 16 + (inA ? ci : (ci - na16) * SB);
    const float* rp = (const float*)smem + ((part * MT + mt) * 4 + e) * 64 + li;
    float v[Cfg::kRanges];
#pragma unroll
    for (int w = 0; w < Cfg::kRanges; ++w) v[w] = rp[w * (Cfg::kWave / 4)];
    float sum = v[0];
#pragma unroll
    for (int w = 1; w < Cfg::kRanges; ++w) sum += (w < NW) ? v[w] : -0.0f;
    const int col = inA ? 16 * wg + ci : na16 * NWG + CB * wg + (ci - na16);
    y[(int64_t)(m0 + row) * ldy + col] = bf16_rne(sum);
  }
}

// ---------------------------------------------------------------------------------------------
// GEMM on pre-quantised input beyond the small-M range: MFMA-tiled over M and the packed columns
// ---------------------------------------------------------------------------------------------

constexpr int kTiledRegions = 4;  // packed column regions per workgroup
constexpr int kTiledMaxKB = 128;  // K blocks the tiled kernel takes (e8m0 weight scales in two registers)
constexpr int kTThreads = 512;    // 8 waves: region w % 4, K half w / 4
constexpr int kTP = 4;            // steps of loads in flight ahead of the one in use

// Byte position of 16-byte chunk c of staged row r: rows are 128 bytes in LDS, chunks XOR-swizzled
// so that the MFMA operand reads (16 rows at a time, two chunks per lane) hit distinct banks both
// 8 and 16 lanes per LDS cycle.
__device__ __forceinline__ int tswz(int r, int c) { return r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Workgroup tile: TM rows x 4 packed column regions (the small-M kernel's per-workgroup column
// shares: 16 NA + CB columns each).  K is cut into two halves of KBh blocks (zero-padded); wave w
// multiplies region w % 4 over half w / 4, and all eight waves walk their halves in lockstep,
// one step (block s of each half) at a time, meeting at one hardware barrier per step:
//   * activations: every wave loads its share of a step's two TM x 128-byte blocks into registers
//     kTP steps ahead (16 bytes a lane, a wave-wide load covering 8 whole rows) and writes them
//     into one of two LDS slots one step ahead; the barrier publishes them, and also means every
//     wave is done with the previous step, whose slot the next writes reuse;
//   * weights: each wave streams its region's fragments of its half kTP steps ahead into
//     registers (16-column fragment per block, a remainder fragment per SB blocks);
//   * per step and 16-row subtile, one 16x16x128 MFMA on the 16-column fragment and one on the
//     remainder fragment with the B operand masked to the lanes of that K block (the others are
//     exact zeros), as the small-M kernel does.
// Scales: every row scale of the tile and the regions' weight block scales are put into LDS at
// the start.  fp32: each block's partial is multiplied by sx[row, kb] * sw[n/128, kb] into the
// accumulator; e8m0: the scales are the MFMA's scale operands.  At the end the second half's
// waves hand their accumulators to the first half's through LDS (first + second), which fold a
// remainder column's SB K-block partials (neighbouring lanes) in a fixed order and write the
// outputs.  The waves of a region past the last mirror the last one and write nothing.
template <int TM, bool E8, int NA, bool HASB, int SB>
__global__ __launch_bounds__(kTThreads) void tiled_gemm_kernel(
    const uint8_t* __restrict__ q, int64_t ldq, const void* __restrict__ sa,
    const uint8_t* __restrict__ wp, const void* __restrict__ sw, uint16_t* __restrict__ y,
    int64_t ldy, int M, int K, int CB, int NWG) {
  constexpr int NSUB = TM / 16;           // 16-row MFMA subtiles
  constexpr int NLD = TM / 32;            // activation loads per wave and step (2 TM x 8 chunks)
  constexpr int SXP = TM + 4;             // LDS pitch of a K block's row scales (16-byte aligned)
  constexpr int HALF = TM * 128;          // bytes of one staged K block
  constexpr int SLOT = 2 * HALF;          // one step: block s of each half
  constexpr int P = kTP;
  constexpr int UJ = 2 * P;               // steps per loop iteration (the register slots cycle whole)
  // remainder fragment slots: a fragment is loaded P steps before its first block, while the
  // slot's previous fragment may still be in use (two sets of P / SB when SB > 1)
  constexpr int NBS = !HASB ? 1 : SB == 1 ? P : 2 * P / SB;
  static_assert(P % SB == 0, "remainder fragments are loaded at whole-fragment steps");
  __shared__ __attribute__((aligned(16))) uint8_t ring[2 * SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t sxs[kTiledMaxKB * SXP];  // row scales, [kb][row]
  __shared__ uint32_t swl[kTiledRegions][2][kTiledMaxKB];                  // weight block scales
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave & 3, kh = wave >> 2;  // region in the tile, K half
  const int KB = K >> 7;
  // blocks per half: a whole number of loop iterations (the padded blocks are zero weights and
  // zero activations)
  const int KBh = ((KB + 1) / 2 + UJ - 1) / UJ * UJ;
  const int m0 = blockIdx.y * TM;
  const int Mt = min(TM, M - m0);
  constexpr uint32_t es = E8 ? 1u : 4u;

  // ---- scales into LDS (issued first; written after the first loads are on their way) ----
  const int nsx = Mt * KB;
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)sa + (int64_t)m0 * KB * es), 0, nsx * (int)es, 0x00020000);
  auto load_sx = [&](uint32_t (&v)[4], int e0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + kTThreads * j + tid;
      const uint32_t o = (e < nsx) ? (uint32_t)e * es : (uint32_t)nsx * es;
      v[j] = E8 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(srsrc, o, 0, 0) : __builtin_amdgcn_raw_buffer_load_b32(srsrc, o, 0, 0);
    }
  };
  // unconditional stores (a conditional one lets the compiler sink its load past the loads issued
  // after it): elements past the tile go to a pad entry nothing reads.  Row e / KB by a float
  // multiply: for an element of the tile (e < TM KB <= 8192), (e + 1/2) / KB < 64 lies at least
  // 1/(2 KB) >= 1/256 from an integer, and the product with the reciprocal (a few units of 2^-24
  // relative) is within 2^-16 of it, so it floors to the exact quotient.
  const float rkb = __builtin_amdgcn_rcpf((float)KB);
  auto store_sx = [&](const uint32_t (&v)[4], int e0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + kTThreads * j + tid;
      const int row = (int)(((float)e + 0.5f) * rkb), kb = e - row * KB;
      sxs[(e < nsx) ? kb * SXP + row : TM] = v[j];
    }
  };
  // weight block scales: wave w takes region w / 2, row (A or remainder) w % 2, K blocks lane and
  // lane + 64 (wave-uniform, so the buffer resource is a scalar one)
  const int sreg = min((int)blockIdx.x * kTiledRegions + (wave >> 1), NWG - 1);
  const int snb = (wave & 1) ? (16 * NA * NWG + CB * sreg) >> 7 : (16 * sreg) >> 7;
  const bool sown = (wave & 1) ? HASB : (NA != 0);
  const __amdgpu_buffer_rsrc_t swsr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)sw + (int64_t)snb * KB * es), 0, sown ? KB * (int)es : 0, 0x00020000);
  uint32_t sv[2], xv[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t k = (uint32_t)lane + 64u * h;
    sv[h] = E8 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(swsr, k, 0, 0) : __builtin_amdgcn_raw_buffer_load_b32(swsr, k * 4u, 0, 0);
  }
  load_sx(xv, 0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- activations: wave w's load l of a step holds LDS bytes [(8 l + w) KiB, +1 KiB) of the
  // slot: half h = (8 l + w) / (TM / 8), rows 8 ((8 l + w) % (TM / 8)) .. + 7, 16 bytes a lane
  const uint32_t abytes = (uint32_t)((int64_t)(Mt - 1) * ldq + K);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(q + (int64_t)m0 * ldq), 0, (int)abytes, 0x00020000);
  uint32_t arow[NLD];
  int ahalf[NLD];
#pragma unroll
  for (int l = 0; l < NLD; ++l) {
    const int u = 8 * l + wave;                    // KiB of the slot
    ahalf[l] = u / (TM / 8);
    const int row = (u % (TM / 8)) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);  // the chunk this lane's bytes hold
    arow[l] = (row < Mt) ? (uint32_t)((int64_t)row * ldq + c * 16) : abytes;
  }
  u32x4 ar[P][NLD];
  auto load_act = [&](int slot, int st) {
#pragma unroll
    for (int l = 0; l < NLD; ++l) {
      const int kb = ahalf[l] * KBh + st;
      const uint32_t o = (kb < KB) ? arow[l] + (uint32_t)kb * 128u : abytes;  // past the end: zeros
      ar[slot][l] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, o, 0, 0));
    }
  };
  auto store_act = [&](int slot, int st) {
    uint8_t* dst = ring + (st & 1) * SLOT + wave * 1024 + lane * 16;
#pragma unroll
    for (int l = 0; l < NLD; ++l) *(u32x4*)(dst + 8 * 1024 * l) = ar[slot][l];
  };

  // ---- weights of this wave's region and half ----
  const int reg = min((int)blockIdx.x * kTiledRegions + rw, NWG - 1);
  const bool owner = (int)(blockIdx.x * kTiledRegions + rw) < NWG;
  const int cols = 16 * NA + CB;
  const int NB = HASB ? CB * SB : 16;  // B columns of a remainder fragment
  const int jl = lane & 15;
  const int sl = jl & (SB - 1);        // K block of this lane within a remainder fragment
  const bool bcol = jl < NB;
  const uint8_t* wreg = wp + (int64_t)reg * cols * K;
  const uint32_t wabytes = (uint32_t)(NA * KB) * 2048u;
  const uint32_t fbytes = (uint32_t)NB * 128u;
  const uint32_t wbbytes = HASB ? (uint32_t)(KB / SB) * fbytes : 0u;
  const __amdgpu_buffer_rsrc_t wrA = __builtin_amdgcn_make_buffer_rsrc((void*)wreg, 0, (int)wabytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrB = __builtin_amdgcn_make_buffer_rsrc((void*)(wreg + wabytes), 0, (int)wbbytes, 0x00020000);
  const uint32_t boff = bcol ? (uint32_t)(((lane >> 4) * NB + jl) * 16) : wbbytes;
  const int kb0 = kh * KBh;            // this wave's first K block
  u32x4 wa[P][2], wb[NBS][2];
  // weight loads through the caches (not non-temporal): the row tiles of one column tile run on
  // one XCD and read the same fragments, so all but the first are L2 hits
  auto load_wa = [&](int slot, int kb) {
    if (NA) {
      const uint32_t o = (kb < KB) ? (uint32_t)kb * 2048u + (uint32_t)lane * 16u : wabytes;
      wa[slot][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrA, o, 0, 0));
      wa[slot][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrA, o + 1024u, 0, 0));
    }
  };
  auto load_wb = [&](int slot, int f) {
    if (HASB) {
      const uint32_t o = (f * SB < KB && bcol) ? (uint32_t)f * fbytes + boff : wbbytes;
      wb[slot][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrB, o, 0, 0));
      wb[slot][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrB, o + (fbytes >> 1), 0, 0));
    }
  };
  // the first P steps, in the order every later step issues its loads (activations, 16-column
  // fragment, remainder fragment at its first block)
#pragma unroll
  for (int t = 0; t < P; ++t) {
    load_act(t, t);
    load_wa(t, kb0 + t);
    if (t % SB == 0) load_wb((t / SB) % NBS, (kb0 + t) / SB);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) swl[tid >> 7][(tid >> 6) & 1][lane + 64 * h] = sv[h];
  store_sx(xv, 0);
  // a tile with more than 2048 scales (K beyond 4096 at 64 rows): the rest, waiting each batch
  for (int e0 = 2048; e0 < nsx; e0 += 2048) {
    load_sx(xv, e0);
    store_sx(xv, e0);
  }
  // the padded K blocks: zero scales (their activations and weights are zeros too)
  for (int e = tid; e < (2 * KBh - KB) * TM; e += kTThreads) sxs[(KB + e / TM) * SXP + e % TM] = 0u;
  const uint32_t* swr = &swl[rw][0][0];
  // step 0's activations into their slot, and step P's loads into the registers they leave
  store_act(0, 0);
  load_act(0, P);

  v4f accA[NSUB], accB[NSUB];
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    accA[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    accB[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  for (int s0 = 0; s0 < KBh; s0 += UJ) {
#pragma unroll
    for (int u = 0; u < UJ; ++u) {
      const int st = s0 + u, kb = kb0 + st;
      // after the barrier every wave's writes of this step's activations are visible, and every
      // wave is done with the previous step, whose slot takes the next step's
      lds_release();
      __builtin_amdgcn_s_barrier();
      lds_acquire();
      store_act((u + 1) % P, st + 1);
      load_act((u + 1) % P, st + 1 + P);
      v8i at[NSUB];
      int sar[NSUB];
      v4f sx4[NSUB];
      v8i bA = v8i{0, 0, 0, 0, 0, 0, 0, 0}, bB = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      const uint8_t* blk = ring + (st & 1) * SLOT + kh * HALF;
      const uint32_t* ss = sxs + kb * SXP;
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
        const int r = i * 16 + jl, c = (lane >> 4) * 2;
        const u32x4 a0 = *(const u32x4*)(blk + tswz(r, c)), a1 = *(const u32x4*)(blk + tswz(r, c + 1));
        at[i] = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        if (E8) sar[i] = (int)ss[r];
        else sx4[i] = *(const v4f*)(ss + i * 16 + 4 * (lane >> 4));
      }
      if (NA) bA = __builtin_bit_cast(v8i, __builtin_shufflevector(wa[u % P][0], wa[u % P][1], 0, 1, 2, 3, 4, 5, 6, 7));
      if (HASB) {
        const int bs = (u / SB) % NBS;
        bB = __builtin_bit_cast(v8i, __builtin_shufflevector(wb[bs][0], wb[bs][1], 0, 1, 2, 3, 4, 5, 6, 7));
        if (SB > 1) {
          const uint32_t bmask = (sl == u % SB) ? 0xFFFFFFFFu : 0u;  // lanes of this K block
#pragma unroll
          for (int d = 0; d < 8; ++d) bB[d] = (int)((uint32_t)bB[d] & bmask);
        }
      }
      const int ea = NA ? (int)swr[kb] : 0;  // past the row: zeros
      const int eb = HASB ? (int)swr[kTiledMaxKB + kb] : 0;
      if (E8) {
#pragma unroll
        for (int i = 0; i < NSUB; ++i) {
          if (NA) accA[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at[i], bA, accA[i], 0, 0, 0, sar[i], 0, ea);
          if (HASB) accB[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at[i], bB, accB[i], 0, 0, 0, sar[i], 0, eb);
        }
      } else {
        v4f fa[NSUB], fb[NSUB];
#pragma unroll
        for (int i = 0; i < NSUB; ++i) {
          if (NA) fa[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at[i], bA, v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                            0, 0, 0, 127, 0, 127);
          if (HASB) fb[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at[i], bB, v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                              0, 0, 0, 127, 0, 127);
        }
        const float swA = __int_as_float(ea), swB = __int_as_float(eb);  // the fp32 scales' bits
#pragma unroll
        for (int i = 0; i < NSUB; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (NA) accA[i][e] = __builtin_fmaf(sx4[i][e] * swA, fa[i][e], accA[i][e]);
            if (HASB) accB[i][e] = __builtin_fmaf(sx4[i][e] * swB, fb[i][e], accB[i][e]);
          }
      }
      // the step's results join the accumulators in the MFMAs' own basic block
#pragma unroll
      for (int i = 0; i < NSUB; ++i) asm volatile("" : "+v"(accA[i]), "+v"(accB[i]));
      __builtin_amdgcn_sched_barrier(0);
      // the registers of this step's fragments take the fragments P steps on
      load_wa(u % P, kb + P);
      if ((u + P) % SB == 0) load_wb(((u + P) / SB) % NBS, (kb + P) / SB);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // 16 wait states on every path before the accumulators are read (the loop ends in branches)
#pragma unroll
  for (int i = 0; i < NSUB; ++i) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(accA[i]), "+v"(accB[i]));
  // this lane's first output row (rows 4 (lane / 16) + e of each subtile), formed before the
  // barriers
  uint16_t* const ylane = y + (int64_t)(m0 + 4 * (lane >> 4)) * ldy;
  // every wave is done reading the ring: it now takes the second half's accumulators
  lds_release();
  __builtin_amdgcn_s_barrier();
  lds_acquire();
  float* red = (float*)ring + rw * (2 * NSUB * 4 * 64);
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < NSUB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (NA) red[(i * 4 + e) * 64 + lane] = accA[i][e];
        if (HASB) red[((NSUB + i) * 4 + e) * 64 + lane] = accB[i][e];
      }
  }
  lds_release();
  __builtin_amdgcn_s_barrier();
  lds_acquire();
  if (kh == 1 || !owner) return;
#pragma unroll
  for (int i = 0; i < NSUB; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (NA) accA[i][e] += red[(i * 4 + e) * 64 + lane];
      if (HASB) accB[i][e] += red[((NSUB + i) * 4 + e) * 64 + lane];
    }
  // output: lane l holds MFMA column l % 16, rows 4 (l / 16) + e of each subtile
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    v4f pb = accB[i];
    if (HASB && SB > 1) {
      // the SB K-block partials of a remainder column sit in SB neighbouring lanes: fold them
      // into the first, in a fixed order
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] += dpp_f32_xor1(pb[e]);
        if (SB > 2) pb[e] += dpp_f32_xor2(pb[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = i * 16 + 4 * (lane >> 4) + e;
      if (r < Mt) {
        uint16_t* const yr = ylane + (int64_t)(i * 16 + e) * ldy;
        if (NA) yr[16 * reg + jl] = bf16_rne(accA[i][e]);
        if (HASB && bcol && sl == 0) yr[16 * NA * NWG + CB * reg + jl / SB] = bf16_rne(pb[e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_mnk(int M, int N, int K) {
  if (M < 1 || M > SMALLM_FP8BS_MAX_M) return SMALLM_ERR_SHAPE;
  if (N <= 0 || K <= 0 || (N & 127) || (K & 127)) return SMALLM_ERR_SHAPE;
  return SMALLM_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? SMALLM_OK : SMALLM_ERR_HIP; }

// ---------------------------------------------------------------------------------------------
// streaming-read reference (the achievable HBM read time of a buffer, for the roofline)
// ---------------------------------------------------------------------------------------------

constexpr int kFloorWGs = 256;    // one workgroup per CU
constexpr int kFloorWaves = 8;
constexpr int kFloorLoads = 10;   // 16-byte loads per lane in flight (a 20 MiB buffer: all of them)

// Workgroup g reads its contiguous share of `bytes` in 1 KiB units (a wave-wide 16-byte load per
// unit), wave w taking units w, w + 8, ..., kFloorLoads at a time, every load issued before any is
// consumed; non-temporal, bounds-checked (units past the end read zeros).  The loaded words are
// folded into one value per wave that is written out only if it equals a constant no random data
// produces, so the loads cannot be dropped and nothing else is written.
__global__ __launch_bounds__(64 * kFloorWaves) void read_floor_kernel(const uint8_t* __restrict__ buf,
                                                                      uint32_t bytes, uint32_t units,
                                                                      uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)buf, 0, (int)bytes, 0x00020000);
  const uint32_t base = (blockIdx.x * units + (uint32_t)wave) * 1024u + (uint32_t)lane * 16u;
  const uint32_t nu = (units > (uint32_t)wave) ? (units - (uint32_t)wave + kFloorWaves - 1) / kFloorWaves : 0u;
  u32x4 x = u32x4{0u, 0u, 0u, 0u};
  for (uint32_t b = 0; b < nu; b += kFloorLoads) {
    u32x4 r[kFloorLoads];
#pragma unroll
    for (int j = 0; j < kFloorLoads; ++j) {
      const uint32_t i = b + (uint32_t)j;
      const uint32_t off = (i < nu) ? base + i * (kFloorWaves * 1024u) : bytes;
      r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
    }
#pragma unroll
    for (int j = 0; j < kFloorLoads; ++j) x ^= r[j];
  }
  const uint32_t v = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (v == 0x9E3779B9u) sink[blockIdx.x * kFloorWaves + wave] = v;
}

constexpr int kTargetWGs = 256;  // one workgroup per CU of the MI355X

// The packed layout and the launch it implies for an [N, K] weight.
struct Layout {
  int nwg;     // workgroups along N
  int na;      // 16-column groups per workgroup (0 or 1)
  int cb;      // remainder columns per workgroup (0, 2, 4 or 8)
  int sb;      // K blocks per remainder fragment
  int r;       // K blocks per wave
  int rc;      // K blocks per round of a wave
  int nw;      // waves per workgroup
};

// Waves split K: each takes r K blocks (the smallest power of two with r * 8 >= K / 128), in
// rounds of at most 4.  Columns: N a multiple of 4096 gives one 16-column group per workgroup
// (N / 16 workgroups, a multiple of 256); N = 256 (16 a + c) with a <= 1 and c in {2, 4, 8}
// gives 256 workgroups, each with a 16-column groups and a c-column remainder group (the pages'
// 5120, 4608 and 2048-column shards: every CU streams the same bytes); any other N falls back to
// one 16-column group per workgroup.
Layout layout_for(int N, int K) {
  const int KB = K / 128;
  Layout L;
  int r = 1;
  while (r * kMaxWaves < KB) r <<= 1;
  L.r = r;
  L.rc = r < 4 ? r : 4;
  L.nw = (KB + r - 1) / r;
  L.na = 1;
  L.cb = 0;
  L.sb = 1;
  L.nwg = N / 16;
  if (N % 4096 != 0 && N % 256 == 0) {
    const int units = N / 256, a = units / 16, c = units % 16;
    if (a <= 1 && (c == 2 || c == 4 || c == 8)) {
      const int sb = min(16 / c, L.rc);
      if (KB % sb == 0) {
        L.na = a;
        L.cb = c;
        L.sb = sb;
        L.nwg = kTargetWGs;
      }
    }
  }
  return L;
}

uint32_t layout_id_for(int N, int K) {
  const Layout L = layout_for(N, K);
  return 0x46390000u | ((uint32_t)L.na << 12) | ((uint32_t)L.cb << 4) | (uint32_t)L.sb;
}

// The K split a launch takes: the layout's ranges of r blocks in rounds of rc, except that up to 4
// rows on a short K (at most 16 blocks) take ranges of twice the blocks (half the waves: the
// per-workgroup cost of the extra waves outweighs their shorter ranges there; measured on
// 4096x2048, 3.8 against 4.1 us).  The remainder fragments' SB blocks still divide the round.
Layout launch_split(const Layout& L, int KB, int M) {
  Layout S = L;
  if (M <= 4 && KB <= 16 && (L.cb == 0 || L.sb >= 2)) {
    S.r = 2 * L.r;
    S.rc = S.r < 4 ? S.r : 4;
  }
  S.nw = (KB + S.r - 1) / S.r;
  return S;
}

template <int MODE, int MT, int NA, bool HASB, int SB, int RC>
void launch_k(int R, int nw, const Layout& L, dim3 grid, hipStream_t stream, const void* a, int64_t lda,
              const void* sa, const uint8_t* wp, const void* sw, uint16_t* y, int64_t ldy, int M, int K,
              uint8_t* q_dbg, void* sx_dbg) {
  hipLaunchKernelGGL((smallm_gemm_kernel<MT, MODE, NA, HASB, SB, RC>), grid, dim3(128 * nw), 0, stream, a, lda,
                     sa, wp, sw, y, ldy, M, K, R, L.cb, L.nwg, q_dbg, sx_dbg);
}

// The launch for a K split (launch_split), for one or two 16-row tiles.
template <int MODE, int MT>
void launch_mt(const Layout& L, int K, dim3 grid, hipStream_t stream, const void* a, int64_t lda, const void* sa,
               const uint8_t* wp, const void* sw, uint16_t* y, int64_t ldy, int M, uint8_t* q_dbg,
               void* sx_dbg) {
  const int R = L.r;
  const int nw = L.nw;
#define SMALLM_K(na, hasb, sb, rc) \
  launch_k<MODE, MT, na, hasb, sb, rc>(R, nw, L, grid, stream, a, lda, sa, wp, sw, y, ldy, M, K, q_dbg, sx_dbg)
  if (L.cb == 0) {
    if (L.rc == 1) SMALLM_K(1, false, 1, 1);
    else if (L.rc == 2) SMALLM_K(1, false, 1, 2);
    else SMALLM_K(1, false, 1, 4);
  } else if (L.na == 1) {
    if (L.rc == 1) SMALLM_K(1, true, 1, 1);
    else if (L.rc == 2) SMALLM_K(1, true, 2, 2);
    else if (L.sb == 4) SMALLM_K(1, true, 4, 4);
    else SMALLM_K(1, true, 2, 4);
  } else {
    if (L.rc == 1) SMALLM_K(0, true, 1, 1);
    else if (L.rc == 2) SMALLM_K(0, true, 2, 2);
    else if (L.sb == 4) SMALLM_K(0, true, 4, 4);
    else SMALLM_K(0, true, 2, 4);
  }
#undef SMALLM_K
}

constexpr int kTiledFromM = 32;  // M above which the pre-quantised GEMM is tiled

// Rows per workgroup tile of the tiled kernel at M rows on layout L.  Up to 128 rows 32-row tiles:
// on the pages' shapes (64 tiles of four column regions) they give 128-256 workgroups where
// 64-row tiles give 64-128, half the CUs idle.  Above 128 rows 64-row tiles (half the weight
// re-reads), except on layouts without a 16-column group, whose 32-row kernel fits two
// workgroups per CU.  Measured (GEMM alone, graph replay over 24 cold copies, us, 32 / 64-row
// tiles): 4096x2048 at 96 / 128 / 192 / 256 rows 5.8 / 7.8, 5.9 / 7.9, 8.0 / 8.0, 8.5 / 8.3;
// 5120x4096 12.0 / 15.7, 12.1 / 16.0, 19.4 / 16.1, 20.4 / 17.3; 4608x4096 like 5120x4096;
// 2048x4096 7.4 / 10.8, 7.7 / 10.9, 10.3 / 10.9, 10.9 / 11.2.
int tiled_tm(int M, const Layout& L) { return (M <= 128 || L.na == 0) ? 32 : 64; }

// The tiled kernel takes the shape: at most 128 K blocks (its e8m0 weight scales sit in two
// registers) and a tile's activation rows inside a 32-bit buffer offset.
bool tiled_ok(int M, int K, int64_t ldq, const Layout& L) {
  return M > kTiledFromM && K / 128 <= kTiledMaxKB &&
         (ldq * (tiled_tm(M, L) - 1) + K) < ((int64_t)1 << 31);
}

template <bool E8, int TM>
void launch_tiled_tm(const Layout& L, int M, int K, const uint8_t* q, int64_t ldq, const void* sa,
                     const uint8_t* wp, const void* sw, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const dim3 grid((L.nwg + kTiledRegions - 1) / kTiledRegions, (M + TM - 1) / TM);
#define TILED_K(na, hasb, sb)                                                                        \
  hipLaunchKernelGGL((tiled_gemm_kernel<TM, E8, na, hasb, sb>), grid, dim3(kTThreads), 0, stream, q, ldq, \
                     sa, wp, sw, y, ldy, M, K, L.cb, L.nwg)
  if (L.cb == 0) TILED_K(1, false, 1);
  else if (L.na == 1) {
    if (L.sb == 1) TILED_K(1, true, 1);
    else if (L.sb == 2) TILED_K(1, true, 2);
    else TILED_K(1, true, 4);
  } else {
    if (L.sb == 1) TILED_K(0, true, 1);
    else if (L.sb == 2) TILED_K(0, true, 2);
    else TILED_K(0, true, 4);
  }
#undef TILED_K
}

template <bool E8>
void launch_tiled(const Layout& L, int M, int K, const uint8_t* q, int64_t ldq, const void* sa,
                  const uint8_t* wp, const void* sw, uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (tiled_tm(M, L) == 32) launch_tiled_tm<E8, 32>(L, M, K, q, ldq, sa, wp, sw, y, ldy, stream);
  else launch_tiled_tm<E8, 64>(L, M, K, q, ldq, sa, wp, sw, y, ldy, stream);
}

template <int MODE>
int launch_gemm(const void* a, int64_t lda, const void* sa, const uint8_t* wp, const void* sw,
                uint16_t* y, int64_t ldy, int M, int N, int K, uint8_t* q_dbg, void* sx_dbg,
                hipStream_t stream) {
  const Layout L = layout_for(N, K);
  if ((MODE & 2) && tiled_ok(M, K, lda, L)) {
    // pre-quantised input beyond the small-M range: every weight fragment is read by
    // ceil(M / TM) workgroups instead of ceil(M / 32) small-M workgroups
    launch_tiled<(MODE & 1) != 0>(L, M, K, (const uint8_t*)a, lda, sa, wp, sw, y, ldy, stream);
    return launch_status();
  }
  const int MT = (M <= 16) ? 1 : 2;
  const int MP = 16 * MT;
  const dim3 grid(L.nwg, (M + MP - 1) / MP);
  const Layout S = launch_split(L, K / 128, M);
  if (MT == 1) launch_mt<MODE, 1>(S, K, grid, stream, a, lda, sa, wp, sw, y, ldy, M, q_dbg, sx_dbg);
  else launch_mt<MODE, 2>(S, K, grid, stream, a, lda, sa, wp, sw, y, ldy, M, q_dbg, sx_dbg);
  return launch_status();
}

int check_gemm_args(const void* a, int64_t lda, int a_elem_bytes, const void* sa_or_null_ok,
                    bool need_sa, const uint8_t* wp, uint32_t layout_id, const void* sw,
                    const uint16_t* y, int64_t ldy, int M, int N, int K) {
  if (!a || !wp || !sw || !y || (need_sa && !sa_or_null_ok)) return SMALLM_ERR_INVALID;
  int st = check_mnk(M, N, K);
  if (st) return st;
  if (lda < K || ldy < N) return SMALLM_ERR_SHAPE;
  if ((lda * 31 + K) * a_elem_bytes >= ((int64_t)1 << 31)) return SMALLM_ERR_SHAPE;  // 32-row window
  if (!aligned16(a) || ((lda * a_elem_bytes) & 15) || !aligned16(wp) || ((uintptr_t)y & 1u))
    return SMALLM_ERR_ALIGN;
  if (layout_id != layout_id_for(N, K)) return SMALLM_ERR_LAYOUT;
  return SMALLM_OK;
}

template <bool PACK>
void launch_pack(const uint8_t* src, uint8_t* dst, int N, int K, hipStream_t stream) {
  const int64_t chunks = (int64_t)N * K / 16;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  const Layout L = layout_for(N, K);
  const PackGeom g{L.na, L.cb, L.sb, L.nwg};
  hipLaunchKernelGGL((pack_kernel<PACK>), grid, dim3(256), 0, stream, src, dst, K, g, chunks);
}

}  // namespace

extern "C" {

int smallm_fp8bs_abi_version(void) { return SMALLM_FP8BS_ABI_VERSION; }

int smallm_fp8bs_read_floor(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return SMALLM_ERR_INVALID;
  if (bytes <= 0 || bytes > ((int64_t)1 << 30)) return SMALLM_ERR_SHAPE;
  if (((uintptr_t)buf & 15) != 0) return SMALLM_ERR_ALIGN;
  const uint32_t units = (uint32_t)((bytes + (int64_t)kFloorWGs * 1024 - 1) / ((int64_t)kFloorWGs * 1024));
  hipLaunchKernelGGL(read_floor_kernel, dim3(kFloorWGs), dim3(64 * kFloorWaves), 0, (hipStream_t)stream,
                     (const uint8_t*)buf, (uint32_t)bytes, units, sink);
  return launch_status();
}

uint32_t smallm_fp8bs_weight_layout_id(int N, int K) {
  if (N <= 0 || K <= 0 || (N & 127) || (K & 127)) return 0;
  return layout_id_for(N, K);
}

const char* smallm_fp8bs_strerror(int status) {
  switch (status) {
    case SMALLM_OK: return "ok";
    case SMALLM_ERR_INVALID: return "a required pointer is NULL";
    case SMALLM_ERR_SHAPE: return "shape out of range (1 <= M <= 256, N and K multiples of 128, ld >= row length)";
    case SMALLM_ERR_ALIGN: return "pointer or row pitch not 16-byte aligned";
    case SMALLM_ERR_LAYOUT: return "packed weight layout id does not match this library and shape";
    case SMALLM_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int smallm_fp8bs_launch_plan(int M, int N, int K, int* plan8) {
  if (!plan8) return SMALLM_ERR_INVALID;
  int st = check_mnk(M, N, K);
  if (st) return st;
  const Layout L = layout_for(N, K);
  const int MT = (M <= 16) ? 1 : 2;
  const Layout S = launch_split(L, K / 128, M);  // as launch_gemm takes it
  const int v[8] = {S.nwg, S.na, S.cb, S.sb, S.r, S.rc, S.nw, MT};
  for (int i = 0; i < 8; ++i) plan8[i] = v[i];
  return SMALLM_OK;
}

int smallm_fp8bs_supported(int M, int N, int K, int64_t ldx) {
  int st = check_mnk(M, N, K);
  if (st) return st;
  if (ldx < K) return SMALLM_ERR_SHAPE;
  if ((ldx * 2) & 15) return SMALLM_ERR_ALIGN;
  return SMALLM_OK;
}

int smallm_fp8bs_quant_weight(const float* w, int64_t ldw, uint8_t* w8, float* sw, int N, int K,
                              void* stream) {
  if (!w || !w8 || !sw) return SMALLM_ERR_INVALID;
  if (N <= 0 || K <= 0 || (N & 127) || (K & 127) || ldw < K) return SMALLM_ERR_SHAPE;
  if (!aligned16(w) || ((ldw * 4) & 15) || !aligned16(w8)) return SMALLM_ERR_ALIGN;
  hipLaunchKernelGGL((quant_weight_kernel<false>), dim3(N / 128, K / 128), dim3(256), 0,
                     (hipStream_t)stream, w, ldw, w8, (void*)sw, K);
  return launch_status();
}

int smallm_fp8bs_quant_weight_e8m0(const float* w, int64_t ldw, uint8_t* w8, uint8_t* sw_e8m0,
                                   int N, int K, void* stream) {
  if (!w || !w8 || !sw_e8m0) return SMALLM_ERR_INVALID;
  if (N <= 0 || K <= 0 || (N & 127) || (K & 127) || ldw < K) return SMALLM_ERR_SHAPE;
  if (!aligned16(w) || ((ldw * 4) & 15) || !aligned16(w8)) return SMALLM_ERR_ALIGN;
  hipLaunchKernelGGL((quant_weight_kernel<true>), dim3(N / 128, K / 128), dim3(256), 0,
                     (hipStream_t)stream, w, ldw, w8, (void*)sw_e8m0, K);
  return launch_status();
}

int smallm_fp8bs_pack_weight(const uint8_t* w8, uint8_t* w_packed, int N, int K, void* stream) {
  if (!w8 || !w_packed) return SMALLM_ERR_INVALID;
  if (N <= 0 || K <= 0 || (N & 127) || (K & 127)) return SMALLM_ERR_SHAPE;
  if (!aligned16(w8) || !aligned16(w_packed)) return SMALLM_ERR_ALIGN;
  launch_pack<true>(w8, w_packed, N, K, (hipStream_t)stream);
  return launch_status();
}

int smallm_fp8bs_unpack_weight(const uint8_t* w_packed, uint8_t* w8, int N, int K, void* stream) {
  if (!w8 || !w_packed) return SMALLM_ERR_INVALID;
  if (N <= 0 || K <= 0 || (N & 127) || (K & 127)) return SMALLM_ERR_SHAPE;
  if (!aligned16(w8) || !aligned16(w_packed)) return SMALLM_ERR_ALIGN;
  launch_pack<false>(w_packed, w8, N, K, (hipStream_t)stream);
  return launch_status();
}

static int quant_common(const uint16_t* x, int64_t ldx, uint8_t* q, int64_t ldq, void* sx, int M,
                        int K, bool e8, void* stream) {
  if (!x || !q || !sx) return SMALLM_ERR_INVALID;
  if (M < 1 || M > SMALLM_FP8BS_MAX_M || K <= 0 || (K & 127) || ldx < K || ldq < K)
    return SMALLM_ERR_SHAPE;
  if (!aligned16(x) || ((ldx * 2) & 15) || !aligned16(q) || (ldq & 15)) return SMALLM_ERR_ALIGN;
  const int groups = M * (K / 128);
  dim3 grid((groups + 63) / 64);
  if (e8)
    hipLaunchKernelGGL((quant_act_kernel<true>), grid, dim3(256), 0, (hipStream_t)stream, x, ldx, q,
                       ldq, sx, M, K);
  else
    hipLaunchKernelGGL((quant_act_kernel<false>), grid, dim3(256), 0, (hipStream_t)stream, x, ldx, q,
                       ldq, sx, M, K);
  return launch_status();
}

int smallm_fp8bs_quant(const uint16_t* x, int64_t ldx, uint8_t* q, int64_t ldq, float* sx, int M,
                       int K, void* stream) {
  return quant_common(x, ldx, q, ldq, (void*)sx, M, K, false, stream);
}

int smallm_fp8bs_quant_e8m0(const uint16_t* x, int64_t ldx, uint8_t* q, int64_t ldq,
                            uint8_t* sx_e8m0, int M, int K, void* stream) {
  return quant_common(x, ldx, q, ldq, (void*)sx_e8m0, M, K, true, stream);
}

static int rmsnorm_quant_common(const uint16_t* x, int64_t ldx, const uint16_t* w, float eps,
                                uint16_t* y, int64_t ldy, uint8_t* q, int64_t ldq, void* sx, int M,
                                int H, bool e8, void* stream) {
  if (!x || !w || (q && !sx) || (!q && !y)) return SMALLM_ERR_INVALID;
  if (!(eps > 0.0f) || !(eps <= 3.40282347e38f)) return SMALLM_ERR_INVALID;
  if (M < 1 || M > SMALLM_FP8BS_RMS_MAX_M || H < 128 || (H & 127) || H > SMALLM_FP8BS_RMS_MAX_H ||
      ldx < H || (y && ldy < H) || (q && ldq < H))
    return SMALLM_ERR_SHAPE;
  if (!aligned16(x) || ((ldx * 2) & 15) || !aligned16(w) || (y && (!aligned16(y) || ((ldy * 2) & 15))) ||
      (q && (!aligned16(q) || (ldq & 15))))
    return SMALLM_ERR_ALIGN;
  const int nl = H / 32;
  const int nt = nl >= 256 ? 256 : (nl + 63) / 64 * 64;
  if (e8)
    hipLaunchKernelGGL((rmsnorm_quant_kernel<true>), dim3(M), dim3(nt), 0, (hipStream_t)stream, x,
                       ldx, w, eps, y, ldy, q, ldq, sx, H);
  else
    hipLaunchKernelGGL((rmsnorm_quant_kernel<false>), dim3(M), dim3(nt), 0, (hipStream_t)stream, x,
                       ldx, w, eps, y, ldy, q, ldq, sx, H);
  return launch_status();
}

int smallm_fp8bs_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* w, float eps,
                               uint16_t* y, int64_t ldy, uint8_t* q, int64_t ldq, float* sx, int M,
                               int H, void* stream) {
  return rmsnorm_quant_common(x, ldx, w, eps, y, ldy, q, ldq, (void*)sx, M, H, false, stream);
}

int smallm_fp8bs_rmsnorm_quant_e8m0(const uint16_t* x, int64_t ldx, const uint16_t* w, float eps,
                                    uint16_t* y, int64_t ldy, uint8_t* q, int64_t ldq,
                                    uint8_t* sx_e8m0, int M, int H, void* stream) {
  return rmsnorm_quant_common(x, ldx, w, eps, y, ldy, q, ldq, (void*)sx_e8m0, M, H, true, stream);
}

int smallm_fp8bs_gemm(const uint8_t* q, int64_t ldq, const float* sx, const uint8_t* w_packed,
                      uint32_t layout_id, const float* sw, uint16_t* y, int64_t ldy, int M, int N,
                      int K, void* stream) {
  int st = check_gemm_args(q, ldq, 1, sx, true, w_packed, layout_id, sw, y, ldy, M, N, K);
  if (st) return st;
  return launch_gemm<kPreqF32>(q, ldq, sx, w_packed, sw, y, ldy, M, N, K, nullptr, nullptr,
                               (hipStream_t)stream);
}

int smallm_fp8bs_gemm_e8m0(const uint8_t* q, int64_t ldq, const uint8_t* sx_e8m0,
                           const uint8_t* w_packed, uint32_t layout_id, const uint8_t* sw_e8m0,
                           uint16_t* y, int64_t ldy, int M, int N, int K, void* stream) {
  int st = check_gemm_args(q, ldq, 1, sx_e8m0, true, w_packed, layout_id, sw_e8m0, y, ldy, M, N, K);
  if (st) return st;
  return launch_gemm<kPreqE8>(q, ldq, sx_e8m0, w_packed, sw_e8m0, y, ldy, M, N, K, nullptr,
                              nullptr, (hipStream_t)stream);
}

int smallm_fp8bs_quant_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                            uint32_t layout_id, const float* sw, uint16_t* y, int64_t ldy, int M,
                            int N, int K, uint8_t* q_dbg, float* sx_dbg, void* stream) {
  int st = check_gemm_args(x, ldx, 2, nullptr, false, w_packed, layout_id, sw, y, ldy, M, N, K);
  if (st) return st;
  if (q_dbg && !aligned16(q_dbg)) return SMALLM_ERR_ALIGN;
  return launch_gemm<kFusedF32>(x, ldx, nullptr, w_packed, sw, y, ldy, M, N, K, q_dbg,
                                (void*)sx_dbg, (hipStream_t)stream);
}

int smallm_fp8bs_quant_gemm_e8m0(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                 uint32_t layout_id, const uint8_t* sw_e8m0, uint16_t* y,
                                 int64_t ldy, int M, int N, int K, uint8_t* q_dbg,
                                 uint8_t* sx_dbg_e8m0, void* stream) {
  int st = check_gemm_args(x, ldx, 2, nullptr, false, w_packed, layout_id, sw_e8m0, y, ldy, M, N, K);
  if (st) return st;
  if (q_dbg && !aligned16(q_dbg)) return SMALLM_ERR_ALIGN;
  return launch_gemm<kFusedE8>(x, ldx, nullptr, w_packed, sw_e8m0, y, ldy, M, N, K, q_dbg,
                               (void*)sx_dbg_e8m0, (hipStream_t)stream);
}

// Rows up to which the fused kernel beats the standalone quantisation plus the tiled GEMM:
// measured on the pages' shapes (5120x4096, 4608x4096, 4096x2048, 2048x4096), graph replay over 24
// cold weight copies -- at 33 rows the quant + tiled pair is faster than the fused kernel's two
// 32-row chunks on all four (8.6 against 10.0 us on 4096x2048, 14.2 against 18.7 on 5120x4096).
constexpr int kFusedUpToM = 32;

size_t smallm_fp8bs_quant_gemm_workspace_bytes(int M, int N, int K) {
  if (check_mnk(M, N, K) != SMALLM_OK || M <= kFusedUpToM || !tiled_ok(M, K, K, layout_for(N, K))) return 0;
  const size_t qb = ((size_t)M * K + 255) / 256 * 256;
  return qb + (size_t)M * (K / 128) * 4;
}

// Beyond the small-M range with a workspace: the standalone quantisation into the workspace (q
// at pitch K, then the scales 256-byte aligned), then the tiled GEMM on it.  Otherwise the fused
// kernel (in 32-row chunks above 32 rows).
static int quant_gemm_ws(const uint16_t* x, int64_t ldx, const uint8_t* w_packed, uint32_t layout_id,
                         const void* sw, uint16_t* y, int64_t ldy, int M, int N, int K, void* workspace,
                         size_t workspace_bytes, bool e8, void* stream) {
  int st = check_gemm_args(x, ldx, 2, nullptr, false, w_packed, layout_id, sw, y, ldy, M, N, K);
  if (st) return st;
  const size_t need = smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K);
  if (need == 0) {
    return e8 ? launch_gemm<kFusedE8>(x, ldx, nullptr, w_packed, sw, y, ldy, M, N, K, nullptr, nullptr,
                                      (hipStream_t)stream)
              : launch_gemm<kFusedF32>(x, ldx, nullptr, w_packed, sw, y, ldy, M, N, K, nullptr, nullptr,
                                       (hipStream_t)stream);
  }
  if (!workspace) return SMALLM_ERR_INVALID;
  if (workspace_bytes < need) return SMALLM_ERR_SHAPE;
  if (((uintptr_t)workspace & 255) != 0) return SMALLM_ERR_ALIGN;
  uint8_t* q = (uint8_t*)workspace;
  void* sx = q + ((size_t)M * K + 255) / 256 * 256;
  st = quant_common(x, ldx, q, K, sx, M, K, e8, stream);
  if (st) return st;
  const Layout L = layout_for(N, K);
  if (e8) launch_tiled<true>(L, M, K, q, K, sx, w_packed, sw, y, ldy, (hipStream_t)stream);
  else launch_tiled<false>(L, M, K, q, K, sx, w_packed, sw, y, ldy, (hipStream_t)stream);
  return launch_status();
}

int smallm_fp8bs_quant_gemm_ws(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                               uint32_t layout_id, const float* sw, uint16_t* y, int64_t ldy, int M,
                               int N, int K, void* workspace, size_t workspace_bytes, void* stream) {
  return quant_gemm_ws(x, ldx, w_packed, layout_id, sw, y, ldy, M, N, K, workspace, workspace_bytes,
                       false, stream);
}

int smallm_fp8bs_quant_gemm_e8m0_ws(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                    uint32_t layout_id, const uint8_t* sw_e8m0, uint16_t* y,
                                    int64_t ldy, int M, int N, int K, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return quant_gemm_ws(x, ldx, w_packed, layout_id, sw_e8m0, y, ldy, M, N, K, workspace,
                       workspace_bytes, true, stream);
}

}  // extern "C"
