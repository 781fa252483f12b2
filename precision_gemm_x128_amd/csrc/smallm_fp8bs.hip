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
//  * Packed weight layout: every 16-column x 128-K block of W8 is one contiguous 2 KiB
//    fragment stored in the lane order of the B operand of v_mfma_*_16x16x128_f8f6f4: lane
//    l = 16*c + j holds column j and K bytes [32c, 32c+32) of the block, bytes 0..15 in the first
//    KiB of the fragment and bytes 16..31 in the second.  A wave therefore fetches a fragment
//    with two 16-byte non-temporal loads per lane, each covering 1 KiB contiguously.  Fragments
//    of one 16-column tile are consecutive along K.
//  * Work split: one workgroup (8 waves) owns NT 16-column tiles and all of K.  Waves 0-3
//    quantise the activation rows for the workgroup (32 contiguous bf16 per lane, a quad of
//    lanes per 1x128 group, the group amax reduced with two DPP quad permutes) and stage the
//    e4m3 bytes in LDS; waves 4-7 issue their share of the weight stream up front, then run the
//    MFMAs with the A operand read from LDS.  Keeping the weight loads and the activation loads
//    in different waves keeps each wave's in-order load counter free of the other stream.
//  * Quantisation is bit-exact with the IEEE definition q = RN(x / RN(amax / 448)): the
//    quotient is formed from a correctly rounded reciprocal y = RN(1/sx) as q0 = x*y,
//    r = fma(q0, sx, -x), q = fma(-r, y, q0), which equals the IEEE quotient for every bf16 x
//    and every scale >= 2^-64 wherever the e4m3 code depends on it (verified exhaustively),
//    keeps the sign of zero, and falls back to a true division for smaller scales.  The fp8
//    encoding uses the hardware round-to-nearest-even conversion, which is exact below 464.
//  * Deterministic reduction: per-wave fp32 partials are summed through LDS in a fixed order.
//
// Build flags (see the package's build module): --offload-arch=gfx950 -O3 -ffp-contract=off,
// no fast-math, fp32 denormals kept, packed-fp32 instructions disabled.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/smallm_fp8bs.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;                // 8 waves: 4 quantise, 4 MFMA
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
__device__ __forceinline__ void quant32_codes(const u32x4 (&xv)[4], float yh, float yl, float k,
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
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
    w[j] = (uint32_t)p;
  }
}

// Quantise 32 consecutive bf16 of one 1x128 group (this lane's quarter; the group is spread
// over a DPP quad) with an fp32 group scale.  Returns the scale, writes 32 e4m3 bytes.
//
// x / s is formed with a two-term reciprocal, 1/s ~ yh + yl: yh is 1/s rounded toward zero (the
// correctly rounded reciprocal, stepped down one unit when the residual 1 - s yh comes out
// negative) and yl = (1 - s yh) yh >= 0 its remainder, so that q = fma(x, yh, x yl) costs a
// multiply and an FMA per element and keeps the sign of a zero x.  A group scale below 2^-64 is
// first rescaled by 2^64 (x 2^64 / (s 2^64) is the same quotient; both products are exact,
// |x| <= 448 s keeping x 2^64 below 448) so that 1/s stays finite.  Over every pair of bf16 amax
// and bf16 x with |x| <= amax, the e4m3 code of q equals that of the correctly rounded division
// RN(x / s): q differs from RN(x / s) only by quotients that no e4m3 rounding boundary separates.
__device__ __forceinline__ float quant32_fp32(const u32x4 (&xv)[4], u32x4 (&qv)[2]) {
  // group amax on the bf16 bit patterns: with the sign cleared, integer order is magnitude order
  u16x2 mx = u16x2{0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, xv[i >> 2][i & 3] & 0x7FFF7FFFu));
  const uint32_t amb = quad_max_u32(max((uint32_t)mx[0], (uint32_t)mx[1]));
  const float am = __uint_as_float(amb << 16);
  const float s = am / 448.0f;                          // correctly rounded fp32 division
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
  if (__builtin_amdgcn_ballot_w64(tiny) != 0) quant32_codes<true>(xv, yh, yl, k, w);
  else quant32_codes<false>(xv, yh, yl, k, w);
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
// Packed layout with C weight columns per group (C in {16, 8, 4, 2}, S = 16 / C K-blocks per
// fragment): fragment f = cg * KG + h (KG = K / (128 S)) holds columns [cg C, cg C + C) and K-blocks
// [h S, h S + S).  Its 16 MFMA B columns are j = c S + s (column c of the group, K-block s of the
// fragment).  Lane l = 16 chunk + j of the fragment holds K bytes [32 chunk, 32 chunk + 32) of that
// column and K-block: bytes 0..15 at l * 16, bytes 16..31 at 1024 + l * 16.

template <bool PACK, int C>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   int K, int64_t chunks) {
  constexpr int S = 16 / C;
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= chunks) return;
  const int KG = (K >> 7) / S;
  const int64_t f = o >> 7;
  const int within = (int)(o & 127), half = within >> 6, lane = within & 63;
  const int chunk = lane >> 4, j = lane & 15;
  const int64_t cg = f / KG, h = f % KG;
  const int64_t n = cg * C + j / S;
  const int64_t k = (h * S + j % S) * 128 + chunk * 32 + half * 16;
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
    const float s = quant32_fp32(xv, qv);
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
        const float sc = quant32_fp32(yv, qv);
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

constexpr int kKCMax = 32;      // K blocks staged per round
constexpr int kMaxMfmaWaves = 12;  // MFMA waves per workgroup (the quantising waves come first)

template <int MT, int C, int NCG, int NKG, int MODE>
struct GemmCfg {
  static constexpr bool kE8 = (MODE & 1) != 0;
  static constexpr bool kPreq = (MODE & 2) != 0;
  static constexpr int kS = 16 / C;                 // K blocks per weight fragment
  static constexpr int kMP = 16 * MT;               // rows per workgroup (M padded to the MFMA)
  static constexpr int kStq = kKCMax * kMP * kRowStride;
  static constexpr int kSts = kKCMax * kMP * (kE8 ? 1 : 4);
  // partial-sum block of one (MFMA wave, column group, M tile): 4 x 64 floats, padded so that
  // consecutive column groups start 16 floats apart modulo the 64 LDS banks
  static constexpr int kRedPitch = 4 * 64 + 16 / MT;
  static constexpr int kRed = kMaxMfmaWaves * NCG * MT * kRedPitch * 4;
  // One M tile with shared activation tiles (NCG > 1): the partial sums get their own LDS space
  // after the staging area, so the last round needs no barrier between the MFMAs and the
  // partial-sum writes.  Otherwise they reuse the staging space.
  static constexpr bool kRedOwn = (MT == 1 && NCG > 1);
  static constexpr int kRedOff = kRedOwn ? (kStq + kSts + 15) / 16 * 16 : 0;
  static constexpr int kSmem = kRedOwn ? kRedOff + kRed : ((kStq + kSts) > kRed ? (kStq + kSts) : kRed);
};

// One workgroup owns CGW consecutive column groups (C columns each) and all of K; with 256
// workgroups every CU streams the same number of weight bytes.  The first QW waves quantise (or
// stage) the activations of a round of K blocks into LDS, two passes of loads in flight per wave.
// The NWK * NWC MFMA waves follow.  MFMA wave (kq, cq) = (w % NWK, w / NWK) owns the column
// groups cq, cq + NWC, ... (NCG at most) and, in every round, part kq of NWK contiguous parts of
// that round's K groups (NKG at most): it reads each staged activation tile of its K groups once and
// multiplies it into the weight fragments of all its column groups, so the activation bytes cross
// the LDS once per NCG column groups.  Every weight load is unconditional (a buffer load whose
// offset points past the workgroup's region when the slot is unused, so the hardware returns zeros
// without touching memory); the code between the loads and the MFMAs is straight-line, which lets
// each MFMA wait only for its own fragment.
//
// A fragment's S K blocks are S MFMAs chained into one accumulator.  MFMA s must only count in
// the lanes whose B column belongs to K block s; the other lanes get the B-scale byte 0 (2^-127)
// for it, so their share is scaled down by 2^-127 (below 2^-127 * 448^2 * 128 of that block's raw
// dot product) instead of costing a masking operation per MFMA.  In the fp32-scale modes each
// lane then multiplies the fragment's partial by x_scale * w_scale of its own K block (the pages'
// 128x128 weight_scale_inv); in the e8m0 modes the scales are the MFMA's own e8m0 scale operands
// and the accumulator runs over all of K.
template <int MT, int C, int NCG, int NKG, int MODE>
__global__ __launch_bounds__(1024) void smallm_gemm_kernel(
    const void* __restrict__ a_src, int64_t lda, const void* __restrict__ sa_src,
    const uint8_t* __restrict__ wp, const void* __restrict__ sw, uint16_t* __restrict__ y,
    int64_t ldy, int M, int K, int CGW, int NWK, int NWC, int QW, uint8_t* __restrict__ q_dbg,
    void* __restrict__ sx_dbg) {
  using Cfg = GemmCfg<MT, C, NCG, NKG, MODE>;
  constexpr int S = Cfg::kS, MP = Cfg::kMP;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::kSmem];
  uint8_t* stq = smem;
  float* sts_f = (float*)(smem + Cfg::kStq);
  uint8_t* sts_b = smem + Cfg::kStq;
  float* red = (float*)(smem + Cfg::kRedOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K >> 7;
  const int KG = KB / S;
  const int KC = NKG * NWK * S;     // K blocks per round
  const int cg0 = blockIdx.x * CGW;
  const int m0 = blockIdx.y * MP;
  const int Mc = min(M - m0, MP);
  const int s_l = (lane & 15) % S;  // K block (within a fragment) of this lane's B column

  const int mw = wave - QW;
  const int kq = (mw >= 0) ? mw % NWK : 0;
  const int cq = (mw >= 0) ? mw / NWK : 0;
  const uint32_t region = (uint32_t)CGW * (uint32_t)KG * 2048u;
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wp + (int64_t)cg0 * KG * 2048), 0, (int)region, 0x00020000);

  v4f acc[NCG][MT];
#pragma unroll
  for (int j = 0; j < NCG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // e8m0 with one column group: odd fragments accumulate separately, so that the MFMA chain of
  // consecutive fragments is two independent chains (added once at the end)
  v4f acc_odd[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_odd[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // Each role runs its own round loop (same number of barriers per round on both sides), so
  // that values one role keeps across rounds take no registers in the other.
  const int rounds = (KB + KC - 1) / KC;
  if (mw >= 0) {
    for (int rd = 0; rd < rounds; ++rd) {
      const int kb0 = rd * KC;
      const int KCr = min(KC, KB - kb0);
      // ---- MFMA waves ----
      // The lane index, formed afresh in every round where the compiler cannot see through it, so
      // that the lane-dependent addresses are computed inside the round instead of held in
      // registers across the whole loop (which would spill: a spill reload waits for every load
      // in flight).
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int s_lr = (ln & 15) % S;  // K block (within a fragment) of this lane's B column
      const int KGr = KCr / S;
      // this wave's K groups of the round: a contiguous share [kg_lo, kg_lo + nkg)
      const int kg_lo = kq * KGr / NWK;
      const int nkg = (kq + 1) * KGr / NWK - kg_lo;
      float swv[NKG][NCG];
      int sbl[NKG][NCG];
      u32x4 wr[NKG][NCG][2];
      // Block scales: a fragment's S scales are contiguous and the same for the whole wave, so
      // they are read with scalar loads (own counter: waiting for them never waits for the weight
      // stream, and they take no vector registers); each lane then picks its own K block's.
#pragma unroll
      for (int i = 0; i < NKG; ++i)
#pragma unroll
        for (int j = 0; j < NCG; ++j) {
          const int cg = min(cq + j * NWC, CGW - 1);
          const int nb = ((cg0 + cg) * C) >> 7;  // 128-column block of the column group
          const int kbs = __builtin_amdgcn_readfirstlane(min(kb0 + (kg_lo + i) * S, KB - S));
          const int base = __builtin_amdgcn_readfirstlane(nb * KB + kbs);
          if (Cfg::kE8) {
            const uint8_t* sp = (const uint8_t*)sw + base;
            uint32_t word = 0;
#pragma unroll
            for (int t = 0; t < (S < 4 ? S : 4); ++t) word |= (uint32_t)sp[t] << (8 * t);
            if (S == 8) {
              uint32_t hi = 0;
#pragma unroll
              for (int t = 4; t < 8; ++t) hi |= (uint32_t)sp[t] << (8 * (t - 4));
              word = (s_lr < 4) ? word : hi;
            }
            sbl[i][j] = (int)((word >> (8 * (s_lr & 3))) & 0xFFu);
          } else {
            const float* sp = (const float*)sw + base;
            float sc[S];
#pragma unroll
            for (int t = 0; t < S; ++t) sc[t] = sp[t];
            float v = sc[0];
#pragma unroll
            for (int t = 1; t < S; ++t) v = (s_lr == t) ? sc[t] : v;
            swv[i][j] = v;
          }
        }
#pragma unroll
      for (int i = 0; i < NKG; ++i)
#pragma unroll
        for (int j = 0; j < NCG; ++j) {
          const int cg = cq + j * NWC;
          const uint32_t off = (i < nkg && cg < CGW)
                                   ? ((uint32_t)(cg * KG + kb0 / S + kg_lo + i) * 2048u + ln * 16u)
                                   : region;
          wr[i][j][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 2));
          wr[i][j][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off + 1024u, 0, 2));
        }
      __syncthreads();  // activation bytes and scales of this round are staged
#pragma unroll
      for (int i = 0; i < NKG; ++i) {
        // K group within the round; a slot past the wave's share has zero weights and reads a
        // staged tile (finite bytes), so its products are exactly zero
        const int kgr = min(kg_lo + i, KGr - 1);
        // with eight fragments, shared tiles or two M tiles of multi-block fragments, keep the
        // scheduler from hoisting the next K group's LDS reads over this one (their registers
        // would not fit, and a spill reload waits for every load in flight)
        if (NKG >= 8 || NCG > 1 || (MT == 2 && S >= 2)) __builtin_amdgcn_sched_barrier(0);
        if constexpr (NCG == 1) {
          // one column group: each activation tile is read right before its MFMA
          const v8i b = __builtin_bit_cast(
              v8i, __builtin_shufflevector(wr[i][0][0], wr[i][0][1], 0, 1, 2, 3, 4, 5, 6, 7));
          v4f fa[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) fa[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < S; ++s) {
            const int kbr = kgr * S + s;  // K block within the round
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int row = mt * 16 + (ln & 15);
              const u32x4* ap = (const u32x4*)(stq + (kbr * MP + row) * kRowStride + (ln >> 4) * 32);
              const u32x4 a0 = ap[0], a1 = ap[1];
              const v8i a = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
              if (Cfg::kE8) {
                const int sa = (int)sts_b[kbr * MP + row];
                const int sb = (S == 1 || s_lr == s) ? sbl[i][0] : 0;
                v4f& dst = (i & 1) ? acc_odd[mt] : acc[0][mt];
                dst = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, dst, 0, 0, 0, sa, 0, sb);
              } else if (S == 1) {
                fa[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, fa[mt], 0, 0, 0, 0, 0, 0);
              } else {
                const int sb = (s_lr == s) ? 127 : 0;
                fa[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, fa[mt], 0, 0, 0, 127, 0, sb);
              }
            }
          }
          if (!Cfg::kE8) {
            const int kbl = kgr * S + s_lr;  // this ln's K block within the round
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const v4f sx4 = *(const v4f*)(sts_f + kbl * MP + mt * 16 + 4 * (ln >> 4));
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[0][mt][e] = __builtin_fmaf(sx4[e] * swv[i][0], fa[mt][e], acc[0][mt][e]);
            }
          }
        } else {
          if constexpr (MT == 1) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              // the K group's S activation tiles, read from LDS once for all NCG column groups
              const int row = mt * 16 + (ln & 15);
              v8i a[S];
              int sa[S];
#pragma unroll
              for (int s = 0; s < S; ++s) {
                const int kbr = kgr * S + s;  // K block within the round
                const u32x4* ap = (const u32x4*)(stq + (kbr * MP + row) * kRowStride + (ln >> 4) * 32);
                const u32x4 a0 = ap[0], a1 = ap[1];
                a[s] = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                sa[s] = Cfg::kE8 ? (int)sts_b[kbr * MP + row] : 127;
              }
              v4f sx4 = v4f{0.0f, 0.0f, 0.0f, 0.0f};
              if (!Cfg::kE8) {
                const int kbl = kgr * S + s_lr;  // this ln's K block within the round
                sx4 = *(const v4f*)(sts_f + kbl * MP + mt * 16 + 4 * (ln >> 4));
              }
              // fragments in groups of up to three, whose MFMA chains interleave (a dependent chain
              // would wait for each MFMA's result), each group consumed as soon as its loads land
              constexpr int JG = NCG < 3 ? NCG : 3;
#pragma unroll
              for (int j0 = 0; j0 < NCG; j0 += JG) {
                v8i b[JG];
                v4f fa[JG];
#pragma unroll
                for (int jj = 0; jj < JG; ++jj) {
                  const int j = min(j0 + jj, NCG - 1);
                  b[jj] = __builtin_bit_cast(
                      v8i, __builtin_shufflevector(wr[i][j][0], wr[i][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
                  fa[jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                }
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                  for (int jj = 0; jj < JG; ++jj) {
                    const int j = j0 + jj;
                    if (j >= NCG) continue;
                    if (Cfg::kE8) {
                      const int sb = (S == 1 || s_lr == s) ? sbl[i][j] : 0;
                      acc[j][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[s], b[jj], acc[j][mt], 0, 0, 0, sa[s], 0, sb);
                    } else if (S == 1) {
                      fa[jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[s], b[jj], fa[jj], 0, 0, 0, 0, 0, 0);
                    } else {
                      const int sb = (s_lr == s) ? 127 : 0;
                      fa[jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[s], b[jj], fa[jj], 0, 0, 0, 127, 0, sb);
                    }
                  }
                if (!Cfg::kE8) {
#pragma unroll
                  for (int jj = 0; jj < JG; ++jj) {
                    const int j = j0 + jj;
                    if (j >= NCG) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                      acc[j][mt][e] = __builtin_fmaf(sx4[e] * swv[i][j], fa[jj][e], acc[j][mt][e]);
                  }
                }
              }
            }
          } else {
            // two M tiles: one activation tile at a time (the accumulators of both tiles are
            // live), the NCG independent MFMA chains interleaved
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int row = mt * 16 + (ln & 15);
              v4f fa[NCG];
#pragma unroll
              for (int j = 0; j < NCG; ++j) fa[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int s = 0; s < S; ++s) {
                const int kbr = kgr * S + s;  // K block within the round
                const u32x4* ap = (const u32x4*)(stq + (kbr * MP + row) * kRowStride + (ln >> 4) * 32);
                const u32x4 a0 = ap[0], a1 = ap[1];
                const v8i a = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                  (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                const int sa = Cfg::kE8 ? (int)sts_b[kbr * MP + row] : 127;
#pragma unroll
                for (int j = 0; j < NCG; ++j) {
                  const v8i b = __builtin_bit_cast(
                      v8i, __builtin_shufflevector(wr[i][j][0], wr[i][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
                  if (Cfg::kE8) {
                    const int sb = (S == 1 || s_lr == s) ? sbl[i][j] : 0;
                    acc[j][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j][mt], 0, 0, 0, sa, 0, sb);
                  } else if (S == 1) {
                    fa[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, fa[j], 0, 0, 0, 0, 0, 0);
                  } else {
                    const int sb = (s_lr == s) ? 127 : 0;
                    fa[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, fa[j], 0, 0, 0, 127, 0, sb);
                  }
                }
                __builtin_amdgcn_sched_barrier(0);
              }
              if (!Cfg::kE8) {
                const int kbl = kgr * S + s_lr;  // this lane's K block within the round
                const v4f sx4 = *(const v4f*)(sts_f + kbl * MP + mt * 16 + 4 * (ln >> 4));
#pragma unroll
                for (int j = 0; j < NCG; ++j)
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    acc[j][mt][e] = __builtin_fmaf(sx4[e] * swv[i][j], fa[j][e], acc[j][mt][e]);
              }
            }
          }
        }
      }
      if (!Cfg::kRedOwn || rd + 1 < rounds) __syncthreads();  // staging buffer free for the next round
    }
    if (Cfg::kE8 && NCG == 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[0][mt] += acc_odd[mt];
    }
  } else {
    // the quantisers' loads and VALU work issue ahead of the MFMA waves' on their SIMD: the MFMA
    // waves only wait for their weights, while the staged activations gate every MFMA
    __builtin_amdgcn_s_setprio(3);
    for (int rd = 0; rd < rounds; ++rd) {
      const int kb0 = rd * KC;
      const int KCr = min(KC, KB - kb0);
      // ---- quantising (or staging) waves: one DPP quad per 1x128 group, two passes in flight ----
      const int grp = lane >> 2;  // this lane's group within a block of 16
      const int c = lane & 3;
      const int G = Mc * KCr;
      constexpr int NV = Cfg::kPreq ? 2 : 4;                    // 16-byte loads per lane per pass
      const int rowb = Cfg::kPreq ? 1 : 2;                        // bytes per activation element
      // the workgroup's activation rows as a bounds-checked buffer: idle lanes and passes past the
      // work use an offset past its end and fetch nothing
      const uint32_t abytes = (uint32_t)((int64_t)(Mc - 1) * lda * rowb + (int64_t)KB * 128 * rowb);
      const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const uint8_t*)a_src + (int64_t)m0 * lda * rowb), 0, (int)abytes, 0x00020000);
      u32x4 xa[4], xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { xa[i] = u32x4{0, 0, 0, 0}; xb[i] = u32x4{0, 0, 0, 0}; }
#define SMALLM_QLOAD(v, b) do {                                                                   \
      const int g_ = (b) * 16 + grp;                                                             \
      const uint32_t off_ = (g_ < G) ? (uint32_t)(((int64_t)(g_ % Mc) * lda + (kb0 + g_ / Mc) * 128 + c * 32) * rowb) \
                                     : abytes;                                                   \
      _Pragma("unroll") for (int i_ = 0; i_ < NV; ++i_)                                          \
        v[i_] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, off_ + 16u * i_, 0, 0)); \
    } while (0)
#define SMALLM_QPROC(v, b) do {                                                                   \
      const int g_ = (b) * 16 + grp;                                                             \
      const bool valid_ = g_ < G;                                                                \
      const int kbl_ = valid_ ? g_ / Mc : 0;                                                     \
      const int m_ = valid_ ? g_ % Mc : 0;                                                       \
      u32x4 qv_[2];                                                                              \
      float s_ = 0.0f;                                                                           \
      uint32_t e_ = 0;                                                                           \
      if (!Cfg::kPreq) {                                                                         \
        if (Cfg::kE8) e_ = quant32_e8m0(v, qv_);                                                 \
        else s_ = quant32_fp32(v, qv_);                                                          \
      } else {                                                                                   \
        qv_[0] = v[0];                                                                           \
        qv_[1] = v[1];                                                                           \
      }                                                                                          \
      if (valid_) {                                                                              \
        u32x4* dp_ = (u32x4*)(stq + (kbl_ * MP + m_) * kRowStride + c * 32);                    \
        dp_[0] = qv_[0];                                                                         \
        dp_[1] = qv_[1];                                                                         \
        if (c == 0) {                                                                            \
          if (Cfg::kPreq) {                                                                      \
            if (Cfg::kE8) sts_b[kbl_ * MP + m_] = ((const uint8_t*)sa_src)[(int64_t)(m0 + m_) * KB + kb0 + kbl_]; \
            else sts_f[kbl_ * MP + m_] = ((const float*)sa_src)[(int64_t)(m0 + m_) * KB + kb0 + kbl_];           \
          } else {                                                                               \
            if (Cfg::kE8) sts_b[kbl_ * MP + m_] = (uint8_t)e_;                                   \
            else sts_f[kbl_ * MP + m_] = s_;                                                     \
          }                                                                                      \
        }                                                                                        \
      }                                                                                          \
    } while (0)
      // Block b of 16 groups: groups 16 b .. 16 b + 15, one per DPP quad of a wave.  Wave w takes
      // blocks w, QW + w, 2 QW + w, ... alternating between its two buffers; the buffer processed
      // next holds the smaller block index, so once it is past the end the other one is too.
      const int nblk = (G + 15) >> 4;
      int b0 = wave, b1 = QW + wave;
      SMALLM_QLOAD(xa, b0);
      SMALLM_QLOAD(xb, b1);
      while (b0 < nblk) {
        SMALLM_QPROC(xa, b0);
        b0 += 2 * QW;
        SMALLM_QLOAD(xa, b0);
        if (b1 >= nblk) break;
        SMALLM_QPROC(xb, b1);
        b1 += 2 * QW;
        SMALLM_QLOAD(xb, b1);
      }
#undef SMALLM_QLOAD
#undef SMALLM_QPROC
      __syncthreads();  // staged: the MFMA waves read it now
      if (!Cfg::kPreq && blockIdx.x == 0) {
        // debug copy of the quantised bytes and scales this round used
        const int qt = tid;  // 0 .. 64*QW-1
        if (q_dbg != nullptr) {
          for (int g = qt; g < Mc * KCr * 8; g += QW * 64) {
            const int row = g / (KCr * 8), rem = g % (KCr * 8), kbl = rem / 8, part16 = rem % 8;
            *(u32x4*)(q_dbg + (int64_t)(m0 + row) * K + (kb0 + kbl) * 128 + part16 * 16) =
                *(const u32x4*)(stq + (kbl * MP + row) * kRowStride + part16 * 16);
          }
        }
        if (sx_dbg != nullptr) {
          for (int g = qt; g < Mc * KCr; g += QW * 64) {
            const int row = g / KCr, kbl = g % KCr;
            if (Cfg::kE8) ((uint8_t*)sx_dbg)[(int64_t)(m0 + row) * KB + kb0 + kbl] = sts_b[kbl * MP + row];
            else ((float*)sx_dbg)[(int64_t)(m0 + row) * KB + kb0 + kbl] = sts_f[kbl * MP + row];
          }
        }
      }
      if (!Cfg::kRedOwn || rd + 1 < rounds) __syncthreads();
    }
  }

  // ---- cross-wave and cross-lane reduction through LDS, fixed order ----
  // (lane and thread index formed again here rather than held across the rounds)
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int tid_e = wave * 64 + lane_e;
  constexpr int RP = Cfg::kRedPitch;
  if (mw >= 0) {
#pragma unroll
    for (int j = 0; j < NCG; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((mw * NCG + j) * MT + mt) * RP + e * 64 + lane_e] = acc[j][mt][e];
  }
  // One output per thread and pass, consecutive threads on consecutive columns of a row.  A
  // column's S K-block partials sit in S consecutive lanes, read as one vector per MFMA wave.
  // The first output's indices are formed before the barrier, off the critical path.
  const unsigned ncols = (unsigned)(CGW * C);
  const unsigned nthreads = blockDim.x;  // > ncols
  unsigned row = (unsigned)tid_e / ncols;
  unsigned col = (unsigned)tid_e - row * ncols;
  const unsigned drow = nthreads / ncols, dcol = nthreads - drow * ncols;
  const int kstride = NCG * MT * RP;
  __syncthreads();
  while (row < (unsigned)Mc) {
    const unsigned cgw = col / C, cc = col % C;
    const unsigned j = cgw / (unsigned)NWC, cqo = cgw - j * (unsigned)NWC;
    const unsigned mt = row >> 4, r = row & 15, e = r & 3;
    const unsigned lbase = (r >> 2) * 16 + cc * S;  // lanes of the column's S K blocks
    const float* rp = red + ((cqo * NWK * NCG + j) * MT + mt) * RP + e * 64 + lbase;
    float sum = 0.0f;
#pragma unroll 4
    for (int k = 0; k < NWK; ++k, rp += kstride) {
      if constexpr (S >= 4) {
#pragma unroll
        for (int s4 = 0; s4 < S; s4 += 4) {
          const v4f v = *(const v4f*)(rp + s4);
          sum += v[0]; sum += v[1]; sum += v[2]; sum += v[3];
        }
      } else if constexpr (S == 2) {
        const v2f v = *(const v2f*)rp;
        sum += v[0]; sum += v[1];
      } else {
        sum += rp[0];
      }
    }
    y[(int64_t)(m0 + row) * ldy + (int64_t)(cg0 + cgw) * C + cc] = bf16_rne(sum);
    row += drow;
    col += dcol;
    if (col >= ncols) { col -= ncols; ++row; }
  }
}

// ---------------------------------------------------------------------------------------------
// GEMM on pre-quantised input beyond the small-M range: MFMA-tiled, for 16-column layouts
// ---------------------------------------------------------------------------------------------

constexpr int kTiledFromM = 32;  // M above which the pre-quantised GEMM is tiled
constexpr int kTM = 32;          // rows per workgroup tile of the tiled kernel
constexpr int kTiledMaxKB = 128;  // K blocks the tiled kernel takes (e8m0 weight scales in two registers)
constexpr int kTD = 8;        // weight fragments in flight per wave (K blocks ahead)
constexpr int kTPitch = 144;  // LDS pitch of a staged 128-byte activation row (conflict-free reads)

// Workgroup tile: TM rows x 64 columns, four waves, wave w owning column group 4 x + w (16
// columns) for all TM rows.  Per K block the tile's TM x 128 activation bytes and their scales
// are staged in LDS by the 256 threads (TM / 2 bytes each; two buffers, one barrier per K block);
// each wave streams its own fragments kTD K blocks ahead and runs one
// 16x16x128 MFMA per 16-row subtile (the activation bytes are fetched kTD K blocks ahead too).
// fp32 scales: each K block's partial is multiplied by
// sx[row, kb] * sw[n/128, kb] into the accumulator; e8m0: the scales are the MFMA's scale
// operands and one accumulator runs over K.  Every wave owns whole outputs: no reduction.
template <int TM, bool E8>
__global__ __launch_bounds__(256) void tiled_gemm_kernel(
    const uint8_t* __restrict__ q, int64_t ldq, const void* __restrict__ sa,
    const uint8_t* __restrict__ wp, const void* __restrict__ sw, uint16_t* __restrict__ y,
    int64_t ldy, int M, int K) {
  constexpr int NSUB = TM / 16;   // 16-row MFMA subtiles
  constexpr int TPR = 256 / TM;   // staging threads per row
  constexpr int BPT = 128 / TPR;  // staged bytes per thread
  constexpr int NLA = BPT / 16;   // 16-byte loads per thread
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][TM * kTPitch];
  __shared__ uint32_t sS[2][TM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K >> 7;
  const int cg = blockIdx.x * 4 + wave;
  const int m0 = blockIdx.y * TM;
  const int Mt = min(TM, M - m0);
  const int nb = (cg * 16) >> 7;

  // the tile's activation rows as a bounds-checked buffer; rows past M and K blocks past the end
  // use an offset beyond it and read zeros without touching memory
  const uint32_t abytes = (uint32_t)((int64_t)(Mt - 1) * ldq + K);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(q + (int64_t)m0 * ldq), 0, (int)abytes, 0x00020000);
  const uint32_t wbytes = (uint32_t)KB * 2048u;
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wp + (int64_t)cg * KB * 2048), 0, (int)wbytes, 0x00020000);
  const int srow = tid / TPR, sch = tid % TPR;  // staging: row and chunk of this thread
  // per-thread bases: a row past the tile starts beyond the buffers, so every K block of it
  // reads zeros; the weight offsets of K blocks past the end are beyond their buffer too
  const uint32_t arow = (srow < Mt) ? (uint32_t)((int64_t)srow * ldq + sch * BPT) : abytes;
  const uint32_t sbytes = (uint32_t)(Mt * KB) * (E8 ? 1u : 4u);
  const uint32_t srowb = (srow < Mt) ? (uint32_t)(srow * KB) * (E8 ? 1u : 4u) : sbytes;
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)sa + (int64_t)m0 * KB * (E8 ? 1 : 4)), 0, (int)sbytes, 0x00020000);

  u32x4 ab[kTD][NLA];
  uint32_t asc[kTD];
  u32x4 wb[kTD][2];
#define TILED_LOAD_A(slot, kb) do {                                                               \
    const uint32_t o_ = arow + (uint32_t)(kb) * 128u;                                              \
    _Pragma("unroll") for (int l_ = 0; l_ < NLA; ++l_)                                             \
      ab[slot][l_] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, o_ + 16u * l_, 0, 0)); \
    const uint32_t so_ = srowb + (uint32_t)(kb) * (E8 ? 1u : 4u);                                 \
    if (E8) asc[slot] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(srsrc, so_, 0, 0);             \
    else asc[slot] = __builtin_amdgcn_raw_buffer_load_b32(srsrc, so_, 0, 0);                          \
  } while (0)
#define TILED_LOAD_W(slot, kb) do {                                                               \
    const uint32_t o_ = (uint32_t)(kb) * 2048u + (uint32_t)lane * 16u;                              \
    wb[slot][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, o_, 0, 2)); \
    wb[slot][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, o_ + 1024u, 0, 2)); \
  } while (0)

  // e8m0 weight scales of the column group's row of blocks, one byte per lane (K blocks 0..63 and
  // 64..127; past the row: zeros), loaded before everything else and taken per K block with
  // readlane, so no load sits on the MFMA's path
  uint32_t swb0 = 0u, swb1 = 0u;
  if (E8) {
    const __amdgpu_buffer_rsrc_t swsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)sw + (int64_t)nb * KB), 0, KB, 0x00020000);
    swb0 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(swsrc, (uint32_t)lane, 0, 0);
    swb1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(swsrc, (uint32_t)lane + 64u, 0, 0);
  }
  // prologue in the loop's own issue order (per K block: activation bytes, scale, weights), so
  // that every wait in the loop counts the same loads behind it
#pragma unroll
  for (int d = 0; d < kTD; ++d) {
    TILED_LOAD_A(d, d);
    TILED_LOAD_W(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  v4f acc[NSUB];
#pragma unroll
  for (int i = 0; i < NSUB; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb0 = 0; kb0 < KB; kb0 += kTD) {
#pragma unroll
    for (int u = 0; u < kTD; ++u) {
      const int kb = kb0 + u;
      if (kb >= KB) break;  // uniform
      const int buf = u & 1;  // kb0 is a multiple of kTD (even): buffer and slots follow u
      // stage K block kb (its rows' last readers, at kb - 2, are past the previous barrier)
      u32x4* dst = (u32x4*)(&sA[buf][srow * kTPitch + sch * BPT]);
#pragma unroll
      for (int l = 0; l < NLA; ++l) dst[l] = ab[u][l];
      sS[buf][srow] = asc[u];  // the threads of a row store the same value
      __syncthreads();
      TILED_LOAD_A(u, kb + kTD);
      const v8i b = __builtin_bit_cast(v8i, __builtin_shufflevector(wb[u][0], wb[u][1], 0, 1, 2, 3, 4, 5, 6, 7));
      if (E8) {
        const int sb = (kb < 64) ? __builtin_amdgcn_readlane((int)swb0, kb) : __builtin_amdgcn_readlane((int)swb1, kb - 64);
#pragma unroll
        for (int i = 0; i < NSUB; ++i) {
          const int r = i * 16 + (lane & 15);
          const u32x4* ap = (const u32x4*)(&sA[buf][r * kTPitch + (lane >> 4) * 32]);
          const u32x4 a0 = ap[0], a1 = ap[1];
          const v8i a = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i], 0, 0, 0, (int)sS[buf][r], 0, sb);
        }
      } else {
        const float swv = ((const float*)sw)[nb * KB + kb];
        v4f fa[NSUB];
#pragma unroll
        for (int i = 0; i < NSUB; ++i) {
          const int r = i * 16 + (lane & 15);
          const u32x4* ap = (const u32x4*)(&sA[buf][r * kTPitch + (lane >> 4) * 32]);
          const u32x4 a0 = ap[0], a1 = ap[1];
          const v8i a = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          fa[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NSUB; ++i) {
          const v4f sx4 = v4f{__uint_as_float(sS[buf][i * 16 + 4 * (lane >> 4) + 0]),
                              __uint_as_float(sS[buf][i * 16 + 4 * (lane >> 4) + 1]),
                              __uint_as_float(sS[buf][i * 16 + 4 * (lane >> 4) + 2]),
                              __uint_as_float(sS[buf][i * 16 + 4 * (lane >> 4) + 3])};
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] = __builtin_fmaf(sx4[e] * swv, fa[i][e], acc[i][e]);
        }
      }
      TILED_LOAD_W(u, kb + kTD);
    }
  }
#undef TILED_LOAD_A
#undef TILED_LOAD_W
  // output: lane l holds column l % 16 of the wave's group, rows 4 (l / 16) + e of each subtile
  const int col = cg * 16 + (lane & 15);
#pragma unroll
  for (int i = 0; i < NSUB; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = i * 16 + 4 * (lane >> 4) + e;
      if (r < Mt) y[(int64_t)(m0 + r) * ldy + col] = bf16_rne(acc[i][e]);
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

constexpr int kTargetWGs = 256;  // one workgroup per CU of the MI355X

// MFMA waves that share one column group when a workgroup owns CGW of them.
int waves_per_group(int CGW) { return CGW >= 3 ? 1 : 4 / CGW; }

// Column groups per workgroup for C-column groups (1 when they do not split evenly over 256).
int groups_per_wg(int N, int C) {
  const int CG = N / C;
  if (CG % kTargetWGs != 0) return 1;
  int nwg = kTargetWGs, CGW = CG / nwg;
  while (CGW > kMaxMfmaWaves && CG % (2 * nwg) == 0) { nwg *= 2; CGW = CG / nwg; }
  return CGW > kMaxMfmaWaves ? 1 : CGW;
}

// Columns per group of the packed layout for an [N, K] weight: the widest C whose column-group
// count is a multiple of 256 (equal weight bytes per CU), whose K-blocks per fragment divide
// K / 128, and whose rounds fit the 32 staged K blocks; 16 when none is.
int layout_columns(int N, int K) {
  const int KB = K / 128;
  for (int c : {16, 8, 4, 2}) {
    const int S = 16 / c;
    if (KB % S != 0 || (N / c) % kTargetWGs != 0) continue;
    if (S * waves_per_group(groups_per_wg(N, c)) * 4 > kKCMax) continue;
    return c;
  }
  return 16;
}

uint32_t layout_id_for(int N, int K) { return 0x46380200u | (uint32_t)layout_columns(N, K); }

struct Plan {
  int C, CGW, nwg, NWK, NWC, NCG, NKG, NWM, KC, QW;
};

// Quantising waves for a round of `groups` 1x128 groups next to nwm MFMA waves: about two
// 16-group passes per wave, as 2, 4, 8 or 12 waves, and a multiple of 4 when more than 2 so that
// every SIMD (wave w runs on SIMD w % 4) carries the same share of the quantiser's VALU work.
int quant_waves(int groups, int nwm) {
  const int need = (groups + 31) / 32;
  const int qw = need <= 2 ? 2 : (need <= 4 ? 4 : (need <= 8 ? 8 : 12));
  const int room = 16 - nwm;
  return min(qw, room >= 4 ? room / 4 * 4 : 2);
}

Plan make_plan(int M, int N, int K) {
  Plan p;
  p.C = layout_columns(N, K);
  const int S = 16 / p.C;
  const int KB = K / 128;
  const int KG = KB / S;
  const int Mr = min(M, 32);  // rows per workgroup
  p.CGW = groups_per_wg(N, p.C);
  p.nwg = (N / p.C) / p.CGW;
  // One M tile: waves that share their activation tiles between NCG = 5 or 3 column groups, one
  // K group per wave and round, when that still gives at least 4 MFMA waves; else (and for two M
  // tiles, whose accumulators would not fit) one column group per wave.  NWK is the largest
  // divisor of the K groups that fits, so that every round is full.
  p.NCG = 0;
  for (int ncg : {5, 3}) {
    if (p.CGW % ncg != 0 || ncg * 8 + S * 8 + ncg * 4 > 100) continue;  // registers
    const int nwc = p.CGW / ncg;
    const int cap = min(kMaxMfmaWaves / nwc, kKCMax / S);
    int nwk = 0;
    for (int d = 1; d <= cap; ++d)
      if (KG % d == 0) nwk = d;
    if (nwk * nwc < 4) continue;
    // When the quantising waves that fit beside nwk * nwc MFMA waves would still take five or
    // more passes each, the next smaller divisor (as long as it needs at most two rounds) frees
    // waves for the quantiser: its VALU work, not the weight stream, is then what the kernel waits for.
    const int g = Mr * min(KB, nwk * S);
    const int qw = quant_waves(g, nwk * nwc);
    const int passes = (g + 16 * qw - 1) / (16 * qw) * ((KB + nwk * S - 1) / (nwk * S));
    if (passes >= 5) {
      int d = nwk - 1;
      while (d >= 1 && KG % d != 0) --d;
      if (d >= 1 && (KB + d * S - 1) / (d * S) <= 2) nwk = d;
    }
    p.NCG = ncg; p.NKG = 1; p.NWC = nwc; p.NWK = nwk;
    break;
  }
  if (p.NCG == 0) {
    p.NCG = 1;
    p.NWC = p.CGW;
    p.NWK = waves_per_group(p.CGW);
    p.NKG = (S * p.NWK * 8 <= kKCMax && KG >= 8 * p.NWK) ? 8 : 4;
  }
  p.NWM = p.NWK * p.NWC;
  p.KC = p.NKG * p.NWK * S;
  p.QW = quant_waves(Mr * min(KB, p.KC), p.NWM);
  return p;
}

template <int MODE, int MT, int C>
void launch_c(const Plan& pl, dim3 grid, hipStream_t stream, const void* a, int64_t lda, const void* sa,
              const uint8_t* wp, const void* sw, uint16_t* y, int64_t ldy, int M, int K, uint8_t* q_dbg,
              void* sx_dbg) {
  const dim3 block(64 * (pl.QW + pl.NWM));
#define SMALLM_LAUNCH(ncg, nkg)                                                                          \
  hipLaunchKernelGGL((smallm_gemm_kernel<MT, C, ncg, nkg, MODE>), grid, block, 0, stream, a, lda, sa, wp, \
                     sw, y, ldy, M, K, pl.CGW, pl.NWK, pl.NWC, pl.QW, q_dbg, sx_dbg)
  if constexpr (C != 2) {
    if (pl.NCG == 5) { SMALLM_LAUNCH(5, 1); return; }
  }
  if (pl.NCG == 3) { SMALLM_LAUNCH(3, 1); return; }
  if (pl.NKG == 8) SMALLM_LAUNCH(1, 8);
  else SMALLM_LAUNCH(1, 4);
#undef SMALLM_LAUNCH
}

template <int MODE>
int launch_gemm(const void* a, int64_t lda, const void* sa, const uint8_t* wp, const void* sw,
                uint16_t* y, int64_t ldy, int M, int N, int K, uint8_t* q_dbg, void* sx_dbg,
                hipStream_t stream) {
  const Plan pl = make_plan(M, N, K);
  const int MT = (M <= 16) ? 1 : 2;
  const int MP = 16 * MT;
  dim3 grid(pl.nwg, (M + MP - 1) / MP);
#define SMALLM_C(mt)                                                                                  \
  switch (pl.C) {                                                                                     \
    case 16: launch_c<MODE, mt, 16>(pl, grid, stream, a, lda, sa, wp, sw, y, ldy, M, K, q_dbg, sx_dbg); break; \
    case 8: launch_c<MODE, mt, 8>(pl, grid, stream, a, lda, sa, wp, sw, y, ldy, M, K, q_dbg, sx_dbg); break;   \
    case 4: launch_c<MODE, mt, 4>(pl, grid, stream, a, lda, sa, wp, sw, y, ldy, M, K, q_dbg, sx_dbg); break;   \
    default: launch_c<MODE, mt, 2>(pl, grid, stream, a, lda, sa, wp, sw, y, ldy, M, K, q_dbg, sx_dbg); break;  \
  }
  if (MT == 1) { SMALLM_C(1) } else { SMALLM_C(2) }
#undef SMALLM_C
  return launch_status();
}

// The pre-quantised GEMM takes the MFMA-tiled kernel beyond the small-M range when the weight
// is packed in 16-column groups (one fragment per MFMA B operand) and a 64-row tile of q spans
// less than 2 GiB.
bool use_tiled(int M, int N, int K, int64_t ldq) {
  return M > kTiledFromM && layout_columns(N, K) == 16 && K / 128 <= kTiledMaxKB &&
         ldq * (kTM - 1) + K < ((int64_t)1 << 31);
}

template <bool E8>
int launch_tiled(const uint8_t* q, int64_t ldq, const void* sa, const uint8_t* wp, const void* sw,
                 uint16_t* y, int64_t ldy, int M, int N, int K, hipStream_t stream) {
  const dim3 grid(N / 64, (M + kTM - 1) / kTM);
  hipLaunchKernelGGL((tiled_gemm_kernel<kTM, E8>), grid, dim3(256), 0, stream, q, ldq, sa, wp, sw,
                     y, ldy, M, K);
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
  switch (layout_columns(N, K)) {
    case 16: hipLaunchKernelGGL((pack_kernel<PACK, 16>), grid, dim3(256), 0, stream, src, dst, K, chunks); break;
    case 8: hipLaunchKernelGGL((pack_kernel<PACK, 8>), grid, dim3(256), 0, stream, src, dst, K, chunks); break;
    case 4: hipLaunchKernelGGL((pack_kernel<PACK, 4>), grid, dim3(256), 0, stream, src, dst, K, chunks); break;
    default: hipLaunchKernelGGL((pack_kernel<PACK, 2>), grid, dim3(256), 0, stream, src, dst, K, chunks); break;
  }
}

}  // namespace

extern "C" {

int smallm_fp8bs_abi_version(void) { return SMALLM_FP8BS_ABI_VERSION; }

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

int smallm_fp8bs_launch_plan(int M, int N, int K, int* plan10) {
  if (!plan10) return SMALLM_ERR_INVALID;
  int st = check_mnk(M, N, K);
  if (st) return st;
  const Plan p = make_plan(M, N, K);
  const int MT = (M <= 16) ? 1 : 2;
  const int v[10] = {p.C, p.CGW, p.nwg, p.NWK, p.NWC, p.NCG, p.NKG, p.KC, p.QW, MT};
  for (int i = 0; i < 10; ++i) plan10[i] = v[i];
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
  if (use_tiled(M, N, K, ldq)) return launch_tiled<false>(q, ldq, sx, w_packed, sw, y, ldy, M, N, K, (hipStream_t)stream);
  return launch_gemm<kPreqF32>(q, ldq, sx, w_packed, sw, y, ldy, M, N, K, nullptr, nullptr,
                               (hipStream_t)stream);
}

int smallm_fp8bs_gemm_e8m0(const uint8_t* q, int64_t ldq, const uint8_t* sx_e8m0,
                           const uint8_t* w_packed, uint32_t layout_id, const uint8_t* sw_e8m0,
                           uint16_t* y, int64_t ldy, int M, int N, int K, void* stream) {
  int st = check_gemm_args(q, ldq, 1, sx_e8m0, true, w_packed, layout_id, sw_e8m0, y, ldy, M, N, K);
  if (st) return st;
  if (use_tiled(M, N, K, ldq)) return launch_tiled<true>(q, ldq, sx_e8m0, w_packed, sw_e8m0, y, ldy, M, N, K, (hipStream_t)stream);
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

}  // extern "C"
