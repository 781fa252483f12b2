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
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kLayoutId = 0x46384231u;  // "1B8F": 16x128 MFMA-B fragments, v1
constexpr int kThreads = 512;                // 8 waves: 4 quantise, 4 MFMA
constexpr int kRowStride = 144;              // LDS row pitch of the staged e4m3 rows (128 + 16 pad)

// ---------------------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float quad_max_f32(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

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

// Quantise 32 consecutive bf16 of one 1x128 group (this lane's quarter; the group is spread
// over a DPP quad) with an fp32 group scale.  Returns the scale, writes 32 e4m3 bytes.
__device__ __forceinline__ float quant32_fp32(const u32x4 (&xv)[4], u32x4 (&qv)[2]) {
  float f[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t d = xv[i >> 2][i & 3];
    f[2 * i] = __uint_as_float(d << 16);
    f[2 * i + 1] = __uint_as_float(d & 0xFFFF0000u);
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(f[i]));
  am = quad_max_f32(am);
  const float s = am / 448.0f;                    // correctly rounded fp32 division
  const float y = (am > 0.0f) ? 1.0f / s : 0.0f;  // correctly rounded reciprocal
  float qf[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float q0 = f[i] * y;
    const float r = __builtin_fmaf(q0, s, -f[i]);
    qf[i] = __builtin_fmaf(-r, y, q0);
  }
  if (s > 0.0f && s < 0x1p-64f) {  // tiny group scale: plain IEEE division
#pragma unroll
    for (int i = 0; i < 32; ++i) qf[i] = f[i] / s;
  }
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(qf[4 * j], qf[4 * j + 1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(qf[4 * j + 2], qf[4 * j + 3], p, true);
    w[j] = (uint32_t)p;
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

template <bool PACK>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   int K, int64_t chunks) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= chunks) return;
  const int KB = K >> 7;
  const int64_t f = o >> 7;
  const int within = (int)(o & 127), h = within >> 6, lane = within & 63;
  const int64_t n = (f / KB) * 16 + (lane & 15);
  const int64_t k = (f % KB) * 128 + (lane >> 4) * 32 + h * 16;
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
// the GEMM (fused quant or pre-quantised input; fp32 or e8m0 scales)
// ---------------------------------------------------------------------------------------------

enum Mode { kFusedF32 = 0, kFusedE8 = 1, kPreqF32 = 2, kPreqE8 = 3 };

template <int MT, int NT, int MODE>
struct GemmCfg {
  static constexpr bool kE8 = (MODE & 1) != 0;
  static constexpr bool kPreq = (MODE & 2) != 0;
  static constexpr int kMP = 16 * MT;               // rows per workgroup (M padded to the MFMA)
  static constexpr int kBPW = (NT <= 2) ? 8 : 4;    // K blocks per MFMA wave per round
  static constexpr int kKC = 4 * kBPW;              // K blocks per round
  static constexpr int kStq = kKC * kMP * kRowStride;
  static constexpr int kSts = kKC * kMP * (kE8 ? 1 : 4);
  static constexpr int kRed = 4 * MT * NT * 4 * 64 * 4;
  static constexpr int kSmem = ((kStq + kSts) > kRed ? (kStq + kSts) : kRed);
};

template <int MT, int NT, int MODE>
__global__ __launch_bounds__(kThreads) void smallm_gemm_kernel(
    const void* __restrict__ a_src, int64_t lda, const void* __restrict__ sa_src,
    const uint8_t* __restrict__ wp, const void* __restrict__ sw, uint16_t* __restrict__ y,
    int64_t ldy, int M, int K, uint8_t* __restrict__ q_dbg, void* __restrict__ sx_dbg) {
  using C = GemmCfg<MT, NT, MODE>;
  constexpr int MP = C::kMP, BPW = C::kBPW, KC = C::kKC;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];
  uint8_t* stq = smem;
  float* sts_f = (float*)(smem + C::kStq);
  uint8_t* sts_b = smem + C::kStq;
  float* red = (float*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K >> 7;
  const int n0 = blockIdx.x * (NT * 16);
  const int m0 = blockIdx.y * MP;
  const int Mc = min(M - m0, MP);

  v4f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int rounds = (KB + KC - 1) / KC;
  for (int rd = 0; rd < rounds; ++rd) {
    const int kb0 = rd * KC;
    const int KBr = min(KC, KB - kb0);
    if (wave >= 4) {
      // ---- MFMA waves: stream this round's weight fragments, then multiply ----
      const int mw = wave - 4;
      u32x4 wr[NT][BPW][2];
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int kbl = mw + 4 * j;
        if (kbl < KBr) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const u32x4* p = (const u32x4*)(wp + ((int64_t)(n0 / 16 + t) * KB + kb0 + kbl) * 2048) + lane;
            wr[t][j][0] = __builtin_nontemporal_load(p);
            wr[t][j][1] = __builtin_nontemporal_load(p + 64);
          }
        }
      }
      __syncthreads();  // activation bytes and scales of this round are staged
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int kbl = mw + 4 * j;
        if (kbl < KBr) {
          const int kb = kb0 + kbl;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int row = mt * 16 + (lane & 15);
            v8i a = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            if (row < Mc) {
              const u32x4* ap = (const u32x4*)(stq + (kbl * MP + row) * kRowStride + (lane >> 4) * 32);
              const u32x4 a0 = ap[0], a1 = ap[1];
              a = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            }
            if (C::kE8) {
              const int sa = (row < Mc) ? (int)sts_b[kbl * MP + row] : 127;
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const int nb = (n0 + 16 * t) >> 7;
                const int sb = (int)((const uint8_t*)sw)[nb * KB + kb];
                const v8i b = __builtin_bit_cast(v8i, __builtin_shufflevector(wr[t][j][0], wr[t][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
                acc[mt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[mt][t], 0, 0, 0, sa, 0, sb);
              }
            } else {
              const v4f sx4 = *(const v4f*)(sts_f + kbl * MP + mt * 16 + 4 * (lane >> 4));
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const int nb = (n0 + 16 * t) >> 7;
                const float swv = ((const float*)sw)[nb * KB + kb];
                const v8i b = __builtin_bit_cast(v8i, __builtin_shufflevector(wr[t][j][0], wr[t][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(sx4[i] * swv, p[i], acc[mt][t][i]);
              }
            }
          }
        }
      }
      __syncthreads();  // staging buffer free for the next round
    } else {
      // ---- quantising (or staging) waves: one DPP quad per 1x128 group ----
      const int slot = wave * 16 + (lane >> 2);
      const int c = lane & 3;
      const int G = Mc * KBr;
      for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + slot;
        const bool valid = g < G;
        const int kbl = valid ? g / Mc : 0;
        const int m = valid ? g % Mc : 0;
        const int kb = kb0 + kbl;
        u32x4 qv[2];
        float s = 0.0f;
        uint32_t e = 0;
        if (!C::kPreq) {
          const u32x4* xp = (const u32x4*)((const uint16_t*)a_src + (int64_t)(m0 + m) * lda + kb * 128 + c * 32);
          u32x4 xv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) xv[i] = valid ? xp[i] : u32x4{0, 0, 0, 0};
          if (C::kE8) e = quant32_e8m0(xv, qv);
          else s = quant32_fp32(xv, qv);
        } else {
          const u32x4* qp = (const u32x4*)((const uint8_t*)a_src + (int64_t)(m0 + m) * lda + kb * 128 + c * 32);
          qv[0] = valid ? qp[0] : u32x4{0, 0, 0, 0};
          qv[1] = valid ? qp[1] : u32x4{0, 0, 0, 0};
          if (valid && c == 0) {
            if (C::kE8) e = ((const uint8_t*)sa_src)[(int64_t)(m0 + m) * KB + kb];
            else s = ((const float*)sa_src)[(int64_t)(m0 + m) * KB + kb];
          }
        }
        if (valid) {
          u32x4* dp = (u32x4*)(stq + (kbl * MP + m) * kRowStride + c * 32);
          dp[0] = qv[0];
          dp[1] = qv[1];
          if (c == 0) {
            if (C::kE8) sts_b[kbl * MP + m] = (uint8_t)e;
            else sts_f[kbl * MP + m] = s;
          }
          if (!C::kPreq && q_dbg != nullptr && blockIdx.x == 0) {
            u32x4* qd = (u32x4*)(q_dbg + (int64_t)(m0 + m) * K + kb * 128 + c * 32);
            qd[0] = qv[0];
            qd[1] = qv[1];
          }
          if (!C::kPreq && sx_dbg != nullptr && blockIdx.x == 0 && c == 0) {
            if (C::kE8) ((uint8_t*)sx_dbg)[(int64_t)(m0 + m) * KB + kb] = (uint8_t)e;
            else ((float*)sx_dbg)[(int64_t)(m0 + m) * KB + kb] = s;
          }
        }
      }
      __syncthreads();
      __syncthreads();
    }
  }

  // ---- cross-wave reduction through LDS (staging space reused), fixed order, bf16 store ----
  if (wave >= 4) {
    const int mw = wave - 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(((mw * MT + mt) * NT + t) * 4 + i) * 64 + lane] = acc[mt][t][i];
  }
  __syncthreads();
  constexpr int NCOL = NT * 16;
  for (int o = tid; o < MP * NCOL; o += kThreads) {
    const int row = o / NCOL, col = o % NCOL;
    if (row < Mc) {
      const int mt = row >> 4, i = row & 3, t = col >> 4;
      const int l = ((row & 15) >> 2) * 16 + (col & 15);
      float sum = 0.0f;
#pragma unroll
      for (int mw = 0; mw < 4; ++mw) sum += red[(((mw * MT + mt) * NT + t) * 4 + i) * 64 + l];
      y[(int64_t)(m0 + row) * ldy + n0 + col] = bf16_rne(sum);
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

int tile_override() {
  static int v = [] {
    const char* e = getenv("SMALLM_FP8BS_NT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// Number of 16-column tiles per workgroup.
int choose_nt(int N, int M) {
  const int tiles = N / 16;
  const int o = tile_override();
  if ((o == 1 || o == 2 || o == 4) && tiles % o == 0) return o;
  (void)M;
  return (tiles % 2 == 0) ? 2 : 1;
}

template <int MODE>
int launch_gemm(const void* a, int64_t lda, const void* sa, const uint8_t* wp, const void* sw,
                uint16_t* y, int64_t ldy, int M, int N, int K, uint8_t* q_dbg, void* sx_dbg,
                hipStream_t stream) {
  const int MT = (M <= 16) ? 1 : 2;
  const int NT = choose_nt(N, M);
  const int MP = 16 * MT;
  dim3 grid(N / (16 * NT), (M + MP - 1) / MP);
  dim3 block(kThreads);
#define SMALLM_LAUNCH(mt, nt)                                                                   \
  hipLaunchKernelGGL((smallm_gemm_kernel<mt, nt, MODE>), grid, block, 0, stream, a, lda, sa, wp, \
                     sw, y, ldy, M, K, q_dbg, sx_dbg)
  if (MT == 1) {
    if (NT == 1) SMALLM_LAUNCH(1, 1);
    else if (NT == 2) SMALLM_LAUNCH(1, 2);
    else SMALLM_LAUNCH(1, 4);
  } else {
    if (NT == 1) SMALLM_LAUNCH(2, 1);
    else if (NT == 2) SMALLM_LAUNCH(2, 2);
    else SMALLM_LAUNCH(2, 4);
  }
#undef SMALLM_LAUNCH
  return launch_status();
}

int check_gemm_args(const void* a, int64_t lda, int a_elem_bytes, const void* sa_or_null_ok,
                    bool need_sa, const uint8_t* wp, uint32_t layout_id, const void* sw,
                    const uint16_t* y, int64_t ldy, int M, int N, int K) {
  if (!a || !wp || !sw || !y || (need_sa && !sa_or_null_ok)) return SMALLM_ERR_INVALID;
  int st = check_mnk(M, N, K);
  if (st) return st;
  if (lda < K || ldy < N) return SMALLM_ERR_SHAPE;
  if (!aligned16(a) || ((lda * a_elem_bytes) & 15) || !aligned16(wp) || ((uintptr_t)y & 1u))
    return SMALLM_ERR_ALIGN;
  if (layout_id != kLayoutId) return SMALLM_ERR_LAYOUT;
  return SMALLM_OK;
}

}  // namespace

extern "C" {

int smallm_fp8bs_abi_version(void) { return SMALLM_FP8BS_ABI_VERSION; }

uint32_t smallm_fp8bs_weight_layout_id(void) { return kLayoutId; }

const char* smallm_fp8bs_strerror(int status) {
  switch (status) {
    case SMALLM_OK: return "ok";
    case SMALLM_ERR_INVALID: return "a required pointer is NULL";
    case SMALLM_ERR_SHAPE: return "shape out of range (1 <= M <= 256, N and K multiples of 128, ld >= row length)";
    case SMALLM_ERR_ALIGN: return "pointer or row pitch not 16-byte aligned";
    case SMALLM_ERR_LAYOUT: return "packed weight layout id does not match this library";
    case SMALLM_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
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
  const int64_t chunks = (int64_t)N * K / 16;
  hipLaunchKernelGGL((pack_kernel<true>), dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, w8, w_packed, K, chunks);
  return launch_status();
}

int smallm_fp8bs_unpack_weight(const uint8_t* w_packed, uint8_t* w8, int N, int K, void* stream) {
  if (!w8 || !w_packed) return SMALLM_ERR_INVALID;
  if (N <= 0 || K <= 0 || (N & 127) || (K & 127)) return SMALLM_ERR_SHAPE;
  if (!aligned16(w8) || !aligned16(w_packed)) return SMALLM_ERR_ALIGN;
  const int64_t chunks = (int64_t)N * K / 16;
  hipLaunchKernelGGL((pack_kernel<false>), dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, w_packed, w8, K, chunks);
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

}  // extern "C"
