// moe_fp8bs.hip -- FP8 block-scale small-M fused MoE layer on MI355X (gfx950 / CDNA4).
//
//   h[t, s] = bf16(silu(g) * u),  (g | u) = x[t] . dequant(w13[e])^T,  e = ids[t, s]
//   y[t]    = bf16( sum_s tw[t, s] * h[t, s] . dequant(w2[e])^T )
//
// What is computed follows sglang "[AMD] gfx950 small-batch MoE: expert-count gate for the small
// sort and FP8 block-scale small-M kernel", section Modifications (e4m3 expert weights converted
// to bf16 at scale 1, one fp32 scale per 128x128 block applied to the block's partial sum), with
// the two-phase structure of sglang "[AMD] Small-M MXFP4 fused-MoE kernel for gfx950 (Qwen)",
// section Modifications (bf16 activations, phase 1 gate/up with silu(g) * u written as bf16,
// phase 2 the down projection with the top-k weights applied in fp32).  w13 holds the gate rows
// [0, I) above the up rows [I, 2 I).
//
// Design points of this implementation:
//
//  * No sort.  Each expert in use is streamed once per phase, with every token routed to it as
//    a row of the MFMA A operand.  Phase 1 works on (expert, 8-column slice) items.  Up to 128
//    pairs (32 for MXFP4) it launches one workgroup per (token, slot) pair and slice, and a
//    workgroup whose pair is not the first pair naming its expert exits.  Above, a fixed grid
//    (2048 workgroups, 3072 for MXFP4) lists the distinct experts in LDS and walks the items.  Either way the
//    expert's tokens are gathered with a ballot.  Phase 2 launches NS workgroups per 16 output
//    columns, each over a contiguous range of pairs; every workgroup finds the first pair of each expert with an LDS integer min
//    and its waves walk the experts whose first pair lies in its range, gathering each expert's
//    tokens into MFMA rows as phase 1 does.  With NS > 1 the workgroups leave fp32 partial sums
//    in the caller's workspace and the last of a tile's workgroups to finish adds them in range
//    order (two launches in every case).
//  * Packed weights: every 16-row x 128-K block of an expert matrix is one 2 KiB fragment in
//    the lane order of an MFMA operand (lane l = 16 c + j holds row j and K bytes [32 c, 32 c + 32)
//    of the block, bytes 0..15 in the first KiB and 16..31 in the second), fragments of one
//    16-row tile consecutive along K.  In w13 a tile holds 8 gate rows and the 8 up rows of the
//    same intermediate columns, so one workgroup owns both halves of silu(g) * u.
//  * Arithmetic: e4m3 bytes become bf16 with v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact), the
//    products run on v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact in fp32), each
//    128-K block's fp32 partial is multiplied by its block scale and added to an fp32
//    accumulator.  Per-wave split-K partials are summed through LDS in a fixed order, so every
//    result is deterministic and graph replays equal eager runs.
//  * MXFP4 experts (sglang "[AMD] Small-M MXFP4 fused-MoE kernel for gfx950 (Qwen)",
//    Modifications; OCP Microscaling e2m1 elements with one e8m0 scale per 32 K elements): the
//    same kernels with FP4 = true.  A fragment is 1 KiB (16 rows x 128 K as fp4x2); each lane's
//    16 bytes are exactly one scale group, whose byte is packed in fragment order beside it, and
//    v_cvt_scalef32_pk_bf16_fp4 applies that power of two while converting (exact).

#include <hip/hip_runtime.h>

#include <mutex>
#include <limits.h>
#include <stdint.h>

#include "../../include/smallm_fp8bs.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// phase 1: 8 waves per workgroup, each over K/128/8 blocks of the expert's 16 rows (16 waves
// measured slower from four tokens on: most workgroups only find that their pair is not the first
// of its expert, and a larger workgroup makes that dearer)
constexpr int kGateThreads = 512;
constexpr int kGateWaves = kGateThreads / 64;
// Phase 1 grid: one workgroup per pair and slice up to kGateItemsFrom pairs; above, a fixed grid
// of kGateGrid (kGateGridFp4) workgroups walking the (expert, two slices) items.  With one slice
// per item both item kernels fitted 64 VGPRs without spills (a scalar wave index; unmasked
// activation loads for FP8), so four workgroups shared a CU: 1024 resident at once; the grids
// below were measured then, and rechecked with two slices (FP8 at three workgroups per CU: 1536
// workgroups were level with 2048).  A grid of exactly
// 1024 assigns every workgroup ceil or floor of items / 1024 items, and a last round that only a
// few workgroups have costs a whole round (3088 items at 24 tokens, intermediate 128: four rounds
// for an average of three).  With two or three workgroups per slot the later ones start as slots
// free up, and the tail shrinks.  Measured (11 slots, hidden 4096): FP8 at intermediate 128, 1024
// / 2048 / 3072 workgroups took 73.7 / 70.5 / 72.4 us at 24 tokens, 87.4 / 83.4 / 84.3 at 32 and
// 113.8 / 109.8 / 109.4 at 48; MXFP4 took 74.6 / 72.8 / 70.8 us at 16 tokens and 145.7 / 141.8 /
// 136.5 at 40; one workgroup per possible item was no better and less steady.
// Against the per-pair grid, on the pages' shapes (11 slots), with one slice per item: the item
// grid took 87 us instead of 102 at 32 tokens and 114 instead of 129 at 48 (FP8, intermediate
// 128), 145 instead of 156 at 40 (MXFP4); 3-4 % faster at 16 tokens for both formats, and for
// MXFP4 3 % faster from four tokens on, while FP8 at 8 tokens and intermediate 256 was 1.6 %
// slower (the FP8 threshold was then 128 pairs).  With two slices per item the FP8 item grid is
// ahead from four tokens on as well: 54.5 -> 49.9 us at 8 tokens and 33.5 -> 31.5 at 4
// (intermediate 256), 34.0 -> 32.5 at 8 (intermediate 128; level at 4); one threshold serves both.
constexpr int kGateItemsFrom = 32;
constexpr int kGateGrid = 2048;
constexpr int kGateGridFp4 = 3072;
// phase 2: 16 waves per workgroup, each walking its own experts, at most 64 VGPRs so that two
// workgroups share a CU (66 VGPRs halved the occupancy and measured up to 25 % slower)
constexpr int kDownThreads = 1024;
constexpr int kDownWaves = kDownThreads / 64;
constexpr int kMoePairs = SMALLM_FP8BS_MOE_MAX_T * SMALLM_FP8BS_MOE_MAX_S;
constexpr uint32_t kMoeLayoutId = 0x4D4F4510u;
constexpr uint32_t kMoeFp4LayoutId = 0x4D4F4504u;

// the eight e4m3 bytes of two dwords as one 8-value bf16 MFMA operand (exact)
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t d0, uint32_t d1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const v2bf e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// the 32 e4m3 bytes a lane holds for one 128-K block, as four 8-value bf16 MFMA operands
__device__ __forceinline__ void e4m3x32_to_bf16(const u32x4& lo, const u32x4& hi, v8bf out[4]) {
  out[0] = e4m3x8_to_bf16(lo.x, lo.y);
  out[1] = e4m3x8_to_bf16(lo.z, lo.w);
  out[2] = e4m3x8_to_bf16(hi.x, hi.y);
  out[3] = e4m3x8_to_bf16(hi.z, hi.w);
}

// the eight e2m1 values of one dword (even K element in each byte's low nibble) as one 8-value
// bf16 MFMA operand, scaled by a power of two inside the conversion
__device__ __forceinline__ v8bf fp4x8_to_bf16(uint32_t d, float scale) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2);
  const v2bf e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// the 16 fp4x2 bytes a lane holds (32 e2m1 values of one 32-wide scale group) as four 8-value
// bf16 MFMA operands, scaled by the group's power of two inside the conversion
__device__ __forceinline__ void fp4x32_to_bf16(const u32x4& w, float scale, v8bf out[4]) {
  out[0] = fp4x8_to_bf16(w.x, scale);
  out[1] = fp4x8_to_bf16(w.y, scale);
  out[2] = fp4x8_to_bf16(w.z, scale);
  out[3] = fp4x8_to_bf16(w.w, scale);
}

// e8m0 byte b (1 <= b <= 254) as the fp32 2^(b - 127)
__device__ __forceinline__ float e8m0_f32(uint32_t b) { return __builtin_bit_cast(float, b << 23); }

__device__ __forceinline__ v4f mfma_bf16(const u32x4& a, const v8bf& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load_nt(const uint8_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ uint16_t bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
}

// ---------------------------------------------------------------------------------------------
// phase 1: gate/up GEMM of one expert for all its tokens, silu(g) * u -> h (bf16)
// ---------------------------------------------------------------------------------------------
//
// Work item (e, q): expert e's 8-column slice q, 512 threads.  Its A rows are the tokens routed to
// e, ascending, in tiles of 16 (rows past the last token are zero); its 16 columns are the gate
// rows 8q..8q+7 and up rows I+8q..I+8q+7 of e.  Two grids hand out the items (below).

// The split-K loop of phase 1 for one 16-row tile: wave w takes K blocks w, w + 8, ...  (one
// block's loads in flight per wave: issuing several blocks' loads first raised the registers from
// 48 to 120 and, with fewer workgroups per CU, measured slower from four tokens on).
// e4m3 weights (FP4 false): each block's four MFMAs give the fp32 partial that its 128x128 scale
// multiplies into acc.  MXFP4 weights (FP4 true): the 32-wide group scales are applied by the
// conversion to bf16, so the MFMAs accumulate into acc.  Every partial is added in the same block
// of code as its MFMAs (no MFMA result crosses a branch).  NSL consecutive slices of the expert
// (16 columns each, their fragments adjacent in the packed layout) share each block's activation
// loads, one accumulator each.
// DENSE: every lane loads its activation row (rows past the token count read a valid row and are
// zeroed after the load), which saves the exec-mask branches and the registers they hold; masked
// loads (DENSE false) keep the empty rows off the load pipeline that the weight stream shares.
template <bool FP4, bool DENSE, int NSL>
__device__ __forceinline__ void gate_up_loop(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr, int srow,
                                             const uint16_t* xr, bool row_ok, int KB, int wave,
                                             v4f (&acc)[NSL]) {
  const int lane = threadIdx.x & 63;
  constexpr uint32_t FB = FP4 ? 1024u : 2048u;  // bytes of a 16-column fragment of one K block
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) acc[sl] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int kb = wave; kb < KB; kb += kGateWaves) {
    // the item's fragments (its NSL slices one after another) through a wave-uniform buffer
    // resource: 32-bit lane offsets instead of 64-bit addresses
    u32x4 b0[NSL], b1[NSL];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const uint32_t o = (uint32_t)(sl * KB + kb) * FB + (uint32_t)lane * 16u;
      b0[sl] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, o, 0, 2));
      if constexpr (!FP4)
        b1[sl] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, o + 1024u, 0, 2));
    }
    const u32x4* xa = (const u32x4*)(xr + kb * 128);
    u32x4 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DENSE) {
        const u32x4 v = xa[i];
        a[i] = row_ok ? v : u32x4{0u, 0u, 0u, 0u};
      } else {
        a[i] = row_ok ? xa[i] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    // each 8-value operand is converted just before the MFMA that takes it
    if constexpr (FP4) {
      // the group scales are applied by the conversion: the MFMAs accumulate into acc
      float scl[NSL];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
        scl[sl] = e8m0_f32(
            __builtin_amdgcn_raw_buffer_load_b8(sr, (uint32_t)((sl * KB + kb) * 64 + lane), 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
          acc[sl] = mfma_bf16(a[i], fp4x8_to_bf16(b0[sl][i], scl[sl]), acc[sl]);
    } else {
      // e4m3: each block's MFMAs give the fp32 partial that its 128x128 scale (the same for the
      // item's slices) multiplies into acc
      const float sc = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(sr, (uint32_t)(srow * KB + kb) * 4u, 0, 0));
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        v4f pm = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4& w = i < 2 ? b0[sl] : b1[sl];
          pm = mfma_bf16(a[i], e4m3x8_to_bf16(w[2 * (i & 1)], w[2 * (i & 1) + 1]), pm);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[sl][i] = acc[sl][i] + sc * pm[i];
      }
    }
  }
  // MXFP4: the loop ends in a branch and its last MFMAs write acc; 16 wait states on every path
  // before acc is read
  if constexpr (FP4) {
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[sl]));
  }
}

// Phase 1 for one work item: expert e's 8-column slices q .. q + NSL - 1, for the Me tokens listed
// (ascending) in s_tok.  All threads of the workgroup call it; it ends with a barrier, after which
// s_tok may be rewritten.
template <bool FP4, bool DENSE, int NSL>
__device__ __forceinline__ void gate_up_item(
    int e, int q, int Me, const int* s_ids, const int* s_tok, float* s_red,
    const uint16_t* __restrict__ x, int64_t ldx, int S, const uint8_t* __restrict__ w13,
    const float* __restrict__ sw13, const uint8_t* __restrict__ s13, int H, int I,
    uint16_t* __restrict__ h) {
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: loop counters, scale loads and addresses derived from it
  // stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the expert, slice and token count are the same in every lane (read from LDS): scalar registers
  e = __builtin_amdgcn_readfirstlane(e);
  q = __builtin_amdgcn_readfirstlane(q);
  Me = __builtin_amdgcn_readfirstlane(Me);
  const int tiles = (Me + 15) >> 4;
  const int KB = H >> 7;
  const int j = lane & 15, chunk = lane >> 4;
  // column j < 8 is gate row 8q + j (scale block row q / 16), j >= 8 the matching up row
  const int srow = (j < 8) ? (q >> 4) : ((I >> 7) + (q >> 4));
  // the item's weights: MXFP4 1 KiB fragments and, in fragment order, one group-scale byte per
  // lane; e4m3 2 KiB fragments and the expert's 128x128 block scales [2I / 128, KB]
  const int64_t wbase = FP4 ? (int64_t)e * I * H + (int64_t)q * KB * 1024
                            : (int64_t)e * 2 * I * H + (int64_t)q * KB * 2048;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w13 + wbase), 0, NSL * KB * (FP4 ? 1024 : 2048), 0x00020000);
  const __amdgpu_buffer_rsrc_t sr =
      FP4 ? __builtin_amdgcn_make_buffer_rsrc(
                (void*)(s13 + (int64_t)e * 2 * I * (H >> 5) + (int64_t)q * KB * 64), 0, NSL * KB * 64, 0x00020000)
          : __builtin_amdgcn_make_buffer_rsrc(
                (void*)(sw13 + (int64_t)e * (I >> 6) * KB), 0, (I >> 6) * KB * 4, 0x00020000);
  // the row tiles one after another (only an expert with more than 16 tokens, in practice the
  // shared one, has a second or third; its weight slice is then re-read from L2)
  for (int tile = 0; tile < tiles; ++tile) {
    const int idx = 16 * tile + j;
    const bool row_ok = idx < Me;
    const uint16_t* xr = x + (int64_t)(row_ok ? s_tok[idx] : 0) * ldx + chunk * 32;
    v4f acc[NSL];
    gate_up_loop<FP4, DENSE, NSL>(wr, sr, srow, xr, row_ok, KB, wave, acc);
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_red[((sl * kGateWaves + wave) * 4 + i) * 64 + lane] = acc[sl][i];
    __syncthreads();
    if (tid < 128 * NSL) {
      const int sl = tid >> 7, r = (tid >> 3) & 15, c = tid & 7;
      const int k = 16 * tile + r;
      if (k < Me) {
        const int t = s_tok[k];
        // D row r, column c sits in lane 16 (r / 4) + c, register r % 4
        const int base = (r & 3) * 64 + 16 * (r >> 2) + c;
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int w = 0; w < kGateWaves; ++w) {
          g = g + s_red[(sl * kGateWaves + w) * 256 + base];
          u = u + s_red[(sl * kGateWaves + w) * 256 + base + 8];
        }
        const uint16_t hb = bf16_bits((g / (1.0f + expf(-g))) * u);
        for (int s = 0; s < S; ++s)
          if (s_ids[t * S + s] == e) h[(int64_t)(t * S + s) * I + 8 * (q + sl) + c] = hb;
      }
    }
    __syncthreads();
  }
}

// Wave 0 lists the tokens routed to expert e in s_tok (ascending), the count in s_tok[MAX_T].
__device__ __forceinline__ void gather_tokens(int e, int T, int S, const int* s_ids, int* s_tok) {
  const int lane = threadIdx.x & 63;
  bool mine = false;
  if (lane < T)
    for (int s = 0; s < S; ++s) mine |= (s_ids[lane * S + s] == e);
  const uint64_t m = __ballot(mine);
  // the routed lanes below this one, counted by mbcnt (no 64-bit lane mask held in registers)
  if (mine) s_tok[__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = lane;
  if (lane == 0) s_tok[SMALLM_FP8BS_MOE_MAX_T] = __popcll(m);
}

// Phase 2's per-tile arrival counters start every call at zero: one workgroup of phase 1 clears
// them (the launches are ordered on the stream, so phase 2 sees the zeros).
__device__ __forceinline__ void zero_counters(uint32_t* cnt, int ncnt) {
  for (int i = threadIdx.x; i < ncnt; i += blockDim.x) cnt[i] = 0u;
}

// Up to 128 pairs (32 for MXFP4): grid (T * S, I / 8).  Workgroup (p, q) works when pair p is
// the first pair naming its expert e, on item (e, q); the others leave after one pass over the
// ids in LDS.
template <bool FP4>
__global__ __launch_bounds__(kGateThreads) void moe_gate_up_pairs_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ ids, int T, int S,
    int E, const uint8_t* __restrict__ w13, const float* __restrict__ sw13,
    const uint8_t* __restrict__ s13, int H, int I, uint16_t* __restrict__ h, uint32_t* __restrict__ cnt,
    int ncnt) {
  __shared__ int s_ids[kMoePairs];
  __shared__ int s_tok[SMALLM_FP8BS_MOE_MAX_T + 1];
  __shared__ float s_red[kGateWaves * 4 * 64];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int P = T * S;
  const int p = blockIdx.x, q = blockIdx.y;
  if (p == 0 && q == 0) zero_counters(cnt, ncnt);
  for (int i = tid; i < P; i += kGateThreads) s_ids[i] = ids[i];
  __syncthreads();
  const int e = s_ids[p];
  if (e < 0 || e >= E) return;
  bool earlier = false;
  for (int i = tid; i < p; i += kGateThreads) earlier |= (s_ids[i] == e);
  if (wave == 0) gather_tokens(e, T, S, s_ids, s_tok);
  if (__syncthreads_or(earlier)) return;
  gate_up_item<FP4, false, 1>(e, q, s_tok[SMALLM_FP8BS_MOE_MAX_T], s_ids, s_tok, s_red, x, ldx, S,
                              w13, sw13, s13, H, I, h);
}

// Above that: at most kGateGrid workgroups.  Every workgroup lists the distinct experts in
// LDS, ordered by the first pair naming each, and takes the items (d-th distinct expert, slices
// q and q + 1) blockIdx.x, blockIdx.x + gridDim.x, ...; every wave runs the same bounded loop.
// MXFP4 fits 64 VGPRs (eight waves per SIMD, four workgroups per CU); FP8, with twice the weight
// registers, 72 (seven waves per SIMD, three workgroups per CU).
template <bool FP4>
__global__ __launch_bounds__(kGateThreads) __attribute__((amdgpu_waves_per_eu(FP4 ? 8 : 7)))
void moe_gate_up_items_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ ids, int T, int S,
    int E, const uint8_t* __restrict__ w13, const float* __restrict__ sw13,
    const uint8_t* __restrict__ s13, int H, int I, uint16_t* __restrict__ h, uint32_t* __restrict__ cnt,
    int ncnt) {
  __shared__ int s_ids[kMoePairs];
  __shared__ int s_first[SMALLM_FP8BS_MOE_MAX_E];   // first pair naming each expert
  __shared__ int s_dexp[kMoePairs];                 // the distinct experts, by first pair
  __shared__ int s_nd;
  __shared__ int s_tok[SMALLM_FP8BS_MOE_MAX_T + 1];
  constexpr int NSL = 2;  // 8-column slices per item
  __shared__ float s_red[NSL * kGateWaves * 4 * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: loop counters, scale loads and addresses derived from it
  // stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = T * S;
  if (blockIdx.x == 0) zero_counters(cnt, ncnt);
  for (int i = tid; i < P; i += kGateThreads) s_ids[i] = ids[i];
  for (int i = tid; i < E; i += kGateThreads) s_first[i] = INT_MAX;
  __syncthreads();
  for (int i = tid; i < P; i += kGateThreads) {
    const int e = s_ids[i];
    if (e >= 0 && e < E) atomicMin(&s_first[e], i);
  }
  __syncthreads();
  if (wave == 0) {
    int nd = 0;
    for (int c0 = 0; c0 < P; c0 += 64) {
      const int pp = c0 + lane;
      const int e = pp < P ? s_ids[pp] : -1;
      const bool first = e >= 0 && e < E && s_first[e] == pp;
      const uint64_t m = __ballot(first);
      if (first) s_dexp[nd + __popcll(m & ((1ull << lane) - 1ull))] = e;
      nd += __popcll(m);
    }
    if (lane == 0) s_nd = nd;
  }
  __syncthreads();
  const int QN = (I >> 3) / NSL;
  const int items = s_nd * QN;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int e = s_dexp[item / QN], q = NSL * (item % QN);
    if (wave == 0) gather_tokens(e, T, S, s_ids, s_tok);
    __syncthreads();
    // masked activation loads (unmasked ones measured no faster with two slices per item)
    gate_up_item<FP4, false, NSL>(e, q, s_tok[SMALLM_FP8BS_MOE_MAX_T], s_ids, s_tok, s_red, x, ldx, S,
                                 w13, sw13, s13, H, I, h);
  }
}

// ---------------------------------------------------------------------------------------------
// phase 2: down projection, top-k weights in fp32, sum over slots -> y (bf16)
// ---------------------------------------------------------------------------------------------
//
// grid (H / 16, NS), 1024 threads.  Workgroup (b, z) owns output columns [16 b, 16 b + 16) and the
// pairs [z P / NS, (z + 1) P / NS).  The experts whose first pair lies in that range, in pair
// order, are dealt round-robin to the 16 waves; for each of its experts e a wave gathers the
// tokens routed to e with a ballot (ascending, each with the first slot naming e and the sum of
// the top-k weights of the slots naming e), runs one 16-row MFMA tile per 16 of those tokens over
// the expert's K blocks, and adds weight * (h . w2[e]^T) into the token's row of its own LDS
// slice.  The slices meet in wave
// order.  With NS = 1 the workgroup writes bf16 y.  Otherwise it writes its fp32 partial
// [z][t][n] with device-coherent stores (written through to the point where every XCD sees them;
// a device-scope fence instead would write back and invalidate the whole L2, which measured
// several times slower), waits until they are complete, and counts its arrival on the tile's
// counter; the workgroup that arrives last reads the other partials with device-coherent loads,
// adds them in z order and writes bf16 y.  Every result is deterministic.

template <int MT, bool FP4>
__global__ __launch_bounds__(kDownThreads, 8) void moe_down_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ tw,
    int T, int S, int E, const uint8_t* __restrict__ w2, const float* __restrict__ sw2,
    const uint8_t* __restrict__ s2, int H, int I, uint16_t* __restrict__ y, int64_t ldy,
    float* __restrict__ part, uint32_t* __restrict__ cnt) {
  constexpr int ROWS = 16 * MT;
  __shared__ int s_last;
  __shared__ int s_ids[kMoePairs];
  __shared__ float s_tw[kMoePairs];
  __shared__ int s_first[SMALLM_FP8BS_MOE_MAX_E];
  __shared__ float s_acc[kDownWaves][ROWS][16];
  __shared__ int s_tok[kDownWaves][ROWS];    // token of gathered row k (this wave's current expert)
  __shared__ int s_hrow[kDownWaves][ROWS];   // its h row t * S + first slot naming the expert
  __shared__ float s_wt[kDownWaves][ROWS];   // its summed top-k weight
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: loop counters, scale loads and addresses derived from it
  // stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = T * S;
  const int NS = gridDim.y, z = blockIdx.y;
  const int lo = (int)((int64_t)z * P / NS), hi = (int)((int64_t)(z + 1) * P / NS);
  for (int i = tid; i < P; i += kDownThreads) {
    s_ids[i] = ids[i];
    s_tw[i] = tw[i];
  }
  for (int i = tid; i < E; i += kDownThreads) s_first[i] = INT_MAX;
  for (int i = lane; i < ROWS * 16; i += 64) s_acc[wave][i >> 4][i & 15] = 0.0f;
  __syncthreads();
  for (int i = tid; i < P; i += kDownThreads) {
    const int e = s_ids[i];
    if (e >= 0 && e < E) atomicMin(&s_first[e], i);
  }
  __syncthreads();

  const int KB2 = I >> 7, nb = blockIdx.x >> 3;
  const int j = lane & 15, chunk = lane >> 4;
  const uint8_t* wtile = w2 + (int64_t)blockIdx.x * KB2 * (FP4 ? 1024 : 2048) + lane * 16;

  // the distinct experts of the range (each at its first pair), in pair order, dealt round-robin
  // to the waves: every wave scans the range 64 pairs at a time and takes the experts whose rank
  // in the list is its index mod kDownWaves, so no wave has more than one expert over another
  int d0 = 0;  // distinct experts before this batch of pairs
  for (int c0 = lo; c0 < hi; c0 += 64) {
    const int pp = c0 + lane;
    const int ec = pp < hi ? s_ids[pp] : -1;
    const bool first = ec >= 0 && ec < E && s_first[ec] == pp;
    const uint64_t m = __ballot(first);
    const int rank =
        d0 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    uint64_t mine = __ballot(first && (rank % kDownWaves) == wave);
    d0 += __popcll(m);
    while (mine) {
      const int e = __builtin_amdgcn_readlane(ec, __builtin_ctzll(mine));
      mine &= mine - 1;
      const float* swp = FP4 ? nullptr : sw2 + ((int64_t)e * (H >> 7) + nb) * KB2;
      const uint8_t* wp = wtile + (int64_t)e * H * I / (FP4 ? 2 : 1);
      // MXFP4: the expert's fragments of this tile and their group-scale bytes
      const __amdgpu_buffer_rsrc_t wr4 = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(w2 + (int64_t)e * H * I / 2 + (int64_t)blockIdx.x * KB2 * 1024), 0, FP4 ? KB2 * 1024 : 0, 0x00020000);
      const __amdgpu_buffer_rsrc_t sr4 = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(s2 + (int64_t)e * H * (I >> 5) + (int64_t)blockIdx.x * KB2 * 64), 0, FP4 ? KB2 * 64 : 0, 0x00020000);
      // the first K block's weights and scale depend only on the expert, so they are loaded before
      // the gather and are in flight during it
      u32x4 pre0 = u32x4{0u, 0u, 0u, 0u}, pre1 = u32x4{0u, 0u, 0u, 0u};
      float pre_s = 0.0f, pre_s1 = 0.0f;
      if constexpr (!FP4) {
        pre0 = load_nt(wp);
        pre1 = load_nt(wp + 1024);
        pre_s = swp[0];
      } else {
        // MXFP4: the second K block's 1 KiB fragment and scale too (zeros past the expert's
        // blocks), through wave-uniform buffer resources
        pre0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr4, (uint32_t)lane * 16u, 0, 2));
        pre1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr4, 1024u + (uint32_t)lane * 16u, 0, 2));
        pre_s = e8m0_f32(__builtin_amdgcn_raw_buffer_load_b8(sr4, (uint32_t)lane, 0, 0));
        pre_s1 = e8m0_f32(__builtin_amdgcn_raw_buffer_load_b8(sr4, 64u + (uint32_t)lane, 0, 0));
      }
      // gather: lane t (< T) is routed to e when some slot of token t names it
      int slot = -1;
      float wsum = 0.0f;
      if (lane < T)
        for (int s = 0; s < S; ++s)
          if (s_ids[lane * S + s] == e) {
            if (slot < 0) slot = s;
            wsum = wsum + s_tw[lane * S + s];
          }
      const uint64_t m = __ballot(slot >= 0);
      if (slot >= 0) {
        const int k = __popcll(m & ((1ull << lane) - 1ull));
        s_tok[wave][k] = lane;
        s_hrow[wave][k] = lane * S + slot;
        s_wt[wave][k] = wsum;
      }
      const int Me = __popcll(m);
      for (int tile = 0; tile * 16 < Me; ++tile) {
        const int k = 16 * tile + j;
        const bool ok = k < Me;
        const uint16_t* hr = h + (int64_t)(ok ? s_hrow[wave][k] : 0) * I + chunk * 32;
        v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        for (int kb = 0; kb < KB2; ++kb) {
          v8bf bv[4];
          float sc;
          if constexpr (FP4) {
            // the group scale is applied by the conversion; the partial needs no block scale
            const bool pre = tile == 0 && kb < 2;
            fp4x32_to_bf16(pre ? (kb == 0 ? pre0 : pre1)
                               : __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                               wr4, (uint32_t)(kb * 1024 + lane * 16), 0, 2)),
                           pre ? (kb == 0 ? pre_s : pre_s1)
                               : e8m0_f32(__builtin_amdgcn_raw_buffer_load_b8(sr4, (uint32_t)(kb * 64 + lane), 0, 0)),
                           bv);
            sc = 1.0f;
          } else {
            const bool first = tile == 0 && kb == 0;
            const u32x4 b0 = first ? pre0 : load_nt(wp + (int64_t)kb * 2048);
            const u32x4 b1 = first ? pre1 : load_nt(wp + (int64_t)kb * 2048 + 1024);
            sc = first ? pre_s : swp[kb];
            e4m3x32_to_bf16(b0, b1, bv);
          }
          const u32x4* ha = (const u32x4*)(hr + kb * 128);
          u32x4 a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = ok ? ha[i] : u32x4{0u, 0u, 0u, 0u};
          v4f pm = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int i = 0; i < 4; ++i) pm = mfma_bf16(a[i], bv[i], pm);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = acc[i] + sc * pm[i];
        }
        // D row r = 4 (lane / 16) + i is gathered row 16 tile + r; its token's LDS row gets the
        // weighted partial (rows are distinct tokens, so no two lanes add to one element)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * tile + 4 * chunk + i;
          if (r < Me) {
            const int t = s_tok[wave][r];
            s_acc[wave][t][j] = s_acc[wave][t][j] + s_wt[wave][r] * acc[i];
          }
        }
      }
    }
  }
  __syncthreads();

  // this workgroup's T x 16 result: the wave slices in wave order (T * 16 <= 768 outputs, at
  // most one per thread)
  static_assert(SMALLM_FP8BS_MOE_MAX_T * 16 <= kDownThreads, "one output per thread");
  const int64_t col0 = (int64_t)blockIdx.x * 16;
  const int o = tid, t = o >> 4, c = o & 15;
  const bool has = o < T * 16;
  float v = 0.0f;
  if (has) {
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) v = v + s_acc[w][t][c];
  }
  if (NS == 1) {
    if (has) y[(int64_t)t * ldy + col0 + c] = bf16_bits(v);
    return;
  }
  if (has) __hip_atomic_store(part + ((int64_t)z * T + t) * H + col0 + c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial is stored
  __syncthreads();                     // and every thread's
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(NS - 1);
  __syncthreads();
  if (!s_last || !has) return;
  float sum = 0.0f;
  for (int zz = 0; zz < NS; ++zz) {
    const float w = zz == z ? v : __hip_atomic_load(part + ((int64_t)zz * T + t) * H + col0 + c, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
    sum = zz == 0 ? w : sum + w;
  }
  y[(int64_t)t * ldy + col0 + c] = bf16_bits(sum);
}

// ---------------------------------------------------------------------------------------------
// weight (un)packing: one thread per 16-byte chunk of the packed layout
// ---------------------------------------------------------------------------------------------
//
// Expert e's [R, K] matrix occupies bytes [e R K, (e + 1) R K) of both layouts.  Packed chunk
// o of an expert: fragment f = o / 128 = tile * (K / 128) + kb, half = (o / 64) % 2, lane =
// o % 64 (column j = lane % 16, K bytes 32 (lane / 16) + 16 half + [0, 16) of block kb).  Tile row
// j is row 16 tile + j, or for w13 (GATE_UP) gate row 8 tile + j (j < 8) / up row I + 8 tile + j - 8.

template <bool PACK, bool GATE_UP>
__global__ __launch_bounds__(256) void moe_pack_kernel(const uint8_t* __restrict__ src,
                                                       uint8_t* __restrict__ dst, int R, int K,
                                                       int64_t chunks) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= chunks) return;
  const int64_t per = (int64_t)R * K / 16;
  const int64_t e = o / per, oe = o % per;
  const int KB = K >> 7;
  const int64_t f = oe >> 7;
  const int within = (int)(oe & 127), half = within >> 6, lane = within & 63;
  const int chunk = lane >> 4, j = lane & 15;
  const int64_t tile = f / KB, kb = f % KB;
  const int64_t n = GATE_UP ? ((j < 8) ? tile * 8 + j : (R >> 1) + tile * 8 + (j - 8)) : tile * 16 + j;
  const int64_t lin = e * R * K + n * K + kb * 128 + chunk * 32 + half * 16;
  const int64_t pk = e * R * K + oe * 16;
  if (PACK)
    *(u32x4*)(dst + pk) = *(const u32x4*)(src + lin);
  else
    *(u32x4*)(dst + lin) = *(const u32x4*)(src + pk);
}

// MXFP4 (un)packing: one thread per 16-byte chunk of fp4x2 bytes, which is one 32-wide scale
// group, so the thread moves the group's scale byte too.  Expert e's matrix [R, K] occupies bytes
// [e R K / 2, (e + 1) R K / 2) of the weight layouts and [e R K / 32, (e + 1) R K / 32) of the
// scale layouts.  Packed chunk o of an expert: fragment f = o / 64 = tile * (K / 128) + kb, lane
// = o % 64 (column j = lane % 16, K elements 32 (lane / 16) + [0, 32) of block kb, row-major bytes
// 64 kb + 16 (lane / 16) + [0, 16)); the packed scale byte o is that group's scale.  Tile rows as
// for e4m3.
template <bool PACK, bool GATE_UP>
__global__ __launch_bounds__(256) void moe_pack_fp4_kernel(const uint8_t* __restrict__ src,
                                                           const uint8_t* __restrict__ src_s,
                                                           uint8_t* __restrict__ dst,
                                                           uint8_t* __restrict__ dst_s, int R,
                                                           int K, int64_t chunks) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= chunks) return;
  const int64_t per = (int64_t)R * K / 32;
  const int64_t e = o / per, oe = o % per;
  const int KB = K >> 7;
  const int64_t f = oe >> 6;
  const int lane = (int)(oe & 63), chunk = lane >> 4, j = lane & 15;
  const int64_t tile = f / KB, kb = f % KB;
  const int64_t n = GATE_UP ? ((j < 8) ? tile * 8 + j : (R >> 1) + tile * 8 + (j - 8)) : tile * 16 + j;
  const int64_t lin = e * R * (K / 2) + n * (K / 2) + kb * 64 + chunk * 16;
  const int64_t lin_s = e * per + n * (K / 32) + kb * 4 + chunk;
  const int64_t pk = e * R * (K / 2) + oe * 16;
  if (PACK) {
    *(u32x4*)(dst + pk) = *(const u32x4*)(src + lin);
    dst_s[o] = src_s[lin_s];
  } else {
    *(u32x4*)(dst + lin) = *(const u32x4*)(src + pk);
    dst_s[lin_s] = src_s[o];
  }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline int launch_status() { return hipGetLastError() == hipSuccess ? SMALLM_OK : SMALLM_ERR_HIP; }

int moe_pack_common(const uint8_t* src, uint8_t* dst, int E, int R, int K, int gate_up, bool pack,
                    void* stream) {
  if (!src || !dst) return SMALLM_ERR_INVALID;
  if (E < 1 || R <= 0 || K <= 0 || (R & 127) || (K & 127)) return SMALLM_ERR_SHAPE;
  if (gate_up != 0 && gate_up != 1) return SMALLM_ERR_INVALID;
  if (!aligned16(src) || !aligned16(dst)) return SMALLM_ERR_ALIGN;
  const int64_t chunks = (int64_t)E * R * K / 16;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  const hipStream_t st = (hipStream_t)stream;
  if (pack) {
    if (gate_up)
      hipLaunchKernelGGL((moe_pack_kernel<true, true>), grid, dim3(256), 0, st, src, dst, R, K, chunks);
    else
      hipLaunchKernelGGL((moe_pack_kernel<true, false>), grid, dim3(256), 0, st, src, dst, R, K, chunks);
  } else {
    if (gate_up)
      hipLaunchKernelGGL((moe_pack_kernel<false, true>), grid, dim3(256), 0, st, src, dst, R, K, chunks);
    else
      hipLaunchKernelGGL((moe_pack_kernel<false, false>), grid, dim3(256), 0, st, src, dst, R, K, chunks);
  }
  return launch_status();
}

int moe_pack_fp4_common(const uint8_t* src, const uint8_t* src_s, uint8_t* dst, uint8_t* dst_s,
                        int E, int R, int K, int gate_up, bool pack, void* stream) {
  if (!src || !src_s || !dst || !dst_s) return SMALLM_ERR_INVALID;
  if (E < 1 || R <= 0 || K <= 0 || (R & 127) || (K & 127)) return SMALLM_ERR_SHAPE;
  if (gate_up != 0 && gate_up != 1) return SMALLM_ERR_INVALID;
  if (!aligned16(src) || !aligned16(dst)) return SMALLM_ERR_ALIGN;
  const int64_t chunks = (int64_t)E * R * K / 32;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  const hipStream_t st = (hipStream_t)stream;
  if (pack) {
    if (gate_up)
      hipLaunchKernelGGL((moe_pack_fp4_kernel<true, true>), grid, dim3(256), 0, st, src, src_s, dst, dst_s, R, K, chunks);
    else
      hipLaunchKernelGGL((moe_pack_fp4_kernel<true, false>), grid, dim3(256), 0, st, src, src_s, dst, dst_s, R, K, chunks);
  } else {
    if (gate_up)
      hipLaunchKernelGGL((moe_pack_fp4_kernel<false, true>), grid, dim3(256), 0, st, src, src_s, dst, dst_s, R, K, chunks);
    else
      hipLaunchKernelGGL((moe_pack_fp4_kernel<false, false>), grid, dim3(256), 0, st, src, src_s, dst, dst_s, R, K, chunks);
  }
  return launch_status();
}

// Workgroups per output tile in phase 2: one up to 128 pairs, else two.  At 64 VGPRs two
// workgroups of 1024 threads share a CU, so on the pages' hidden size (256 column tiles) two splits
// fill the chip in one round and a third adds a second, partly empty one.  Measured at 11 slots,
// hidden 4096: two beat one from 176 pairs on; at 528 pairs (intermediate 128) two took 118 us per
// layer, three 126, four 129 and six 131; at 440 pairs (MXFP4) two took 147 us, three or more 156.
inline int moe_splits(int T, int S) { return T * S <= 128 ? 1 : 2; }

inline size_t moe_h_bytes(int T, int S, int I) { return ((size_t)T * S * I * 2 + 255) & ~(size_t)255; }

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline size_t moe_part_bytes(int T, int S, int H) {
  const int ns = moe_splits(T, S);
  return ns > 1 ? align256((size_t)ns * T * H * 4) : 0;
}
// h, then with NS > 1 the partial sums and one arrival counter per 16-column output tile
inline size_t moe_workspace_bytes(int T, int S, int H, int I) {
  return moe_h_bytes(T, S, I) + (moe_splits(T, S) > 1 ? moe_part_bytes(T, S, H) + align256((size_t)(H / 16) * 4) : 0);
}

template <int MT, bool FP4>
void launch_moe(const uint16_t* x, int64_t ldx, const int32_t* ids, const float* tw, int T, int S,
                const uint8_t* w13, const float* sw13, const uint8_t* s13, const uint8_t* w2,
                const float* sw2, const uint8_t* s2, int E, int H, int I, uint8_t* ws,
                uint16_t* y, int64_t ldy, hipStream_t st) {
  uint16_t* h = (uint16_t*)ws;
  const int ns = moe_splits(T, S);
  float* part = ns > 1 ? (float*)(ws + moe_h_bytes(T, S, I)) : nullptr;
  uint32_t* cnt = ns > 1 ? (uint32_t*)(ws + moe_h_bytes(T, S, I) + moe_part_bytes(T, S, H)) : nullptr;
  const int ncnt = ns > 1 ? H / 16 : 0;
  if (T * S <= kGateItemsFrom) {
    hipLaunchKernelGGL((moe_gate_up_pairs_kernel<FP4>), dim3(T * S, I / 8), dim3(kGateThreads), 0, st,
                       x, ldx, ids, T, S, E, w13, sw13, s13, H, I, h, cnt, ncnt);
  } else {
    const int max_items = (T * S < E ? T * S : E) * (I / 16);  // items of two slices
    const int most = FP4 ? kGateGridFp4 : kGateGrid;
    const int grid = max_items < most ? max_items : most;
    hipLaunchKernelGGL((moe_gate_up_items_kernel<FP4>), dim3(grid),
                       dim3(kGateThreads), 0, st, x, ldx, ids, T, S, E, w13, sw13, s13, H, I, h, cnt, ncnt);
  }
  hipLaunchKernelGGL((moe_down_kernel<MT, FP4>), dim3(H / 16, ns), dim3(kDownThreads), 0, st, h, ids,
                     tw, T, S, E, w2, sw2, s2, H, I, y, ldy, part, cnt);
}

// Shared argument checks (all before any launch) and the M-bucket dispatch of both weight formats.
template <bool FP4>
int moe_call(const uint16_t* x, int64_t ldx, const int32_t* topk_ids, const float* topk_w, int T,
             int S, const uint8_t* w13, const float* sw13, const uint8_t* s13, const uint8_t* w2,
             const float* sw2, const uint8_t* s2, uint32_t layout_id, uint32_t want_layout, int E,
             int H, int I, void* workspace, size_t workspace_bytes, uint16_t* y, int64_t ldy,
             void* stream) {
  if (!x || !topk_ids || !topk_w || !w13 || !w2 || !workspace || !y) return SMALLM_ERR_INVALID;
  int st = smallm_fp8bs_moe_supported(T, S, E, H, I);
  if (st) return st;
  if (ldx < H || ldy < H) return SMALLM_ERR_SHAPE;
  if (workspace_bytes < moe_workspace_bytes(T, S, H, I)) return SMALLM_ERR_SHAPE;
  if (!aligned16(x) || ((ldx * 2) & 15) || !aligned16(w13) || !aligned16(w2) ||
      ((uintptr_t)workspace & 255u) || ((uintptr_t)y & 1u) || ((uintptr_t)topk_ids & 3u) ||
      ((uintptr_t)topk_w & 3u))
    return SMALLM_ERR_ALIGN;
  if (layout_id != want_layout) return SMALLM_ERR_LAYOUT;
  const hipStream_t hs = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  if (T <= 16)
    launch_moe<1, FP4>(x, ldx, topk_ids, topk_w, T, S, w13, sw13, s13, w2, sw2, s2, E, H, I, ws, y, ldy, hs);
  else if (T <= 32)
    launch_moe<2, FP4>(x, ldx, topk_ids, topk_w, T, S, w13, sw13, s13, w2, sw2, s2, E, H, I, ws, y, ldy, hs);
  else
    launch_moe<3, FP4>(x, ldx, topk_ids, topk_w, T, S, w13, sw13, s13, w2, sw2, s2, E, H, I, ws, y, ldy, hs);
  return launch_status();
}

// ---------------------------------------------------------------------------------------------
// allocation-free variant: the workspace in a static device array
// ---------------------------------------------------------------------------------------------

constexpr size_t kMoeScratchBytes = SMALLM_FP8BS_MOE_NOALLOC_MAX_BYTES;  // largest workspace the variant takes
constexpr int kMaxDevices = 64;

// Each GPU the library runs on holds its own copy until the process ends.  In host code this name
// is a host-side stand-in, never a device address: the per-device address comes from
// hipGetSymbolAddress below.
static __device__ __align__(256) uint8_t scratch[kMoeScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` runs on, looked up once per device with
// that device current.
int scratch_for_stream(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SMALLM_ERR_HIP;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return SMALLM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SMALLM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return SMALLM_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return SMALLM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SMALLM_OK;
}

}  // namespace

extern "C" {

uint32_t smallm_fp8bs_moe_layout_id(void) { return kMoeLayoutId; }

int smallm_fp8bs_moe_pack(const uint8_t* w8, uint8_t* w_packed, int E, int R, int K, int gate_up,
                          void* stream) {
  return moe_pack_common(w8, w_packed, E, R, K, gate_up, true, stream);
}

int smallm_fp8bs_moe_unpack(const uint8_t* w_packed, uint8_t* w8, int E, int R, int K, int gate_up,
                            void* stream) {
  return moe_pack_common(w_packed, w8, E, R, K, gate_up, false, stream);
}

int smallm_fp8bs_moe_supported(int T, int S, int E, int H, int I) {
  if (T < 1 || T > SMALLM_FP8BS_MOE_MAX_T || S < 1 || S > SMALLM_FP8BS_MOE_MAX_S || E < 1 ||
      E > SMALLM_FP8BS_MOE_MAX_E || H <= 0 || H > SMALLM_FP8BS_MOE_MAX_H || (H & 127) || I <= 0 ||
      I > SMALLM_FP8BS_MOE_MAX_I || (I & 127))
    return SMALLM_ERR_SHAPE;
  return SMALLM_OK;
}

size_t smallm_fp8bs_moe_workspace_bytes(int T, int S, int H, int I) {
  if (T < 1 || T > SMALLM_FP8BS_MOE_MAX_T || S < 1 || S > SMALLM_FP8BS_MOE_MAX_S || H <= 0 ||
      H > SMALLM_FP8BS_MOE_MAX_H || (H & 127) || I <= 0 || I > SMALLM_FP8BS_MOE_MAX_I || (I & 127))
    return 0;
  return moe_workspace_bytes(T, S, H, I);
}

int smallm_fp8bs_moe_splits(int T, int S) {
  if (T < 1 || T > SMALLM_FP8BS_MOE_MAX_T || S < 1 || S > SMALLM_FP8BS_MOE_MAX_S) return 0;
  return moe_splits(T, S);
}

int smallm_fp8bs_moe(const uint16_t* x, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                     int T, int S, const uint8_t* w13_packed, const float* sw13,
                     const uint8_t* w2_packed, const float* sw2, uint32_t layout_id, int E, int H,
                     int I, void* workspace, size_t workspace_bytes, uint16_t* y, int64_t ldy,
                     void* stream) {
  if (!sw13 || !sw2) return SMALLM_ERR_INVALID;
  if (((uintptr_t)sw13 & 3u) || ((uintptr_t)sw2 & 3u)) return SMALLM_ERR_ALIGN;
  return moe_call<false>(x, ldx, topk_ids, topk_w, T, S, w13_packed, sw13, nullptr, w2_packed, sw2,
                         nullptr, layout_id, kMoeLayoutId, E, H, I, workspace, workspace_bytes, y,
                         ldy, stream);
}

int smallm_fp8bs_moe_noalloc(const uint16_t* x, int64_t ldx, const int32_t* topk_ids,
                             const float* topk_w, int T, int S, const uint8_t* w13_packed,
                             const float* sw13, const uint8_t* w2_packed, const float* sw2,
                             uint32_t layout_id, int E, int H, int I, uint16_t* y, int64_t ldy,
                             void* stream) {
  if (!sw13 || !sw2) return SMALLM_ERR_INVALID;
  if (((uintptr_t)sw13 & 3u) || ((uintptr_t)sw2 & 3u)) return SMALLM_ERR_ALIGN;
  const int st = smallm_fp8bs_moe_supported(T, S, E, H, I);
  if (st) return st;
  const size_t need = moe_workspace_bytes(T, S, H, I);
  if (need > kMoeScratchBytes) return SMALLM_ERR_SHAPE;
  void* ws = nullptr;
  const int sst = scratch_for_stream((hipStream_t)stream, &ws);
  if (sst) return sst;
  return moe_call<false>(x, ldx, topk_ids, topk_w, T, S, w13_packed, sw13, nullptr, w2_packed, sw2,
                         nullptr, layout_id, kMoeLayoutId, E, H, I, ws, kMoeScratchBytes, y, ldy,
                         stream);
}

uint32_t smallm_fp8bs_moe_mxfp4_layout_id(void) { return kMoeFp4LayoutId; }

int smallm_fp8bs_moe_mxfp4_pack(const uint8_t* w4, const uint8_t* s, uint8_t* w_packed,
                                uint8_t* s_packed, int E, int R, int K, int gate_up, void* stream) {
  return moe_pack_fp4_common(w4, s, w_packed, s_packed, E, R, K, gate_up, true, stream);
}

int smallm_fp8bs_moe_mxfp4_unpack(const uint8_t* w_packed, const uint8_t* s_packed, uint8_t* w4,
                                  uint8_t* s, int E, int R, int K, int gate_up, void* stream) {
  return moe_pack_fp4_common(w_packed, s_packed, w4, s, E, R, K, gate_up, false, stream);
}

int smallm_fp8bs_moe_mxfp4(const uint16_t* x, int64_t ldx, const int32_t* topk_ids,
                           const float* topk_w, int T, int S, const uint8_t* w13_packed,
                           const uint8_t* s13_packed, const uint8_t* w2_packed,
                           const uint8_t* s2_packed, uint32_t layout_id, int E, int H, int I,
                           void* workspace, size_t workspace_bytes, uint16_t* y, int64_t ldy,
                           void* stream) {
  if (!s13_packed || !s2_packed) return SMALLM_ERR_INVALID;
  return moe_call<true>(x, ldx, topk_ids, topk_w, T, S, w13_packed, nullptr, s13_packed, w2_packed,
                        nullptr, s2_packed, layout_id, kMoeFp4LayoutId, E, H, I, workspace,
                        workspace_bytes, y, ldy, stream);
}

}  // extern "C"
