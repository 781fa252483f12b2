/*
 * smallm_fp8bs.h -- C ABI of libsmallm_fp8bs.so: small-M FP8 block-scale GEMM with fused
 * activation quantisation for MI355X (gfx950).
 *
 *   Y[m, n] (bf16) = sum_k q(X)[m, k] * sx[m, k/128] * W8[n, k] * sw[n/128, k/128]
 *
 * The operation is the one described on the sglang page "[AMD] Small-M FP8 block-scale GEMM
 * with fused activation quant for gfx950 (Qwen3.5)", section Modifications: bf16 activations
 * are quantised to e4m3 in 1x128 groups (one scale per row and 128-column group), the e4m3
 * weight carries one fp32 scale per 128x128 block (shape [N/128, K/128]), each 128-wide K
 * block's partial sum is multiplied by x_scale * w_scale in fp32, and the result is written
 * as bf16.  The e8m0 entry points follow "[Perf] [AMD] dsv4: optional e8m0 mxscale GEMM for
 * dense 128x128 fp8 linears" (Modifications, commit message): the same GEMM with
 * power-of-two scales stored as one e8m0 byte each (value 2^(byte - 127)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library allocates no
 *    memory, keeps no state between calls, never synchronises the host and enqueues work only
 *    on `stream` (a hipStream_t; NULL is the legacy default stream).  Every call can therefore
 *    be captured into a HIP graph.
 *  - bf16 is passed as uint16_t bit patterns; e4m3 (OCP float8 e4m3fn) and e8m0 as uint8_t.
 *  - Matrices are row-major with an explicit leading dimension in ELEMENTS (ldx, ldq, ldy).
 *  - Activation scales are [M, K/128] row-major (fp32 or e8m0 bytes); weight scales are
 *    [N/128, K/128] row-major, contiguous.
 *  - Shapes: 1 <= M <= SMALLM_FP8BS_MAX_M, N and K positive multiples of 128, else
 *    SMALLM_ERR_SHAPE; the GEMM entries also need 32 activation rows to span less than 2 GiB
 *    ((31 * ld + K) * element bytes < 2^31).  M <= 32 is the design range (decode and verify rows); larger M is
 *    accepted to locate the crossover with tiled GEMMs.
 *  - Alignment: x, q, w8, w_packed and w must be 16-byte aligned and their row pitches
 *    multiples of 16 bytes; y must be 2-byte aligned; else SMALLM_ERR_ALIGN.
 *  - Every error except SMALLM_ERR_HIP is detected before anything is enqueued; on an error
 *    the outputs are left untouched.  SMALLM_ERR_HIP means the launch itself failed.
 *  - Inputs must be finite; the results for NaN or infinite inputs are unspecified.
 *  - Results are deterministic: the same inputs give bit-identical outputs, eagerly or replayed
 *    from a graph (fixed reduction order; the only atomic is the MoE's integer LDS min, whose
 *    result does not depend on order).
 */
#ifndef SMALLM_FP8BS_H
#define SMALLM_FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMALLM_FP8BS_ABI_VERSION 7
#define SMALLM_FP8BS_MAX_M 256
#define SMALLM_FP8BS_RMS_MAX_M (1 << 20) /* rows of one producer call */
#define SMALLM_FP8BS_RMS_MAX_H 16384     /* values per row of one producer call */
#define SMALLM_FP8BS_MOE_MAX_T 48        /* tokens of one MoE call */
#define SMALLM_FP8BS_MOE_MAX_S 16        /* expert slots per token */
#define SMALLM_FP8BS_MOE_MAX_E 4096      /* experts */
#define SMALLM_FP8BS_MOE_MAX_H 16384     /* hidden size */
#define SMALLM_FP8BS_MOE_MAX_I 2048      /* intermediate size per expert */
#define SMALLM_FP8BS_MOE_NOALLOC_MAX_BYTES ((size_t)4 << 20) /* workspace of smallm_fp8bs_moe_noalloc */

typedef enum {
  SMALLM_OK = 0,
  SMALLM_ERR_INVALID = 1, /* a required pointer is NULL, or an invalid scalar argument */
  SMALLM_ERR_SHAPE = 2,   /* M, N, K or a leading dimension out of range */
  SMALLM_ERR_ALIGN = 3,   /* pointer or row pitch misaligned */
  SMALLM_ERR_LAYOUT = 4,  /* packed-weight layout id does not match this library */
  SMALLM_ERR_HIP = 5      /* the HIP launch failed */
} smallm_status;

/* Version of this ABI (SMALLM_FP8BS_ABI_VERSION of the header the library was built with). */
int smallm_fp8bs_abi_version(void);

/* Identifier of the packed layout smallm_fp8bs_pack_weight produces for an [N, K] weight (0 for
 * an invalid shape).  The layout deals the columns to workgroups: each gets NA (0 or 1) group of
 * 16 columns, stored as one 2 KiB fragment per 128-wide K block, and a remainder group of CB
 * (0, 2, 4 or 8) columns whose fragments hold SB consecutive K blocks, chosen from N and K so
 * that the GPU's 256 compute units each stream the same number of weight bytes.  The id is
 * 0x46390000 | NA << 12 | CB << 4 | SB.  The GEMM entry points take the id back and refuse
 * weights packed for another layout (the pages' guard only takes the fused path for a weight
 * marked as preshuffled, section Modifications). */
uint32_t smallm_fp8bs_weight_layout_id(int N, int K);

/* Static description of a status code.  Never NULL. */
const char* smallm_fp8bs_strerror(int status);

/* Host-only shape check for the fused path: SMALLM_OK if (M, N, K, ldx) is accepted by
 * smallm_fp8bs_quant_gemm, else the status it would return.  Enqueues nothing. */
int smallm_fp8bs_supported(int M, int N, int K, int64_t ldx);

/* Host-only description of the launch the GEMM entry points make for (M, N, K), for tools and
 * benchmarks.  plan8 receives, in order: the number of workgroups along N, NA, CB and SB (the
 * packed layout, as in smallm_fp8bs_weight_layout_id), R (K blocks per K range), RC (K blocks
 * per round), NW (K ranges per workgroup; each range has an MFMA wave and a quantising wave, so
 * a workgroup has 128 * NW threads) and MT (16-row M tiles per workgroup; M above 32 runs in
 * 32-row chunks along the grid's second dimension).  Returns SMALLM_OK or the shape error. */
int smallm_fp8bs_launch_plan(int M, int N, int K, int* plan8);

/* Roofline reference, not part of the method: stream `bytes` (1 .. 2^30) of device memory at buf
 * (16-byte aligned) through the GPU with plain non-temporal 16-byte loads, one workgroup per CU,
 * each reading a contiguous share with every load issued before any is consumed -- the launch
 * shape that reads a weight-sized buffer fastest on this part.  Its time over the same bytes (a
 * packed weight) is the achievable floor the GEMM is measured against.  sink: device memory of
 * at least 2048 uint32 that the kernel practically never writes.  Returns a status. */
int smallm_fp8bs_read_floor(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* --------------------------------------------------------------------------------------------
 * Load-time weight preparation (not on the per-token path)
 * ------------------------------------------------------------------------------------------ */

/* Quantise an fp32 weight to e4m3 with one fp32 scale per 128x128 block:
 * sw = RN32(amax / 448) over the block, w8 = e4m3_rne_sat(RN32(w / sw)); an all-zero block gets
 * sw = 0 and signed-zero codes.  w: fp32 [N, ldw]; w8: e4m3 [N, K] (row pitch K);
 * sw: fp32 [N/128, K/128].  The pages start from weights already in this form
 * (weight_scale_inv, section Modifications); this entry produces them from fp32 masters. */
int smallm_fp8bs_quant_weight(const float* w, int64_t ldw, uint8_t* w8, float* sw,
                              int N, int K, void* stream);

/* Same with power-of-two block scales stored as e8m0 bytes: E = log2(amax / 448) rounded to the
 * nearest integer, clamped to [-127, 127] (all-zero block: -127); byte = E + 127;
 * w8 = e4m3_rne(w * 2^-E) saturated to +-448. */
int smallm_fp8bs_quant_weight_e8m0(const float* w, int64_t ldw, uint8_t* w8, uint8_t* sw_e8m0,
                                   int N, int K, void* stream);

/* Permute a row-major e4m3 weight [N, K] (row pitch K) into the library's packed layout
 * (N*K bytes, id smallm_fp8bs_weight_layout_id(N, K)).  With C columns per group and S = 16/C,
 * every (C columns x S K-blocks of 128) piece becomes one contiguous 2 KiB fragment laid out in
 * the lane order of the B operand of the gfx950 16x16x128 fp8 MFMA (B column j = c*S + s is
 * column c of the group in K-block s), so that one wave reads it with two fully coalesced
 * 16-byte loads per lane; the fragments of a column group follow each other along K, and the
 * column groups follow each other along N.  w8 and w_packed must not overlap. */
int smallm_fp8bs_pack_weight(const uint8_t* w8, uint8_t* w_packed, int N, int K, void* stream);

/* Inverse of smallm_fp8bs_pack_weight (used by tests). */
int smallm_fp8bs_unpack_weight(const uint8_t* w_packed, uint8_t* w8, int N, int K, void* stream);

/* --------------------------------------------------------------------------------------------
 * Per-token path
 * ------------------------------------------------------------------------------------------ */

/* Activation quantisation in 1x128 groups with fp32 scales (the pages' standalone quant, the
 * first of the two launches the fused kernel replaces; section Motivation):
 * sx[m, g] = RN32(amax_g / 448); q = e4m3_rne(RN32(x / sx)) with the sign of zero kept; an
 * all-zero group gets sx = 0 and signed-zero codes.  x: bf16 [M, ldx]; q: e4m3 [M, ldq];
 * sx: fp32 [M, K/128]. */
int smallm_fp8bs_quant(const uint16_t* x, int64_t ldx, uint8_t* q, int64_t ldq, float* sx,
                       int M, int K, void* stream);

/* Activation quantisation with ue8m0 group scales ("per-1x128 ue8m0 quant", commit message of
 * the e8m0 page): E = smallest integer with amax_g <= 448 * 2^E, clamped to [-127, 127]
 * (all-zero group: -127); sx byte = E + 127; q = e4m3_rne(x * 2^-E). */
int smallm_fp8bs_quant_e8m0(const uint16_t* x, int64_t ldx, uint8_t* q, int64_t ldq,
                            uint8_t* sx_e8m0, int M, int K, void* stream);

/* GEMM on pre-quantised activations (the second of the two launches): q e4m3 [M, ldq],
 * sx fp32 [M, K/128], packed weight, sw fp32 [N/128, K/128]  ->  y bf16 [M, ldy] (RNE).
 * Beyond M = 32 with K <= 16384 it runs an MFMA-tiled kernel over M and four of the packed
 * layout's column shares per workgroup (32- or 64-row tiles; eight waves on two halves of K whose
 * sums meet once in LDS, first half + second; every weight fragment read once per row tile): the
 * continuation past the small-M range, where the pages'
 * path falls back to a tiled library GEMM ("[AMD] Small-M FP8 block-scale GEMM with fused
 * activation quant for gfx950 (Qwen3.5)", Modifications). */
int smallm_fp8bs_gemm(const uint8_t* q, int64_t ldq, const float* sx, const uint8_t* w_packed,
                      uint32_t layout_id, const float* sw, uint16_t* y, int64_t ldy,
                      int M, int N, int K, void* stream);

/* Same with e8m0 activation and weight scales. */
int smallm_fp8bs_gemm_e8m0(const uint8_t* q, int64_t ldq, const uint8_t* sx_e8m0,
                           const uint8_t* w_packed, uint32_t layout_id, const uint8_t* sw_e8m0,
                           uint16_t* y, int64_t ldy, int M, int N, int K, void* stream);

/* --------------------------------------------------------------------------------------------
 * Producer: RMSNorm with the per-1x128 quantisation of its output
 * ------------------------------------------------------------------------------------------ */

/* The step before the GEMM, emitting the activation bytes and scales once for every consumer
 * ("[Perf] [AMD] dsv4: optional e8m0 mxscale GEMM for dense 128x128 fp8 linears",
 * Modifications and commit message: the fused input_norm / q_norm producers emit the
 * activation scales, so no launch is added).  The page names the fusion, not its arithmetic;
 * this library's reading, per row of H values:
 *   ms = mean of x^2 taken exactly and rounded once to fp32;  v = RN32(ms + eps);
 *   r  = RN32(1 / sqrt(v)), correctly rounded;  y = RNE_bf16(RN32(RN32(x * r) * w));
 *   q, sx = exactly what smallm_fp8bs_quant gives for y (fp32 group scales).
 * x: bf16 [M, ldx]; w: bf16 norm weight [H]; eps: positive finite fp32 (else
 * SMALLM_ERR_INVALID); y: bf16 [M, ldy] or NULL (not written); q: e4m3 [M, ldq] or NULL, in
 * which case sx is not written and the call is a plain RMSNorm (y must then be non-NULL);
 * sx: fp32 [M, H/128].  1 <= M <= SMALLM_FP8BS_RMS_MAX_M; H a multiple of 128 in
 * [128, SMALLM_FP8BS_RMS_MAX_H].  A row whose mean square exceeds the fp32 range is outside the
 * contract (it normalises to zeros).  The mean is exact except when it lies within about 2^-48
 * (relative) of an fp32 rounding boundary, where the per-lane fp64 sums may decide it. */
int smallm_fp8bs_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* w, float eps,
                               uint16_t* y, int64_t ldy, uint8_t* q, int64_t ldq, float* sx,
                               int M, int H, void* stream);

/* Same with ue8m0 group scales (q, sx as smallm_fp8bs_quant_e8m0 gives for y). */
int smallm_fp8bs_rmsnorm_quant_e8m0(const uint16_t* x, int64_t ldx, const uint16_t* w, float eps,
                                    uint16_t* y, int64_t ldy, uint8_t* q, int64_t ldq,
                                    uint8_t* sx_e8m0, int M, int H, void* stream);

/* The fused path (one launch): quantise x exactly as smallm_fp8bs_quant does, then the GEMM,
 * without writing q to memory.  If q_dbg / sx_dbg are non-NULL the kernel also writes the q
 * bytes ([M, K], pitch K) and scales ([M, K/128]) it used, for bit-exact testing. */
int smallm_fp8bs_quant_gemm(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                            uint32_t layout_id, const float* sw, uint16_t* y, int64_t ldy,
                            int M, int N, int K, uint8_t* q_dbg, float* sx_dbg, void* stream);

/* Fused path with e8m0 scales (activation quant as smallm_fp8bs_quant_e8m0). */
int smallm_fp8bs_quant_gemm_e8m0(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                 uint32_t layout_id, const uint8_t* sw_e8m0, uint16_t* y,
                                 int64_t ldy, int M, int N, int K, uint8_t* q_dbg,
                                 uint8_t* sx_dbg_e8m0, void* stream);

/* Bytes of workspace smallm_fp8bs_quant_gemm_ws takes for (M, N, K): 0 when it runs the fused
 * kernel (M <= 32, or a shape the tiled kernel does not take), else M * K rounded up to 256 plus 4 * M * K / 128. */
size_t smallm_fp8bs_quant_gemm_workspace_bytes(int M, int N, int K);

/* smallm_fp8bs_quant_gemm for any M with a caller-owned workspace (device memory, 256-byte
 * aligned, at least smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K) bytes; may be NULL when that
 * is 0).  Up to 32 rows: the fused kernel.  Beyond: the standalone quantisation into the
 * workspace, then the tiled GEMM on it -- the pages hand inputs past the small-M cap to a
 * separate quant + GEMM path ("[AMD] Small-M FP8 block-scale GEMM with fused activation quant for
 * gfx950 (Qwen3.5)", Modifications); the results equal smallm_fp8bs_quant then smallm_fp8bs_gemm
 * bit for bit.  Without a workspace, smallm_fp8bs_quant_gemm above 32 rows runs the fused kernel
 * in 32-row chunks, each reading the whole weight.  Errors: SMALLM_ERR_INVALID (NULL workspace
 * when one is needed), SMALLM_ERR_SHAPE (too small), SMALLM_ERR_ALIGN, and those of
 * smallm_fp8bs_quant_gemm.  The workspace is overwritten; calls sharing one must not overlap. */
int smallm_fp8bs_quant_gemm_ws(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                               uint32_t layout_id, const float* sw, uint16_t* y, int64_t ldy,
                               int M, int N, int K, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Same with e8m0 scales (quantisation as smallm_fp8bs_quant_e8m0, GEMM as smallm_fp8bs_gemm_e8m0). */
int smallm_fp8bs_quant_gemm_e8m0_ws(const uint16_t* x, int64_t ldx, const uint8_t* w_packed,
                                    uint32_t layout_id, const uint8_t* sw_e8m0, uint16_t* y,
                                    int64_t ldy, int M, int N, int K, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------------------------
 * FP8 block-scale small-M fused MoE layer
 * ------------------------------------------------------------------------------------------ */

/* The layer of sglang "[AMD] gfx950 small-batch MoE: expert-count gate for the small sort and
 * FP8 block-scale small-M kernel" (Modifications: e4m3 expert weights with one fp32 scale per
 * 128x128 block, converted to bf16 at scale 1 with the block scale applied to the partial sum)
 * in the two phases of sglang "[AMD] Small-M MXFP4 fused-MoE kernel for gfx950 (Qwen)"
 * (Modifications: bf16 activations; phase 1 gate/up, silu(g) * u written as bf16; phase 2 the
 * down projection with the top-k weights applied in fp32), for T tokens and S slots per token:
 *   (g | u) = x[t] . dequant(w13[e])^T,   h[t, s] = RNE_bf16(silu(g) * u),   e = topk_ids[t, s]
 *   y[t]    = RNE_bf16( sum_s topk_w[t, s] * h[t, s] . dequant(w2[e])^T )
 * with silu(g) = g / (1 + e^-g) in fp32 and fp32 accumulation.  Expert e's w13 is e4m3 [2 I, H]
 * (gate rows [0, I) above up rows [I, 2 I)) with sw13 fp32 [2 I/128, H/128]; its w2 is e4m3
 * [H, I] with sw2 fp32 [H/128, I/128]; experts are stacked: w13 [E, 2 I, H], sw13
 * [E, 2 I/128, H/128], w2 [E, H, I], sw2 [E, H/128, I/128], all contiguous. */

/* Tag of the packed MoE weight layout (both w13 and w2). */
uint32_t smallm_fp8bs_moe_layout_id(void);

/* SMALLM_OK when (T, S, E, H, I) is in range: 1 <= T <= SMALLM_FP8BS_MOE_MAX_T,
 * 1 <= S <= SMALLM_FP8BS_MOE_MAX_S, 1 <= E <= SMALLM_FP8BS_MOE_MAX_E, H and I positive multiples
 * of 128 up to SMALLM_FP8BS_MOE_MAX_H / SMALLM_FP8BS_MOE_MAX_I; else SMALLM_ERR_SHAPE. */
int smallm_fp8bs_moe_supported(int T, int S, int E, int H, int I);

/* Weight preparation at load time (not timed): permute E stacked row-major e4m3 [R, K] expert
 * matrices (R, K multiples of 128) into the packed layout, E * R * K bytes, each expert in its
 * own [e R K, (e + 1) R K) byte range, so experts may be packed in batches.  gate_up = 1 for w13
 * (R = 2 I, K = H: gate and up rows of the same intermediate columns are interleaved in 8-row
 * groups), 0 for w2 (R = H, K = I).  16-byte aligned pointers.  unpack is the inverse. */
int smallm_fp8bs_moe_pack(const uint8_t* w8, uint8_t* w_packed, int E, int R, int K, int gate_up,
                          void* stream);
int smallm_fp8bs_moe_unpack(const uint8_t* w_packed, uint8_t* w8, int E, int R, int K,
                            int gate_up, void* stream);

/* Workspace bytes smallm_fp8bs_moe needs for (T, S, H, I), 0 when out of range: the bf16
 * intermediate h [T * S, I] rounded up to 256 bytes, then, when the down projection is split over
 * NS = smallm_fp8bs_moe_splits(T, S) > 1 workgroups per output tile, fp32 partial sums
 * [NS, T, H] and one uint32 arrival counter per 16 output columns (each rounded up to 256
 * bytes).  Its contents need no initialisation (the first launch clears the counters); calls that
 * share a workspace must not overlap. */
size_t smallm_fp8bs_moe_workspace_bytes(int T, int S, int H, int I);

/* NS for (T, S): 1 when T * S <= 128, else 2; 0 when out of range. */
int smallm_fp8bs_moe_splits(int T, int S);

/* The layer: two launches on `stream` (with NS > 1 the second launch's workgroup that finishes a
 * tile last adds the tile's partial sums, in split order).  x: bf16 [T, ldx]; topk_ids: int32
 * [T, S] expert ids (a pair whose id lies outside [0, E) contributes nothing and its h row is not
 * written; a token may name one expert in several slots, whose weights then add); topk_w: fp32
 * [T, S]; w13_packed / w2_packed from smallm_fp8bs_moe_pack with layout_id =
 * smallm_fp8bs_moe_layout_id() (else SMALLM_ERR_LAYOUT); workspace: caller-owned device memory of
 * at least smallm_fp8bs_moe_workspace_bytes(T, S, H, I) bytes (else SMALLM_ERR_SHAPE), 256-byte
 * aligned; on return its first T * S * I bf16 values hold h[t, s] at row t * S + s (the
 * intermediate between the launches, also the test surface).  y: bf16 [T, ldy].  Each expert in
 * use is read once per phase however many tokens name it.  ids, weights and scales must be
 * 4-byte aligned, x 16-byte aligned with ldx a multiple of 8. */
int smallm_fp8bs_moe(const uint16_t* x, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                     int T, int S, const uint8_t* w13_packed, const float* sw13,
                     const uint8_t* w2_packed, const float* sw2, uint32_t layout_id, int E, int H,
                     int I, void* workspace, size_t workspace_bytes, uint16_t* y, int64_t ldy,
                     void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture that must not
 * call hipMalloc, tight serving loops, harnesses that forbid allocation): smallm_fp8bs_moe with the
 * workspace held in a static device array of SMALLM_FP8BS_MOE_NOALLOC_MAX_BYTES inside the
 * library, one per GPU, kept until the process ends (its device address is looked up once per
 * device, on the first call there).  The call allocates nothing.  Same arguments, formulas, limits
 * and results as smallm_fp8bs_moe without the workspace, plus: SMALLM_ERR_SHAPE (before anything
 * is enqueued) when smallm_fp8bs_moe_workspace_bytes(T, S, H, I) exceeds that size.  Every call on
 * a GPU uses that GPU's one array, so calls that overlap on one GPU (several streams, several host
 * threads) race and must be serialised by the caller; the array needs no initialisation between
 * calls (the layer writes every byte it reads).  h is not returned. */
int smallm_fp8bs_moe_noalloc(const uint16_t* x, int64_t ldx, const int32_t* topk_ids,
                             const float* topk_w, int T, int S, const uint8_t* w13_packed,
                             const float* sw13, const uint8_t* w2_packed, const float* sw2,
                             uint32_t layout_id, int E, int H, int I, uint16_t* y, int64_t ldy,
                             void* stream);

/* --------------------------------------------------------------------------------------------
 * The same MoE layer with MXFP4 expert weights
 * ------------------------------------------------------------------------------------------ */

/* The layer of sglang "[AMD] Small-M MXFP4 fused-MoE kernel for gfx950 (Qwen)" (Motivation and
 * Modifications: fp4x2 expert weights converted to bf16 with their power-of-two scales, bf16
 * activations, the two phases above), with the OCP Microscaling Formats v1.0 encodings: e2m1
 * elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; values 0, 0.5 .. 6) two per
 * byte, the even K element in the low nibble, and one e8m0 scale byte b (value 2^(b - 127)) per
 * 32 consecutive K elements of a row.  Expert e's w13 is fp4x2 [2 I, H/2] with scales [2 I, H/32]
 * (gate rows [0, I) above up rows [I, 2 I)); its w2 is fp4x2 [H, I/2] with scales [H, I/32];
 * experts are stacked and contiguous.  Every scale byte of a group that holds a non-zero code must
 * lie in [2, 252], so every dequantised weight is zero or a normal, finite bf16; other bytes give
 * unspecified results.  Same formulas, shapes, limits and workspace as smallm_fp8bs_moe. */

/* Tag of the packed MXFP4 MoE weight layout (weights and scales of both w13 and w2). */
uint32_t smallm_fp8bs_moe_mxfp4_layout_id(void);

/* Weight preparation at load time (not timed): permute E stacked fp4x2 [R, K/2] expert matrices
 * (R, K multiples of 128) and their e8m0 scales [R, K/32] into the packed layouts, E * R * K / 2
 * and E * R * K / 32 bytes, each expert in its own byte ranges.  gate_up = 1 for w13 (R = 2 I,
 * K = H), 0 for w2 (R = H, K = I).  Weight pointers 16-byte aligned; scale pointers any alignment.
 * unpack is the inverse. */
int smallm_fp8bs_moe_mxfp4_pack(const uint8_t* w4, const uint8_t* s, uint8_t* w_packed,
                                uint8_t* s_packed, int E, int R, int K, int gate_up, void* stream);
int smallm_fp8bs_moe_mxfp4_unpack(const uint8_t* w_packed, const uint8_t* s_packed, uint8_t* w4,
                                  uint8_t* s, int E, int R, int K, int gate_up, void* stream);

/* The layer, as smallm_fp8bs_moe but with packed MXFP4 weights and their packed scales, and
 * layout_id = smallm_fp8bs_moe_mxfp4_layout_id() (else SMALLM_ERR_LAYOUT).  Each expert in use
 * is read once per phase: (3 H I) / 2 weight bytes and (3 H I) / 32 scale bytes. */
int smallm_fp8bs_moe_mxfp4(const uint16_t* x, int64_t ldx, const int32_t* topk_ids,
                           const float* topk_w, int T, int S, const uint8_t* w13_packed,
                           const uint8_t* s13_packed, const uint8_t* w2_packed,
                           const uint8_t* s2_packed, uint32_t layout_id, int E, int H, int I,
                           void* workspace, size_t workspace_bytes, uint16_t* y, int64_t ldy,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMALLM_FP8BS_H */
