"""CPU oracle for the small-M FP8 block-scale GEMM with fused activation quantisation.

TEST INFRASTRUCTURE ONLY.  This package is the checker that the GPU library is held to: only
the test suite, the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64 where the pages fix no precision); this
module builds it with gcc and wraps it with ctypes over numpy arrays.  Every function cites the
passage of the pages it follows in the C source:

* sglang "[AMD] Small-M FP8 block-scale GEMM with fused activation quant for gfx950 (Qwen3.5)",
  section Modifications (1x128 activation groups, 128x128 fp32 weight scales, x_scale * w_scale
  applied per 128-wide K block, bf16 output);
* sglang "[Perf] [AMD] dsv4: optional e8m0 mxscale GEMM for dense 128x128 fp8 linears",
  Modifications and commit message (power-of-two scales stored as e8m0 bytes).

The FP8 block-scale MoE layer (dequantised fp64 reference in numpy, at the end of this module)
follows sglang "[AMD] gfx950 small-batch MoE: expert-count gate for the small sort and FP8
block-scale small-M kernel", Modifications, and the phase structure of sglang "[AMD] Small-M
MXFP4 fused-MoE kernel for gfx950 (Qwen)", Modifications.  The same layer with MXFP4 expert
weights (e2m1 elements, one e8m0 scale per 32 K elements, OCP Microscaling Formats v1.0) follows
that page's Motivation and Modifications.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
             "-std=c11", "-Wall"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        I = ctypes.c_int
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_e8m0_ceil_exponent.restype = I
        L.oracle_e8m0_ceil_exponent.argtypes = [ctypes.c_double]
        L.oracle_e8m0_round_exponent.restype = I
        L.oracle_e8m0_round_exponent.argtypes = [ctypes.c_double]
        L.oracle_quant_act_fp32.restype = None
        L.oracle_quant_act_fp32.argtypes = [P, i64, I, I, P, i64, P]
        L.oracle_quant_act_e8m0.restype = None
        L.oracle_quant_act_e8m0.argtypes = [P, i64, I, I, P, i64, P]
        L.oracle_quant_weight_fp32.restype = None
        L.oracle_quant_weight_fp32.argtypes = [P, i64, I, I, P, P]
        L.oracle_quant_weight_e8m0.restype = None
        L.oracle_quant_weight_e8m0.argtypes = [P, i64, I, I, P, P]
        L.oracle_gemm_fp32.restype = None
        L.oracle_gemm_fp32.argtypes = [P, i64, P, P, P, I, I, I, I, I, P, I]
        L.oracle_gemm_e8m0.restype = None
        L.oracle_gemm_e8m0.argtypes = [P, i64, P, P, P, I, I, I, I, I, P, I]
        L.oracle_round_bf16.restype = None
        L.oracle_round_bf16.argtypes = [P, i64, P]
        L.oracle_quant_gemm.restype = None
        L.oracle_quant_gemm.argtypes = [P, i64, P, P, I, I, I, I, I, I, P, P, P, P, I]
        L.oracle_max_threads.restype = I
        L.oracle_max_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------------------------------------
# scalar codecs
# ---------------------------------------------------------------------------------------------

def e4m3_decode(b: int) -> float:
    return lib().oracle_e4m3_decode(int(b))


def e4m3_decode_array(codes: np.ndarray) -> np.ndarray:
    table = np.array([e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(f: float) -> int:
    return int(lib().oracle_e4m3_encode(float(f)))


def bf16_from_double(v: float) -> int:
    return int(lib().oracle_bf16_from_double(float(v)))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e8m0_ceil_exponent(amax: float) -> int:
    return int(lib().oracle_e8m0_ceil_exponent(float(amax)))


def e8m0_round_exponent(amax: float) -> int:
    return int(lib().oracle_e8m0_round_exponent(float(amax)))


# ---------------------------------------------------------------------------------------------
# array entry points
# ---------------------------------------------------------------------------------------------

def quant_act(x_bits: np.ndarray, e8m0: bool = False):
    """x_bits: uint16 [M, K] (bf16).  Returns (q uint8 [M, K], sx float32 or uint8 [M, K/128])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    assert K % 128 == 0
    q = np.empty((M, K), dtype=np.uint8)
    if e8m0:
        sx = np.empty((M, K // 128), dtype=np.uint8)
        lib().oracle_quant_act_e8m0(_ptr(x_bits), K, M, K, _ptr(q), K, _ptr(sx))
    else:
        sx = np.empty((M, K // 128), dtype=np.float32)
        lib().oracle_quant_act_fp32(_ptr(x_bits), K, M, K, _ptr(q), K, _ptr(sx))
    return q, sx


def quant_weight(w: np.ndarray, e8m0: bool = False):
    """w: float32 [N, K].  Returns (w8 uint8 [N, K], sw float32 or uint8 [N/128, K/128])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    w8 = np.empty((N, K), dtype=np.uint8)
    if e8m0:
        sw = np.empty((N // 128, K // 128), dtype=np.uint8)
        lib().oracle_quant_weight_e8m0(_ptr(w), K, N, K, _ptr(w8), _ptr(sw))
    else:
        sw = np.empty((N // 128, K // 128), dtype=np.float32)
        lib().oracle_quant_weight_fp32(_ptr(w), K, N, K, _ptr(w8), _ptr(sw))
    return w8, sw


def gemm(q: np.ndarray, sx: np.ndarray, w8: np.ndarray, sw: np.ndarray, e8m0: bool = False,
         n0: int = 0, n1: int | None = None, threads: int = 0) -> np.ndarray:
    """fp64 reference [M, N] (only columns [n0, n1) are filled; the rest are zero)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    w8 = np.ascontiguousarray(w8, dtype=np.uint8)
    M, K = q.shape
    N = w8.shape[0]
    n1 = N if n1 is None else n1
    if not (0 <= n0 <= n1 <= N) or w8.shape[1] != K or sx.shape != (M, K // 128) or sw.shape != (N // 128, K // 128):
        raise ValueError("gemm: column window or operand shapes out of range")
    ref = np.zeros((M, N), dtype=np.float64)
    if e8m0:
        sx = np.ascontiguousarray(sx, dtype=np.uint8)
        sw = np.ascontiguousarray(sw, dtype=np.uint8)
        lib().oracle_gemm_e8m0(_ptr(q), K, _ptr(sx), _ptr(w8), _ptr(sw), M, N, K, n0, n1,
                               _ptr(ref), threads)
    else:
        sx = np.ascontiguousarray(sx, dtype=np.float32)
        sw = np.ascontiguousarray(sw, dtype=np.float32)
        lib().oracle_gemm_fp32(_ptr(q), K, _ptr(sx), _ptr(w8), _ptr(sw), M, N, K, n0, n1,
                               _ptr(ref), threads)
    return ref


def round_bf16(ref: np.ndarray) -> np.ndarray:
    ref = np.ascontiguousarray(ref, dtype=np.float64)
    y = np.empty(ref.shape, dtype=np.uint16)
    lib().oracle_round_bf16(_ptr(ref), ref.size, _ptr(y))
    return y


def quant_gemm(x_bits: np.ndarray, w8: np.ndarray, sw: np.ndarray, e8m0: bool = False,
               n0: int = 0, n1: int | None = None, threads: int = 0):
    """Whole path: returns (y bf16 bits [M, N], ref fp64 [M, N], q, sx)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w8 = np.ascontiguousarray(w8, dtype=np.uint8)
    M, K = x_bits.shape
    N = w8.shape[0]
    n1 = N if n1 is None else n1
    if not (0 <= n0 <= n1 <= N) or w8.shape[1] != K or np.shape(sw) != (N // 128, K // 128):
        raise ValueError("quant_gemm: column window or operand shapes out of range")
    q = np.empty((M, K), dtype=np.uint8)
    sx = np.empty((M, K // 128), dtype=np.uint8 if e8m0 else np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.uint8 if e8m0 else np.float32)
    ref = np.zeros((M, N), dtype=np.float64)
    y = np.zeros((M, N), dtype=np.uint16)
    lib().oracle_quant_gemm(_ptr(x_bits), K, _ptr(w8), _ptr(sw), M, N, K, n0, n1, int(e8m0),
                            _ptr(q), _ptr(sx), _ptr(ref), _ptr(y), threads)
    return y, ref, q, sx


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# ---------------------------------------------------------------------------------------------
# RMSNorm producer with per-1x128 quantisation (the step before the GEMM)
# ---------------------------------------------------------------------------------------------
# sglang "[Perf] [AMD] dsv4: optional e8m0 mxscale GEMM for dense 128x128 fp8 linears",
# Modifications and commit message: the fused input_norm / q_norm producers emit the activation
# quantisation (ue8m0 scales when every consumer uses the e8m0 GEMM) so that no launch is added.
# The pages name the fusion but not its arithmetic; the reading taken here, per row of H values:
#   ms = mean of x^2, taken exactly and rounded once to fp32;
#   v  = RN32(ms + eps);  r = RN32(1 / sqrt(v)), correctly rounded;
#   y  = RNE_bf16(RN32(RN32(x * r) * w))   (w: the bf16 norm weight);
#   q, sx = the 1x128 activation quantisation of y (quant_act), fp32 or ue8m0 scales.
# So the quantised bytes are those the separate RMSNorm then quant launches would give.

def _rn32_ratio(p: int, d: int) -> float:
    """IEEE binary32 round-to-nearest-even of the positive rational p / d (inf above the range)."""
    assert p >= 0 and d > 0
    if p == 0:
        return 0.0
    e = p.bit_length() - d.bit_length()          # p / d in [2^(e-1), 2^(e+1))
    if (p << max(0, -e)) < (d << max(0, e)):     # p / d < 2^e
        e -= 1
    e = max(e, -126)                              # subnormals share the 2^-149 quantum
    sh = 23 - e                                   # quantum 2^(e - 23)
    num, den = (p << sh, d) if sh >= 0 else (p, d << -sh)
    fl, rem = divmod(num, den)
    if 2 * rem > den or (2 * rem == den and fl & 1):
        fl += 1
    if fl.bit_length() + (e - 23) > 128:          # fl * 2^(e-23) >= 2^128
        return math.inf
    return math.ldexp(fl, e - 23)


def _bf16_parts(bits: np.ndarray):
    """bf16 patterns -> (integer significand, power of two): |value| = sig * 2^p2."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    ef = (bits >> 7) & 0xFF
    fr = bits & 0x7F
    sig = np.where(ef == 0, fr, fr | 0x80)
    p2 = np.where(ef == 0, -133, ef - 134)
    return sig, p2


def mean_square_f32(x_row_bits: np.ndarray) -> float:
    """RN32(sum x^2 / H) for one bf16 row, the sum taken exactly (integers scaled by 2^-266)."""
    sig, p2 = _bf16_parts(x_row_bits)
    total = 0
    for s, e in zip(sig.tolist(), p2.tolist()):
        if s:
            total += (s * s) << (2 * e + 266)
    return _rn32_ratio(total, len(sig) << 266)


def rsqrt_f32(v: float) -> float:
    """RN32(1 / sqrt(v)) for a positive finite fp32 v, correctly rounded: a candidate from the
    double-precision formula, then moved until 1/sqrt(v) lies between the midpoints with its
    fp32 neighbours (compared exactly as rationals: m^2 v against 1)."""
    assert v > 0 and math.isfinite(v)
    V = Fraction(v)
    r = np.float32(1.0 / math.sqrt(v))
    for _ in range(8):
        up = np.nextafter(r, np.float32(np.inf))
        dn = np.nextafter(r, np.float32(0))
        mu = (Fraction(float(r)) + Fraction(float(up))) / 2
        ml = (Fraction(float(r)) + Fraction(float(dn))) / 2
        if mu * mu * V < 1:
            r = up
        elif ml * ml * V > 1:
            r = dn
        else:
            assert mu * mu * V != 1 and ml * ml * V != 1   # no ties: 1/sqrt(v) is never a midpoint
            return float(r)
    raise AssertionError("rsqrt_f32 did not settle")


def rmsnorm(x_bits: np.ndarray, w_bits: np.ndarray, eps: float):
    """x_bits bf16 [M, H], w_bits bf16 [H], eps > 0 (fp32).  Returns (y bf16 bits [M, H],
    r float32 [M]) with the reading stated above."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, H = x_bits.shape
    eps32 = np.float32(eps)
    assert eps32 > 0
    r = np.empty(M, dtype=np.float32)
    for m in range(M):
        ms = np.float32(mean_square_f32(x_bits[m]))
        v = np.float32(ms + eps32)                 # one fp32 addition
        r[m] = np.float32(rsqrt_f32(float(v)))
    xf = bf16_to_f32(x_bits)
    wf = bf16_to_f32(np.asarray(w_bits, dtype=np.uint16))
    t = (xf * r[:, None]).astype(np.float32)       # RN32(x * r)
    yf = (t * wf[None, :]).astype(np.float32)       # RN32(t * w)
    y = round_bf16(yf.astype(np.float64))
    return y, r


def rmsnorm_quant(x_bits: np.ndarray, w_bits: np.ndarray, eps: float, e8m0: bool = False):
    """Producer: (y bf16 bits [M, H], q e4m3 [M, H], sx fp32 or e8m0 [M, H/128])."""
    y, _ = rmsnorm(x_bits, w_bits, eps)
    q, sx = quant_act(y, e8m0=e8m0)
    return y, q, sx


# ---------------------------------------------------------------------------------------------
# FP8 block-scale small-M fused MoE
# ---------------------------------------------------------------------------------------------
#
# sglang "[AMD] gfx950 small-batch MoE: expert-count gate for the small sort and FP8 block-scale
# small-M kernel", section Modifications: e4m3 expert weights with one fp32 scale per 128x128
# block, converted to bf16 at scale 1 with each block's scale applied to the partial sum, and a
# test against a dequantised reference.  The phase structure comes from sglang "[AMD] Small-M
# MXFP4 fused-MoE kernel for gfx950 (Qwen)", section Modifications: bf16 activations, phase 1
# gate/up with silu(g) * u stored as bf16, phase 2 the down projection with the top-k weights
# applied in fp32.  Readings where the pages are silent: w13 holds the gate rows [0, I) above the
# up rows [I, 2 I); a (token, slot) pair whose expert id lies outside [0, E) contributes nothing.
#
# Since a block scale multiplies every product of its block, applying it to the block's partial
# sum equals multiplying by the dequantised weight; the reference below is that dequantised
# product, in fp64.

_E4M3_TABLE = None


def _e4m3_table() -> np.ndarray:
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = np.array([e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return _E4M3_TABLE


def dequant_weight(w8: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """fp64 [N, K] with entry dec(w8[n, k]) * sw[n // 128, k // 128] (exact: a 4-bit significand
    times an fp32 scale fits in a double)."""
    w8 = np.asarray(w8, dtype=np.uint8)
    N, K = w8.shape
    s = np.asarray(sw, dtype=np.float32).astype(np.float64)
    assert s.shape == (N // 128, K // 128)
    return _e4m3_table()[w8] * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)


def silu(g: np.ndarray) -> np.ndarray:
    """g * sigmoid(g) = g / (1 + e^-g), in fp64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def moe_gate_up(x: np.ndarray, W13: np.ndarray):
    """Phase-1 GEMM of one expert for fp64 activations x [..., H] and its dequantised w13
    [2 I, H]: returns (g, u), each [..., I], from the gate rows [0, I) and the up rows [I, 2 I)."""
    I = W13.shape[0] // 2
    gu = np.asarray(x, dtype=np.float64) @ W13.T
    return gu[..., :I], gu[..., I:]


def _moe_layer(x_bits: np.ndarray, ids: np.ndarray, tw: np.ndarray, E: int, I: int, W13_of, W2_of):
    """The layer for dequantised expert weights: W13_of(e) fp64 [2 I, H], W2_of(e) fp64 [H, I]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = np.asarray(ids)
    tw = np.asarray(tw, dtype=np.float32)
    T, H = x_bits.shape
    S = ids.shape[1]
    x = bf16_to_f32(x_bits).astype(np.float64)
    h = np.zeros((T, S, I), dtype=np.uint16)
    # every pair's term tw * (w2 @ h), computed expert by expert so that each expert is
    # dequantised once, then summed over the slots in slot order
    term = np.zeros((T, S, H), dtype=np.float64)
    for e in sorted(set(int(v) for v in ids.ravel() if 0 <= v < E)):
        pairs = [(t, s) for t in range(T) for s in range(S) if int(ids[t, s]) == e]
        W13 = W13_of(e)
        W2 = W2_of(e)
        for t, s in pairs:
            g, u = moe_gate_up(x[t], W13)
            h[t, s] = round_bf16(silu(g) * u)
            hv = bf16_to_f32(h[t, s]).astype(np.float64)
            term[t, s] = float(tw[t, s]) * (W2 @ hv)
    ref = np.zeros((T, H), dtype=np.float64)
    for s in range(S):
        ref += term[:, s]
    return h, ref


def moe(x_bits: np.ndarray, ids: np.ndarray, tw: np.ndarray, w13, sw13, w2, sw2,
        E: int | None = None):
    """Whole MoE layer.

    x_bits bf16 bits [T, H]; ids int [T, S]; tw float32 [T, S]; for every expert id e in use,
    w13[e] e4m3 [2 I, H] with sw13[e] fp32 [2 I/128, H/128] and w2[e] e4m3 [H, I] with sw2[e] fp32
    [H/128, I/128] (w13/w2 may be arrays or mappings holding only the experts in use; E
    defaults to len(sw13)).  Returns (h bf16 bits [T, S, I], ref fp64 [T, H]):
      h[t, s] = RNE_bf16(silu(g) * u), g and u the expert's gate and up outputs for token t;
      ref[t]  = sum over slots s of tw[t, s] * (dequantised w2[e]) @ h[t, s].
    Pairs with an id outside [0, E) leave h at zero and add nothing.  The bf16 output is
    round_bf16(ref)."""
    E = len(sw13) if E is None else E
    some_w2 = next(iter(w2.values())) if isinstance(w2, dict) else w2[0]
    I = np.asarray(some_w2).shape[1]
    return _moe_layer(x_bits, ids, tw, E, I, lambda e: dequant_weight(w13[e], sw13[e]),
                      lambda e: dequant_weight(w2[e], sw2[e]))


# ---------------------------------------------------------------------------------------------
# MXFP4 expert weights for the same MoE layer
# ---------------------------------------------------------------------------------------------
#
# sglang "[AMD] Small-M MXFP4 fused-MoE kernel for gfx950 (Qwen)", sections Motivation and
# Modifications: the expert weights are MXFP4 (fp4x2 bytes, e2m1 elements with a power-of-two
# e8m0 scale per 32 consecutive K elements of a row, the OCP Microscaling format), converted to
# bf16 with the scale applied by the conversion, against bf16 activations; the test compares with
# a dequantised reference.  The element and scale codecs follow the OCP Microscaling Formats (MX)
# specification v1.0: e2m1 has one sign bit, two exponent bits with bias 1 and one mantissa bit
# (exponent field 0 is subnormal: 0.5 * m), no infinities or NaN; the e8m0 scale byte b is
# 2^(b - 127), 0xFF being NaN.  Reading where the pages are silent: in an fp4x2 byte the low
# nibble holds the even K element and the high nibble the odd one; the scales of expert matrix
# [R, K] are the row-major byte array [R, K/32].

def e2m1_decode(c: int) -> float:
    """Value of the 4-bit e2m1 code c (bit 3 sign, bits 2..1 exponent, bit 0 mantissa)."""
    c = int(c) & 15
    sign = -1.0 if c & 8 else 1.0
    e, m = (c >> 1) & 3, c & 1
    mag = 0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return sign * mag


def e8m0_decode(b: int) -> float:
    """Value of the e8m0 scale byte b: 2^(b - 127); NaN for 0xFF."""
    b = int(b) & 255
    return math.nan if b == 255 else math.ldexp(1.0, b - 127)


def dequant_mxfp4(w4: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp64 [R, K] from fp4x2 bytes w4 [R, K/2] and e8m0 scales s [R, K/32]: element (r, k) is
    e2m1(nibble k % 2 of byte k // 2) * 2^(s[r, k // 32] - 127), exact in a double."""
    w4 = np.asarray(w4, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    R, K2 = w4.shape
    K = 2 * K2
    assert s.shape == (R, K // 32)
    table = np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)
    codes = np.empty((R, K), dtype=np.uint8)
    codes[:, 0::2] = w4 & 15
    codes[:, 1::2] = w4 >> 4
    scale = np.array([e8m0_decode(b) for b in range(256)], dtype=np.float64)[s]
    return table[codes] * np.repeat(scale, 32, axis=1)


def moe_mxfp4(x_bits: np.ndarray, ids: np.ndarray, tw: np.ndarray, w13, s13, w2, s2,
              E: int | None = None):
    """The MoE layer of moe() with MXFP4 expert weights: w13[e] fp4x2 [2 I, H/2] with e8m0
    s13[e] [2 I, H/32]; w2[e] fp4x2 [H, I/2] with e8m0 s2[e] [H, I/32].  Returns (h, ref) as
    moe() does."""
    E = len(s13) if E is None else E
    some_w2 = next(iter(w2.values())) if isinstance(w2, dict) else w2[0]
    I = 2 * np.asarray(some_w2).shape[1]
    return _moe_layer(x_bits, ids, tw, E, I, lambda e: dequant_mxfp4(w13[e], s13[e]),
                      lambda e: dequant_mxfp4(w2[e], s2[e]))
