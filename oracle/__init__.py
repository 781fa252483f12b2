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
"""
from __future__ import annotations

import ctypes
import os
import subprocess

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
