"""Python binding of libsmallm_fp8bs.so: small-M FP8 block-scale GEMM with fused activation
quantisation for MI355X (gfx950).

The functions below carry the names of the C entry points declared in include/smallm_fp8bs.h
and only marshal arguments: torch provides device memory and the current HIP stream, every step
of the computation runs in the library's HIP kernels.  There is no CPU or PyTorch fallback: if
the shared library is missing or a call fails, an exception is raised.

The library must bind to the HIP runtime torch already loaded (a second libamdhip64 in the
process makes launches on torch's streams fail; sglang "[AMD] Small-M MXFP4 fused-MoE kernel for
gfx950 (Qwen)", loader fix in the commit history).  torch is therefore imported and initialised
before the library is opened, and the loader checks that only one libamdhip64 is mapped.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmallm_fp8bs.so")

SMALLM_OK = 0
SMALLM_ERR_INVALID = 1
SMALLM_ERR_SHAPE = 2
SMALLM_ERR_ALIGN = 3
SMALLM_ERR_LAYOUT = 4
SMALLM_ERR_HIP = 5
MAX_M = 256

EXPORTS = (
    "smallm_fp8bs_abi_version",
    "smallm_fp8bs_weight_layout_id",
    "smallm_fp8bs_strerror",
    "smallm_fp8bs_supported",
    "smallm_fp8bs_launch_plan",
    "smallm_fp8bs_read_floor",
    "smallm_fp8bs_quant_weight",
    "smallm_fp8bs_quant_weight_e8m0",
    "smallm_fp8bs_pack_weight",
    "smallm_fp8bs_unpack_weight",
    "smallm_fp8bs_quant",
    "smallm_fp8bs_quant_e8m0",
    "smallm_fp8bs_gemm",
    "smallm_fp8bs_gemm_e8m0",
    "smallm_fp8bs_quant_gemm",
    "smallm_fp8bs_quant_gemm_e8m0",
    "smallm_fp8bs_quant_gemm_workspace_bytes",
    "smallm_fp8bs_quant_gemm_ws",
    "smallm_fp8bs_quant_gemm_e8m0_ws",
    "smallm_fp8bs_rmsnorm_quant",
    "smallm_fp8bs_rmsnorm_quant_e8m0",
    "smallm_fp8bs_moe_layout_id",
    "smallm_fp8bs_moe_supported",
    "smallm_fp8bs_moe_pack",
    "smallm_fp8bs_moe_unpack",
    "smallm_fp8bs_moe_workspace_bytes",
    "smallm_fp8bs_moe_splits",
    "smallm_fp8bs_moe",
    "smallm_fp8bs_moe_noalloc",
    "smallm_fp8bs_moe_mxfp4_layout_id",
    "smallm_fp8bs_moe_mxfp4_pack",
    "smallm_fp8bs_moe_mxfp4_unpack",
    "smallm_fp8bs_moe_mxfp4",
)


class SmallmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({strerror(status)})")


_lib = None


def _hip_runtimes_mapped() -> set:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                p = line.split()[-1]
                if "libamdhip64" in p:
                    paths.add(os.path.realpath(p))
    except OSError:
        pass
    return paths


def lib():
    """Open libsmallm_fp8bs.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with precision_gemm_x128_amd.build.build() "
                          "(there is no fallback path)")
    if torch.cuda.is_available():
        torch.cuda.init()
    L = ctypes.CDLL(LIB_PATH)
    rts = _hip_runtimes_mapped()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process: {sorted(rts)}")
    P, I, I64, U32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32
    sig = {
        "smallm_fp8bs_abi_version": (I, []),
        "smallm_fp8bs_weight_layout_id": (U32, [I, I]),
        "smallm_fp8bs_strerror": (ctypes.c_char_p, [I]),
        "smallm_fp8bs_supported": (I, [I, I, I, I64]),
        "smallm_fp8bs_launch_plan": (I, [I, I, I, P]),
        "smallm_fp8bs_read_floor": (I, [P, I64, P, P]),
        "smallm_fp8bs_quant_weight": (I, [P, I64, P, P, I, I, P]),
        "smallm_fp8bs_quant_weight_e8m0": (I, [P, I64, P, P, I, I, P]),
        "smallm_fp8bs_pack_weight": (I, [P, P, I, I, P]),
        "smallm_fp8bs_unpack_weight": (I, [P, P, I, I, P]),
        "smallm_fp8bs_quant": (I, [P, I64, P, I64, P, I, I, P]),
        "smallm_fp8bs_quant_e8m0": (I, [P, I64, P, I64, P, I, I, P]),
        "smallm_fp8bs_gemm": (I, [P, I64, P, P, U32, P, P, I64, I, I, I, P]),
        "smallm_fp8bs_gemm_e8m0": (I, [P, I64, P, P, U32, P, P, I64, I, I, I, P]),
        "smallm_fp8bs_quant_gemm": (I, [P, I64, P, U32, P, P, I64, I, I, I, P, P, P]),
        "smallm_fp8bs_quant_gemm_e8m0": (I, [P, I64, P, U32, P, P, I64, I, I, I, P, P, P]),
        "smallm_fp8bs_quant_gemm_workspace_bytes": (ctypes.c_size_t, [I, I, I]),
        "smallm_fp8bs_quant_gemm_ws": (I, [P, I64, P, U32, P, P, I64, I, I, I, P, ctypes.c_size_t, P]),
        "smallm_fp8bs_quant_gemm_e8m0_ws": (I, [P, I64, P, U32, P, P, I64, I, I, I, P, ctypes.c_size_t, P]),
        "smallm_fp8bs_rmsnorm_quant": (I, [P, I64, P, ctypes.c_float, P, I64, P, I64, P, I, I, P]),
        "smallm_fp8bs_rmsnorm_quant_e8m0": (I, [P, I64, P, ctypes.c_float, P, I64, P, I64, P, I, I, P]),
        "smallm_fp8bs_moe_layout_id": (U32, []),
        "smallm_fp8bs_moe_supported": (I, [I, I, I, I, I]),
        "smallm_fp8bs_moe_pack": (I, [P, P, I, I, I, I, P]),
        "smallm_fp8bs_moe_unpack": (I, [P, P, I, I, I, I, P]),
        "smallm_fp8bs_moe_workspace_bytes": (ctypes.c_size_t, [I, I, I, I]),
        "smallm_fp8bs_moe_splits": (I, [I, I]),
        "smallm_fp8bs_moe": (I, [P, I64, P, P, I, I, P, P, P, P, U32, I, I, I, P, ctypes.c_size_t, P, I64, P]),
        "smallm_fp8bs_moe_noalloc": (I, [P, I64, P, P, I, I, P, P, P, P, U32, I, I, I, P, I64, P]),
        "smallm_fp8bs_moe_mxfp4_layout_id": (U32, []),
        "smallm_fp8bs_moe_mxfp4_pack": (I, [P, P, P, P, I, I, I, I, P]),
        "smallm_fp8bs_moe_mxfp4_unpack": (I, [P, P, P, P, I, I, I, I, P]),
        "smallm_fp8bs_moe_mxfp4": (I, [P, I64, P, P, I, I, P, P, P, P, U32, I, I, I, P, ctypes.c_size_t, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


# ---------------------------------------------------------------------------------------------
# host-only queries
# ---------------------------------------------------------------------------------------------

def smallm_fp8bs_abi_version() -> int:
    return int(lib().smallm_fp8bs_abi_version())


def smallm_fp8bs_weight_layout_id(N: int, K: int) -> int:
    """Id of the packed layout smallm_fp8bs_pack_weight produces for an [N, K] weight."""
    return int(lib().smallm_fp8bs_weight_layout_id(N, K))


def weight_layout(N: int, K: int) -> dict:
    """The packed layout for an [N, K] weight: NA 16-column groups and a CB-column remainder group
    per workgroup, SB K blocks per remainder fragment (decoded from the layout id)."""
    lid = smallm_fp8bs_weight_layout_id(N, K)
    if lid == 0:
        raise ValueError(f"no packed layout for N={N} K={K}")
    return {"NA": (lid >> 12) & 0xF, "CB": (lid >> 4) & 0xFF, "SB": lid & 0xF}


def strerror(status: int) -> str:
    return lib().smallm_fp8bs_strerror(int(status)).decode()


smallm_fp8bs_strerror = strerror


def smallm_fp8bs_supported(M: int, N: int, K: int, ldx: int) -> int:
    return int(lib().smallm_fp8bs_supported(M, N, K, ldx))


PLAN_FIELDS = ("nwg", "NA", "CB", "SB", "R", "RC", "NW", "MT")


def smallm_fp8bs_launch_plan(M: int, N: int, K: int) -> dict:
    """The launch the GEMM entry points make for (M, N, K) (host-only query)."""
    buf = (ctypes.c_int * len(PLAN_FIELDS))()
    _check(lib().smallm_fp8bs_launch_plan(M, N, K, ctypes.cast(buf, ctypes.c_void_p)), "smallm_fp8bs_launch_plan")
    return dict(zip(PLAN_FIELDS, list(buf)))


def kernel_name(M: int, N: int, K: int, mode: int = 0) -> str:
    """Name of the GEMM kernel instantiation (mode 0 fused fp32, 1 fused e8m0, 2/3 pre-quantised),
    as the profiler prints it.  Above the small-M range the pre-quantised entries run the tiled
    kernel (32-row tiles up to 128 rows or on layouts without a 16-column group, else 64), and
    the fused entries with a workspace run the
    standalone quantisation before it (the library asks for a workspace exactly then)."""
    p = smallm_fp8bs_launch_plan(M, N, K)
    hasb = "true" if p["CB"] else "false"
    if smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K) > 0:
        e8 = "true" if mode in (1, 3) else "false"
        tm = 32 if (M <= 128 or p["NA"] == 0) else 64
        tiled = f"tiled_gemm_kernel<{tm}, {e8}, {p['NA']}, {hasb}, {p['SB']}>"
        return tiled if mode >= 2 else f"quant_act_kernel<{e8}> + {tiled}"
    return f"smallm_gemm_kernel<{p['MT']}, {mode}, {p['NA']}, {hasb}, {p['SB']}, {p['RC']}>"


# ---------------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------------

def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int, where: str):
    if status != SMALLM_OK:
        raise SmallmError(status, where)


def _need(t, dtypes, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_exact(t, dtypes, shape, name, device=None):
    """t must be a contiguous device tensor of exactly this shape and one of these dtypes (on the
    given device when one is named): the kernels write or read it as a dense array of that shape,
    and the C entry points cannot see sizes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_rows(t, M, K, name, device):
    """t must be an [M, K] byte matrix on the device with unit column stride (any row pitch)."""
    _need(t, _F8, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != (M, K):
        raise ValueError(f"{name} must be ({M}, {K}), got {tuple(t.shape)}")


_U8 = (torch.uint8,)
_F8 = (torch.uint8, torch.float8_e4m3fn)
_BF = (torch.bfloat16,)
_F32 = (torch.float32,)


# ---------------------------------------------------------------------------------------------
# load-time weight preparation
# ---------------------------------------------------------------------------------------------

def smallm_fp8bs_quant_weight(w, w8=None, sw=None, stream=None):
    """fp32 [N, K] -> (e4m3 bytes uint8 [N, K], fp32 block scales [N/128, K/128])."""
    _need(w, _F32, "w")
    N, K = w.shape
    w8 = torch.empty((N, K), dtype=torch.uint8, device=w.device) if w8 is None else w8
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device) if sw is None else sw
    _need_exact(w8, _F8, (N, K), "w8", w.device)
    _need_exact(sw, _F32, (N // 128, K // 128), "sw", w.device)
    _check(lib().smallm_fp8bs_quant_weight(_ptr(w), w.stride(0), _ptr(w8), _ptr(sw), N, K, _stream(stream)),
           "smallm_fp8bs_quant_weight")
    return w8, sw


def smallm_fp8bs_quant_weight_e8m0(w, w8=None, sw=None, stream=None):
    """fp32 [N, K] -> (e4m3 bytes uint8 [N, K], e8m0 block scale bytes uint8 [N/128, K/128])."""
    _need(w, _F32, "w")
    N, K = w.shape
    w8 = torch.empty((N, K), dtype=torch.uint8, device=w.device) if w8 is None else w8
    sw = torch.empty((N // 128, K // 128), dtype=torch.uint8, device=w.device) if sw is None else sw
    _need_exact(w8, _F8, (N, K), "w8", w.device)
    _need_exact(sw, _U8, (N // 128, K // 128), "sw", w.device)
    _check(lib().smallm_fp8bs_quant_weight_e8m0(_ptr(w), w.stride(0), _ptr(w8), _ptr(sw), N, K, _stream(stream)),
           "smallm_fp8bs_quant_weight_e8m0")
    return w8, sw


def smallm_fp8bs_pack_weight(w8, out=None, stream=None):
    """Row-major e4m3 [N, K] -> packed weight (uint8, same shape, library layout)."""
    _need(w8, _F8, "w8")
    _contig(w8, "w8")
    N, K = w8.shape
    out = torch.empty((N, K), dtype=torch.uint8, device=w8.device) if out is None else out
    _need_exact(out, _U8, (N, K), "out", w8.device)
    _check(lib().smallm_fp8bs_pack_weight(_ptr(w8), _ptr(out), N, K, _stream(stream)), "smallm_fp8bs_pack_weight")
    return out


def smallm_fp8bs_unpack_weight(w_packed, out=None, stream=None):
    _need(w_packed, _U8, "w_packed")
    _contig(w_packed, "w_packed")
    N, K = w_packed.shape
    out = torch.empty((N, K), dtype=torch.uint8, device=w_packed.device) if out is None else out
    _need_exact(out, _F8, (N, K), "out", w_packed.device)
    _check(lib().smallm_fp8bs_unpack_weight(_ptr(w_packed), _ptr(out), N, K, _stream(stream)),
           "smallm_fp8bs_unpack_weight")
    return out


# ---------------------------------------------------------------------------------------------
# per-token path
# ---------------------------------------------------------------------------------------------

def smallm_fp8bs_quant(x, q=None, sx=None, stream=None):
    """bf16 [M, K] -> (e4m3 bytes uint8 [M, K], fp32 group scales [M, K/128])."""
    _need(x, _BF, "x")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
    sx = torch.empty((M, K // 128), dtype=torch.float32, device=x.device) if sx is None else sx
    _need_rows(q, M, K, "q", x.device)
    _need_exact(sx, _F32, (M, K // 128), "sx", x.device)
    _check(lib().smallm_fp8bs_quant(_ptr(x), x.stride(0), _ptr(q), q.stride(0), _ptr(sx), M, K, _stream(stream)),
           "smallm_fp8bs_quant")
    return q, sx


def smallm_fp8bs_quant_e8m0(x, q=None, sx=None, stream=None):
    """bf16 [M, K] -> (e4m3 bytes uint8 [M, K], ue8m0 group scale bytes uint8 [M, K/128])."""
    _need(x, _BF, "x")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
    sx = torch.empty((M, K // 128), dtype=torch.uint8, device=x.device) if sx is None else sx
    _need_rows(q, M, K, "q", x.device)
    _need_exact(sx, _U8, (M, K // 128), "sx", x.device)
    _check(lib().smallm_fp8bs_quant_e8m0(_ptr(x), x.stride(0), _ptr(q), q.stride(0), _ptr(sx), M, K,
                                         _stream(stream)), "smallm_fp8bs_quant_e8m0")
    return q, sx


def _rmsnorm_quant(x, w, eps, y, q, sx, emit_y, emit_q, e8m0, stream):
    _need(x, _BF, "x")
    M, H = x.shape
    if not isinstance(w, torch.Tensor) or w.dtype != torch.bfloat16 or not w.is_cuda:
        raise TypeError("w must be a bf16 device tensor")
    if w.dim() != 1 or w.shape[0] != H or not w.is_contiguous():
        raise ValueError(f"w must be contiguous of shape [{H}]")
    if emit_y and y is None:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    if emit_q:
        q = torch.empty((M, H), dtype=torch.uint8, device=x.device) if q is None else q
        sdt = torch.uint8 if e8m0 else torch.float32
        sx = torch.empty((M, H // 128), dtype=sdt, device=x.device) if sx is None else sx
    else:
        q = sx = None
    if y is not None:
        _need(y, _BF, "y")
        if tuple(y.shape) != (M, H) or y.device != x.device:
            raise ValueError(f"y must be [{M}, {H}] on {x.device}")
    if q is not None:
        _need_rows(q, M, H, "q", x.device)
        _need_exact(sx, _U8 if e8m0 else _F32, (M, H // 128), "sx", x.device)
    fn = lib().smallm_fp8bs_rmsnorm_quant_e8m0 if e8m0 else lib().smallm_fp8bs_rmsnorm_quant
    _check(fn(_ptr(x), x.stride(0), _ptr(w), ctypes.c_float(eps), _ptr(y), y.stride(0) if y is not None else 0,
              _ptr(q), q.stride(0) if q is not None else 0, _ptr(sx), M, H, _stream(stream)),
           "smallm_fp8bs_rmsnorm_quant" + ("_e8m0" if e8m0 else ""))
    return y, q, sx


def smallm_fp8bs_rmsnorm_quant(x, w, eps, y=None, q=None, sx=None, emit_y=True, emit_q=True, stream=None):
    """RMSNorm of bf16 x [M, H] with bf16 weight w [H], then the 1x128 quantisation of the bf16
    output with fp32 group scales.  Returns (y or None, q or None, sx or None)."""
    return _rmsnorm_quant(x, w, eps, y, q, sx, emit_y, emit_q, False, stream)


def smallm_fp8bs_rmsnorm_quant_e8m0(x, w, eps, y=None, q=None, sx=None, emit_y=True, emit_q=True, stream=None):
    """As smallm_fp8bs_rmsnorm_quant with ue8m0 group scales."""
    return _rmsnorm_quant(x, w, eps, y, q, sx, emit_y, emit_q, True, stream)


def _check_weight(w_packed, sw, K, e8m0):
    N = w_packed.shape[0]
    if w_packed.shape[1] != K:
        raise ValueError(f"packed weight is [{N}, {w_packed.shape[1]}] but the activations have K={K}")
    if tuple(sw.shape) != (N // 128, K // 128):
        raise ValueError(f"weight scales must be [{N // 128}, {K // 128}], got {tuple(sw.shape)}")
    if sw.dtype != (torch.uint8 if e8m0 else torch.float32):
        raise TypeError(f"weight scales must be {'uint8 (e8m0)' if e8m0 else 'float32'}, got {sw.dtype}")
    _need_exact(sw, (sw.dtype,), (N // 128, K // 128), "weight scales", w_packed.device)
    return N


def _check_act_scales(sx, M, K, e8m0):
    if tuple(sx.shape) != (M, K // 128):
        raise ValueError(f"activation scales must be [{M}, {K // 128}], got {tuple(sx.shape)}")
    if sx.dtype != (torch.uint8 if e8m0 else torch.float32):
        raise TypeError(f"activation scales must be {'uint8 (e8m0)' if e8m0 else 'float32'}, got {sx.dtype}")
    _need_exact(sx, (sx.dtype,), (M, K // 128), "activation scales")


def _out(y, M, N, device):
    if y is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device)
    _need(y, _BF, "y")
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be [{M}, {N}], got {tuple(y.shape)}")
    if y.device != device:
        raise ValueError(f"y is on {y.device}, expected {device}")
    return y


def _check_dbg(q_dbg, sx_dbg, M, K, e8m0, device):
    """The fused kernels write the debug copies as dense arrays: q_dbg [M, K] bytes at row pitch K,
    sx_dbg [M, K/128] (fp32, or e8m0 bytes)."""
    if q_dbg is not None:
        _need_exact(q_dbg, _F8, (M, K), "q_dbg", device)
    if sx_dbg is not None:
        _need_exact(sx_dbg, _U8 if e8m0 else _F32, (M, K // 128), "sx_dbg", device)


def smallm_fp8bs_gemm(q, sx, w_packed, sw, y=None, layout_id=None, stream=None):
    """Pre-quantised q [M, K] (uint8) and fp32 sx [M, K/128] times the packed weight -> bf16 [M, N]."""
    _need(q, _F8, "q")
    _need(w_packed, _U8, "w_packed")
    _contig(sx, "sx")
    _contig(sw, "sw")
    M, K = q.shape
    N = _check_weight(w_packed, sw, K, False)
    _check_act_scales(sx, M, K, False)
    y = _out(y, M, N, q.device)
    lid = smallm_fp8bs_weight_layout_id(N, K) if layout_id is None else layout_id
    _check(lib().smallm_fp8bs_gemm(_ptr(q), q.stride(0), _ptr(sx), _ptr(w_packed), lid, _ptr(sw), _ptr(y),
                                   y.stride(0), M, N, K, _stream(stream)), "smallm_fp8bs_gemm")
    return y


def smallm_fp8bs_gemm_e8m0(q, sx, w_packed, sw, y=None, layout_id=None, stream=None):
    _need(q, _F8, "q")
    _need(w_packed, _U8, "w_packed")
    _contig(sx, "sx")
    _contig(sw, "sw")
    M, K = q.shape
    N = _check_weight(w_packed, sw, K, True)
    _check_act_scales(sx, M, K, True)
    y = _out(y, M, N, q.device)
    lid = smallm_fp8bs_weight_layout_id(N, K) if layout_id is None else layout_id
    _check(lib().smallm_fp8bs_gemm_e8m0(_ptr(q), q.stride(0), _ptr(sx), _ptr(w_packed), lid, _ptr(sw), _ptr(y),
                                        y.stride(0), M, N, K, _stream(stream)), "smallm_fp8bs_gemm_e8m0")
    return y


_floor_sink = {}


def smallm_fp8bs_read_floor(buf, stream=None):
    """Stream every byte of the device tensor buf with the library's plain streaming-read kernel
    (a roofline reference, not part of the method)."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    sink = _floor_sink.get(buf.device)
    if sink is None:
        sink = _floor_sink[buf.device] = torch.zeros(2048, dtype=torch.int32, device=buf.device)
    _check(lib().smallm_fp8bs_read_floor(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                         _stream(stream)), "smallm_fp8bs_read_floor")


def smallm_fp8bs_quant_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K))


def _fused(x, w_packed, sw, y, q_dbg, sx_dbg, layout_id, stream, workspace, e8m0):
    _need(x, _BF, "x")
    _need(w_packed, _U8, "w_packed")
    _contig(sw, "sw")
    M, K = x.shape
    N = _check_weight(w_packed, sw, K, e8m0)
    y = _out(y, M, N, x.device)
    _check_dbg(q_dbg, sx_dbg, M, K, e8m0, x.device)
    lid = smallm_fp8bs_weight_layout_id(N, K) if layout_id is None else layout_id
    sfx = "_e8m0" if e8m0 else ""
    need = smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K)
    if need and q_dbg is None and sx_dbg is None:
        # beyond the small-M range: quantisation into a workspace, then the tiled GEMM
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        if (workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous()
                or not workspace.is_cuda or workspace.device != x.device):
            raise ValueError("workspace must be a contiguous 1-D uint8 tensor on the device of x")
        fn = getattr(lib(), "smallm_fp8bs_quant_gemm" + sfx + "_ws")
        _check(fn(_ptr(x), x.stride(0), _ptr(w_packed), lid, _ptr(sw), _ptr(y), y.stride(0), M, N, K,
                  _ptr(workspace), workspace.numel(), _stream(stream)), "smallm_fp8bs_quant_gemm" + sfx + "_ws")
        return y
    fn = getattr(lib(), "smallm_fp8bs_quant_gemm" + sfx)
    _check(fn(_ptr(x), x.stride(0), _ptr(w_packed), lid, _ptr(sw), _ptr(y), y.stride(0), M, N, K,
              _ptr(q_dbg), _ptr(sx_dbg), _stream(stream)), "smallm_fp8bs_quant_gemm" + sfx)
    return y


def smallm_fp8bs_quant_gemm(x, w_packed, sw, y=None, q_dbg=None, sx_dbg=None, layout_id=None, stream=None,
                            workspace=None):
    """Fused path: bf16 x [M, K], packed weight [N, K], fp32 sw [N/128, K/128] -> bf16 y [M, N].
    Beyond 32 rows (without debug copies) it takes the quant + tiled GEMM path through a workspace
    (allocated here when none is given, smallm_fp8bs_quant_gemm_workspace_bytes long); with q_dbg /
    sx_dbg it always runs the fused kernel, which writes the quantised bytes and scales it used."""
    return _fused(x, w_packed, sw, y, q_dbg, sx_dbg, layout_id, stream, workspace, False)


def smallm_fp8bs_quant_gemm_e8m0(x, w_packed, sw, y=None, q_dbg=None, sx_dbg=None, layout_id=None, stream=None,
                                 workspace=None):
    """As smallm_fp8bs_quant_gemm with e8m0 scales (sw uint8 [N/128, K/128])."""
    return _fused(x, w_packed, sw, y, q_dbg, sx_dbg, layout_id, stream, workspace, True)


def algorithmic_bytes(M: int, N: int, K: int, e8m0: bool = False) -> int:
    """Bytes one fused call must move at minimum: the fp8 weight once, its block scales, the bf16
    activations and the bf16 output."""
    s_w = 1 if e8m0 else 4
    return N * K + s_w * (N // 128) * (K // 128) + 2 * M * K + 2 * M * N


# ---------------------------------------------------------------------------------------------
# FP8 block-scale small-M fused MoE layer
# ---------------------------------------------------------------------------------------------

MOE_MAX_T = 48


def smallm_fp8bs_moe_layout_id() -> int:
    return int(lib().smallm_fp8bs_moe_layout_id())


def smallm_fp8bs_moe_supported(T: int, S: int, E: int, H: int, I: int) -> int:
    return int(lib().smallm_fp8bs_moe_supported(T, S, E, H, I))


def _need3(t, dtypes, name):
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes:
        raise TypeError(f"{name} must be a tensor with dtype in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 3 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 3-D tensor")


def _moe_pack(w, gate_up, out, stream, pack):
    _need3(w, _F8, "w")
    E, R, K = w.shape
    out = torch.empty((E, R, K), dtype=torch.uint8, device=w.device) if out is None else out
    _need3(out, _F8, "out")
    fn = lib().smallm_fp8bs_moe_pack if pack else lib().smallm_fp8bs_moe_unpack
    _check(fn(_ptr(w), _ptr(out), E, R, K, int(bool(gate_up)), _stream(stream)),
           "smallm_fp8bs_moe_pack" if pack else "smallm_fp8bs_moe_unpack")
    return out


def smallm_fp8bs_moe_pack(w8, gate_up: bool, out=None, stream=None):
    """Stacked row-major e4m3 expert matrices [E, R, K] -> packed MoE layout (same shape).
    gate_up=True for w13 [E, 2 I, H], False for w2 [E, H, I]."""
    return _moe_pack(w8, gate_up, out, stream, True)


def smallm_fp8bs_moe_unpack(w_packed, gate_up: bool, out=None, stream=None):
    return _moe_pack(w_packed, gate_up, out, stream, False)


def smallm_fp8bs_moe_workspace_bytes(T: int, S: int, H: int, I: int) -> int:
    return int(lib().smallm_fp8bs_moe_workspace_bytes(T, S, H, I))


def smallm_fp8bs_moe_splits(T: int, S: int) -> int:
    return int(lib().smallm_fp8bs_moe_splits(T, S))


def moe_h_view(workspace, T: int, S: int, I: int):
    """The bf16 intermediate h [T * S, I] at the start of a MoE workspace."""
    return workspace[: T * S * I * 2].view(torch.bfloat16).view(T * S, I)


def _moe_common(x, topk_ids, topk_w, w13_packed, w2_packed, fp4):
    _need(x, _BF, "x")
    T, H = x.shape
    for t_, n_, dt in ((topk_ids, "topk_ids", torch.int32), (topk_w, "topk_w", torch.float32)):
        if not isinstance(t_, torch.Tensor) or t_.dtype != dt or not t_.is_cuda or t_.dim() != 2:
            raise TypeError(f"{n_} must be a 2-D {dt} device tensor")
        _contig(t_, n_)
    S = topk_ids.shape[1]
    if tuple(topk_ids.shape) != (T, S) or tuple(topk_w.shape) != (T, S):
        raise ValueError(f"topk_ids and topk_w must both be [{T}, S]")
    _need3(w13_packed, _U8, "w13_packed")
    _need3(w2_packed, _U8, "w2_packed")
    E, I2, H2 = w13_packed.shape
    I = I2 // 2
    f = 2 if fp4 else 1           # K elements per byte
    if H2 * f != H or tuple(w2_packed.shape) != (E, H, I // f):
        raise ValueError(f"w13 must be [E, 2 I, {H // f}] and w2 [E, {H}, I/{f}], got {tuple(w13_packed.shape)} "
                         f"and {tuple(w2_packed.shape)}")
    return T, S, E, H, I


def _moe_workspace_arg(workspace, T, S, H, I, device):
    need = smallm_fp8bs_moe_workspace_bytes(T, S, H, I)
    if workspace is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if not workspace.is_cuda:
        raise ValueError("workspace must be a device tensor")
    return workspace


def smallm_fp8bs_moe(x, topk_ids, topk_w, w13_packed, sw13, w2_packed, sw2, workspace=None, y=None,
                     layout_id=None, stream=None):
    """MoE layer: bf16 x [T, H], int32 topk_ids / fp32 topk_w [T, S], packed w13 [E, 2 I, H] with fp32
    sw13 [E, 2 I/128, H/128], packed w2 [E, H, I] with fp32 sw2 [E, H/128, I/128].  Returns (y bf16
    [T, H], h bf16 [T * S, I]); h, the intermediate silu(g) * u of every (token, slot) pair, is a view
    of the workspace (uint8, smallm_fp8bs_moe_workspace_bytes long; allocated when None)."""
    T, S, E, H, I = _moe_common(x, topk_ids, topk_w, w13_packed, w2_packed, False)
    for t_, n_, shp in ((sw13, "sw13", (E, 2 * I // 128, H // 128)), (sw2, "sw2", (E, H // 128, I // 128))):
        if not isinstance(t_, torch.Tensor) or t_.dtype != torch.float32 or tuple(t_.shape) != shp:
            raise ValueError(f"{n_} must be float32 {shp}")
        if not t_.is_cuda:
            raise ValueError(f"{n_} must be a device tensor")
        _contig(t_, n_)
    workspace = _moe_workspace_arg(workspace, T, S, H, I, x.device)
    y = _out(y, T, H, x.device)
    lid = smallm_fp8bs_moe_layout_id() if layout_id is None else layout_id
    _check(lib().smallm_fp8bs_moe(_ptr(x), x.stride(0), _ptr(topk_ids), _ptr(topk_w), T, S, _ptr(w13_packed),
                                  _ptr(sw13), _ptr(w2_packed), _ptr(sw2), lid, E, H, I, _ptr(workspace),
                                  workspace.numel(), _ptr(y), y.stride(0), _stream(stream)), "smallm_fp8bs_moe")
    return y, moe_h_view(workspace, T, S, I)


MOE_NOALLOC_MAX_BYTES = 4 << 20


def smallm_fp8bs_moe_noalloc(x, topk_ids, topk_w, w13_packed, sw13, w2_packed, sw2, y=None, layout_id=None,
                             stream=None):
    """smallm_fp8bs_moe with the library's own static workspace (the C entry point allocates
    nothing; pass y to avoid the output allocation here too).  Returns y."""
    T, S, E, H, I = _moe_common(x, topk_ids, topk_w, w13_packed, w2_packed, False)
    for t_, n_, shp in ((sw13, "sw13", (E, 2 * I // 128, H // 128)), (sw2, "sw2", (E, H // 128, I // 128))):
        if not isinstance(t_, torch.Tensor) or t_.dtype != torch.float32 or tuple(t_.shape) != shp:
            raise ValueError(f"{n_} must be float32 {shp}")
        if not t_.is_cuda:
            raise ValueError(f"{n_} must be a device tensor")
        _contig(t_, n_)
    y = _out(y, T, H, x.device)
    lid = smallm_fp8bs_moe_layout_id() if layout_id is None else layout_id
    _check(lib().smallm_fp8bs_moe_noalloc(_ptr(x), x.stride(0), _ptr(topk_ids), _ptr(topk_w), T, S,
                                          _ptr(w13_packed), _ptr(sw13), _ptr(w2_packed), _ptr(sw2), lid, E, H, I,
                                          _ptr(y), y.stride(0), _stream(stream)), "smallm_fp8bs_moe_noalloc")
    return y


# ---------------------------------------------------------------------------------------------
# the MoE layer with MXFP4 expert weights
# ---------------------------------------------------------------------------------------------

def smallm_fp8bs_moe_mxfp4_layout_id() -> int:
    return int(lib().smallm_fp8bs_moe_mxfp4_layout_id())


def _moe_mxfp4_pack(w, s, gate_up, out, out_s, stream, pack):
    _need3(w, _U8, "w")
    _need3(s, _U8, "s")
    E, R, K2 = w.shape
    K = 2 * K2
    if tuple(s.shape) != (E, R, K // 32):
        raise ValueError(f"scales must be uint8 [{E}, {R}, {K // 32}], got {tuple(s.shape)}")
    out = torch.empty_like(w) if out is None else out
    out_s = torch.empty_like(s) if out_s is None else out_s
    _need3(out, _U8, "out")
    _need3(out_s, _U8, "out_s")
    fn = lib().smallm_fp8bs_moe_mxfp4_pack if pack else lib().smallm_fp8bs_moe_mxfp4_unpack
    _check(fn(_ptr(w), _ptr(s), _ptr(out), _ptr(out_s), E, R, K, int(bool(gate_up)), _stream(stream)),
           "smallm_fp8bs_moe_mxfp4_pack" if pack else "smallm_fp8bs_moe_mxfp4_unpack")
    return out, out_s


def smallm_fp8bs_moe_mxfp4_pack(w4, s, gate_up: bool, out=None, out_s=None, stream=None):
    """Stacked fp4x2 expert matrices [E, R, K/2] (uint8) and their e8m0 scales [E, R, K/32] ->
    (packed weights, packed scales), same shapes.  gate_up=True for w13 (R = 2 I, K = H), False
    for w2 (R = H, K = I)."""
    return _moe_mxfp4_pack(w4, s, gate_up, out, out_s, stream, True)


def smallm_fp8bs_moe_mxfp4_unpack(w_packed, s_packed, gate_up: bool, out=None, out_s=None, stream=None):
    return _moe_mxfp4_pack(w_packed, s_packed, gate_up, out, out_s, stream, False)


def smallm_fp8bs_moe_mxfp4(x, topk_ids, topk_w, w13_packed, s13_packed, w2_packed, s2_packed, workspace=None,
                           y=None, layout_id=None, stream=None):
    """MoE layer with MXFP4 experts: bf16 x [T, H], int32 topk_ids / fp32 topk_w [T, S], packed fp4x2
    w13 [E, 2 I, H/2] with packed e8m0 scales [E, 2 I, H/32], packed w2 [E, H, I/2] with scales
    [E, H, I/32].  Returns (y bf16 [T, H], h bf16 [T * S, I]) as smallm_fp8bs_moe does."""
    T, S, E, H, I = _moe_common(x, topk_ids, topk_w, w13_packed, w2_packed, True)
    for t_, n_, shp in ((s13_packed, "s13_packed", (E, 2 * I, H // 32)), (s2_packed, "s2_packed", (E, H, I // 32))):
        if not isinstance(t_, torch.Tensor) or t_.dtype != torch.uint8 or tuple(t_.shape) != shp:
            raise ValueError(f"{n_} must be uint8 {shp}")
        if not t_.is_cuda:
            raise ValueError(f"{n_} must be a device tensor")
        _contig(t_, n_)
    workspace = _moe_workspace_arg(workspace, T, S, H, I, x.device)
    y = _out(y, T, H, x.device)
    lid = smallm_fp8bs_moe_mxfp4_layout_id() if layout_id is None else layout_id
    _check(lib().smallm_fp8bs_moe_mxfp4(_ptr(x), x.stride(0), _ptr(topk_ids), _ptr(topk_w), T, S,
                                        _ptr(w13_packed), _ptr(s13_packed), _ptr(w2_packed), _ptr(s2_packed), lid,
                                        E, H, I, _ptr(workspace), workspace.numel(), _ptr(y), y.stride(0),
                                        _stream(stream)), "smallm_fp8bs_moe_mxfp4")
    return y, moe_h_view(workspace, T, S, I)


def moe_algorithmic_bytes(ids, E: int, H: int, I: int, mxfp4: bool = False) -> int:
    """Bytes one MoE call must move at minimum: each expert in use once (e4m3 w13 and w2 with
    their fp32 block scales, or MXFP4 with their e8m0 group scales), the bf16 activations, ids and
    weights, the bf16 intermediate written and read once, and the bf16 output."""
    import numpy as np
    ids = np.asarray(ids)
    T, S = ids.shape
    used = np.unique(ids[(ids >= 0) & (ids < E)])
    if mxfp4:
        per_expert = 3 * H * I // 2 + 3 * H * I // 32
    else:
        per_expert = 3 * H * I + 4 * (2 * I // 128) * (H // 128) + 4 * (H // 128) * (I // 128)
    return int(len(used) * per_expert + 2 * T * H + 8 * T * S + 2 * 2 * T * S * I + 2 * T * H)


def moe_workspace(T: int, S: int, H: int, I: int, device="cuda:0"):
    """A workspace tensor for smallm_fp8bs_moe (256-byte aligned by the caching allocator)."""
    return torch.empty(max(smallm_fp8bs_moe_workspace_bytes(T, S, H, I), 256), dtype=torch.uint8, device=device)
