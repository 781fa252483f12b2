"""GPU parity: the HIP library against the CPU oracle, element by element.

Quantised bytes and scales must be identical to the oracle's; the bf16 output must satisfy
|y - ref| <= 8e-3 * |ref| + 1e-3 * max|ref| for every element, with ref the oracle's fp64 result
built from the same quantised operands.  Full-size shapes are checked on column windows at both
ends of N (the first and last workgroups), in the launch configuration the benchmark uses.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import precision_gemm_x128_amd as P
import synthgen

pytestmark = pytest.mark.gpu

REL_TOL = 8e-3
ABS_TOL_FRAC = 1e-3

DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x_bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_to_np_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def assert_within_tol(y_dev: torch.Tensor, ref: np.ndarray, cols=None, what=""):
    y = bf16_to_np_f64(y_dev)
    if cols is not None:
        y, ref = y[:, cols], ref[:, cols]
    tol = REL_TOL * np.abs(ref) + ABS_TOL_FRAC * np.abs(ref).max()
    err = np.abs(y - ref)
    bad = err > tol
    assert np.isfinite(y).all(), what
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, worst err {err.max():.3e}, " \
                          f"at {np.unravel_index(np.argmax(err - tol), err.shape)}"


def windows(N, width=256):
    if N <= 2 * width:
        return np.arange(N), [(0, N)]
    return np.r_[0:width, N - width:N], [(0, width), (N - width, N)]


_weight_cache = {}


def prepared_weight(N, K, seed=0, copy=0, e8m0=False):
    """(w8 oracle bytes, sw oracle, packed device weight, device scales); oracle-quantised."""
    key = (N, K, seed, copy, e8m0)
    if key not in _weight_cache:
        w = synthgen.gen_w(N, K, seed=seed, copy=copy)
        w8, sw = oracle.quant_weight(w, e8m0=e8m0)
        wp = P.smallm_fp8bs_pack_weight(to_dev(w8))
        _weight_cache.clear()
        _weight_cache[key] = (w8, sw, wp, to_dev(sw))
    return _weight_cache[key]


def oracle_ref(x_bits, w8, sw, e8m0, col_ranges):
    q, sx = oracle.quant_act(x_bits, e8m0=e8m0)
    ref = np.zeros((x_bits.shape[0], w8.shape[0]))
    for a, b in col_ranges:
        ref[:, a:b] = oracle.gemm(q, sx, w8, sw, e8m0=e8m0, n0=a, n1=b)[:, a:b]
    return q, sx, ref


# ---------------------------------------------------------------------------------------------
# load-time kernels
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("e8m0", [False, True])
def test_quant_weight_bitexact(e8m0):
    note(f"quant_weight e8m0={e8m0}")
    w = synthgen.gen_w(384, 512, seed=5, copy=1)
    w[0:128, 0:128] = 0.0                                   # all-zero block
    w[128:256, 128:256] *= np.float32(1e-30)                # tiny block
    w[256:384, 256:384] *= np.float32(1e4)                  # large block
    w[0, 300] = -0.0
    w8_ref, sw_ref = oracle.quant_weight(w, e8m0=e8m0)
    fn = P.smallm_fp8bs_quant_weight_e8m0 if e8m0 else P.smallm_fp8bs_quant_weight
    w8, sw = fn(to_dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(w8.cpu().numpy(), w8_ref)
    assert np.array_equal(sw.cpu().numpy().view(np.uint8 if e8m0 else np.uint32),
                          sw_ref.view(np.uint8 if e8m0 else np.uint32))


@pytest.mark.parametrize("N,K", [(256, 384), (4096, 2048), (5120, 512), (4608, 1024), (2048, 512)])
def test_pack_unpack_roundtrip_and_fragment_order(N, K):
    note(f"pack/unpack N={N} K={K}")
    rng = np.random.default_rng(N + K)
    w8 = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    wd = to_dev(w8)
    wp = P.smallm_fp8bs_pack_weight(wd)
    back = P.smallm_fp8bs_unpack_weight(wp)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), w8)
    packed = wp.cpu().numpy().reshape(-1)
    assert np.array_equal(np.sort(packed), np.sort(w8.reshape(-1)))
    # fragment f = cg * KG + h: lane 16*chunk + j holds column cg*C + j//S, K block h*S + j%S,
    # bytes [32 chunk, 32 chunk + 32) of it (first 16 at lane*16, next 16 at 1024 + lane*16)
    C = P.layout_columns(N, K)
    S = 16 // C
    KG = K // 128 // S
    for cg, h in ((0, 0), (1, KG - 1), (N // C - 1, KG // 2)):
        f = cg * KG + h
        frag = packed[f * 2048:(f + 1) * 2048]
        for chunk in range(4):
            for j in (0, 5, 15):
                lane = 16 * chunk + j
                got = np.r_[frag[lane * 16:lane * 16 + 16], frag[1024 + lane * 16:1024 + lane * 16 + 16]]
                k0 = (h * S + j % S) * 128 + 32 * chunk
                assert np.array_equal(got, w8[cg * C + j // S, k0:k0 + 32])


# ---------------------------------------------------------------------------------------------
# activation quantisation (standalone and inside the fused kernel)
# ---------------------------------------------------------------------------------------------

def special_x(M, K, seed):
    """gen_x rows plus groups that stress the quantiser: all-zero (with signed zeros), amax exactly
    448, tiny amax (scale below 2^-64: true-division path), bf16 subnormals, huge values."""
    x = synthgen.gen_x(M, K, seed=seed, outliers=True)
    f = synthgen.bf16_bits_to_f32(x)
    G = K // 128
    if M >= 1 and G >= 4:
        x[0, 0:128] = 0
        x[0, 5] = 0x8000
        x[0, 128:256] = synthgen.f32_to_bf16_bits(f[0, 128:256] / np.abs(f[0, 128:256]).max() * 448.0)
        x[0, 256:384] = synthgen.f32_to_bf16_bits(f[0, 256:384] * np.float32(1e-30))
        x[0, 384:512] = synthgen.f32_to_bf16_bits(f[0, 384:512] * np.float32(1e-36))
    if M >= 2 and G >= 4:
        x[1, 0:128] = synthgen.f32_to_bf16_bits(f[1, 0:128] * np.float32(1e-39))   # bf16 subnormals
        x[1, 128:256] = synthgen.f32_to_bf16_bits(f[1, 128:256] * np.float32(1e34))
        x[1, 256:384] = synthgen.f32_to_bf16_bits(f[1, 256:384] * np.float32(2.0 ** -70))
        x[1, 384] = 0x0001                                                           # min subnormal
    return x


QUANT_SHAPES = [(1, 2048), (3, 512), (4, 2048), (9, 4096), (16, 4096), (17, 2048), (32, 4096), (256, 2048),
                (2, 16384), (33, 12416)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
@pytest.mark.parametrize("e8m0", [False, True])
def test_quant_bitexact(M, K, e8m0):
    note(f"quant M={M} K={K} e8m0={e8m0}")
    x = special_x(M, K, seed=M + K)
    q_ref, sx_ref = oracle.quant_act(x, e8m0=e8m0)
    fn = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
    q, sx = fn(to_dev_bf16(x))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy().view(np.uint8 if e8m0 else np.uint32),
                          sx_ref.view(np.uint8 if e8m0 else np.uint32))


def test_quant_exhaustive_bf16_values():
    """Every finite bf16 value appears in a group whose amax is 448 (scale 1) and in groups with
    non-power-of-two scales: bytes must match the oracle's IEEE-division reading."""
    note("quant exhaustive bf16")
    vals = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = synthgen.bf16_bits_to_f32(vals)
    fin = vals[np.isfinite(f) & (np.abs(f) <= 448.0)]
    pad = (-len(fin)) % 127
    fin = np.r_[fin, np.zeros(pad, dtype=np.uint16)].reshape(-1, 127)
    rows = []
    for amax_bits in (0x43E0, 0x43E1, 0x4040, 0x3F81, 0x0F23):   # 448, 450, 3, 1.0078125, tiny
        a = float(synthgen.bf16_bits_to_f32(np.array([amax_bits], dtype=np.uint16))[0])
        vf = synthgen.bf16_bits_to_f32(fin) * np.float32(a / 448.0)
        g = np.c_[synthgen.f32_to_bf16_bits(vf), np.full((fin.shape[0], 1), amax_bits, dtype=np.uint16)]
        rows.append(g.reshape(-1))
    x = np.concatenate(rows)
    x = np.r_[x, np.zeros((-len(x)) % 1024, dtype=np.uint16)].reshape(-1, 1024)
    for e8m0 in (False, True):
        q_ref, sx_ref = oracle.quant_act(x, e8m0=e8m0)
        fn = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
        q, sx = fn(to_dev_bf16(x))
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q_ref), f"e8m0={e8m0}"
        assert np.array_equal(sx.cpu().numpy().view(np.uint8 if e8m0 else np.uint32),
                              sx_ref.view(np.uint8 if e8m0 else np.uint32))


def every_amax_groups(seed=7):
    """One 1x128 group per positive finite bf16 amax (0x0001 .. 0x7F7F): the amax itself plus 127
    random bf16 of magnitude <= amax with random signs, as rows of 32 groups (K = 4096).  Covers
    the tiny-scale rescaling, subnormal scales and reciprocals, and the largest scales."""
    rng = np.random.default_rng([seed, 11])
    amax = np.arange(1, 0x7F80, dtype=np.uint32)
    mag = (rng.random((len(amax), 127)) * (amax[:, None] + 1)).astype(np.uint32)
    mag = np.minimum(mag, amax[:, None])
    sgn = rng.integers(0, 2, (len(amax), 127), dtype=np.uint32) << 15
    g = np.c_[(mag | sgn), amax].astype(np.uint16)
    g = np.take_along_axis(g, rng.permuted(np.tile(np.arange(128), (len(amax), 1)), axis=1), axis=1)
    pad = (-len(amax)) % 32
    g = np.r_[g, np.zeros((pad, 128), dtype=np.uint16)]
    return g.reshape(-1, 4096)


def test_quant_every_bf16_amax():
    note("quant every bf16 amax")
    x = every_amax_groups()
    for e8m0 in (False, True):
        q_ref, sx_ref = oracle.quant_act(x, e8m0=e8m0)
        fn = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
        for r0 in range(0, x.shape[0], 256):                # at most 256 rows per call
            q, sx = fn(to_dev_bf16(x[r0:r0 + 256]))
            torch.cuda.synchronize()
            assert np.array_equal(q.cpu().numpy(), q_ref[r0:r0 + 256]), f"e8m0={e8m0} rows {r0}.."
            assert np.array_equal(sx.cpu().numpy().view(np.uint8 if e8m0 else np.uint32),
                                  sx_ref[r0:r0 + 256].view(np.uint8 if e8m0 else np.uint32))


@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_debug_quant_every_bf16_amax(e8m0):
    """The fused kernel's quantiser on the same groups, 32 rows (1024 groups) per call."""
    note(f"fused debug quant every bf16 amax e8m0={e8m0}")
    x = every_amax_groups()
    q_ref, sx_ref = oracle.quant_act(x, e8m0=e8m0)
    N, K = 256, 4096
    w8, sw, wp, swd = prepared_weight(N, K, seed=3, e8m0=e8m0)
    fn = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    for r0 in range(0, x.shape[0], 32):
        xs = x[r0:r0 + 32]
        M = xs.shape[0]
        q_dbg = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
        sx_dbg = torch.zeros((M, K // 128), dtype=torch.uint8 if e8m0 else torch.float32, device=DEV)
        fn(to_dev_bf16(xs), wp, swd, q_dbg=q_dbg, sx_dbg=sx_dbg)
        torch.cuda.synchronize()
        assert np.array_equal(q_dbg.cpu().numpy(), q_ref[r0:r0 + M]), f"rows {r0}.."
        assert np.array_equal(sx_dbg.cpu().numpy().view(np.uint8 if e8m0 else np.uint32),
                              sx_ref[r0:r0 + M].view(np.uint8 if e8m0 else np.uint32)), f"rows {r0}.."


@pytest.mark.parametrize("M", [1, 4, 16, 17, 32, 48])
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_debug_quant_bitexact(M, e8m0):
    note(f"fused debug quant M={M} e8m0={e8m0}")
    N, K = 256, 2048
    x = special_x(M, K, seed=100 + M)
    w8, sw, wp, swd = prepared_weight(N, K, seed=3, e8m0=e8m0)
    q_ref, sx_ref = oracle.quant_act(x, e8m0=e8m0)
    q_dbg = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    sx_dbg = torch.zeros((M, K // 128), dtype=torch.uint8 if e8m0 else torch.float32, device=DEV)
    fn = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    fn(to_dev_bf16(x), wp, swd, q_dbg=q_dbg, sx_dbg=sx_dbg)
    torch.cuda.synchronize()
    assert np.array_equal(q_dbg.cpu().numpy(), q_ref)
    assert np.array_equal(sx_dbg.cpu().numpy().view(np.uint8 if e8m0 else np.uint32),
                          sx_ref.view(np.uint8 if e8m0 else np.uint32))


# ---------------------------------------------------------------------------------------------
# GEMM: fused and on pre-quantised input, fp32 and e8m0 scales
# ---------------------------------------------------------------------------------------------

SMALL_SHAPES = [(128, 128), (256, 384), (384, 640), (128, 4736)]   # several tiles, ragged K rounds
FULL_SHAPES = [(4096, 2048), (5120, 4096), (4608, 4096), (2048, 4096)]
M_LIST = [1, 3, 4, 8, 9, 16, 17, 24, 32]


@pytest.mark.parametrize("N,K", SMALL_SHAPES)
@pytest.mark.parametrize("M", [1, 5, 16, 23, 32])
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_small_shapes_full_output(N, K, M, e8m0):
    note(f"fused small N={N} K={K} M={M} e8m0={e8m0}")
    x = special_x(M, K, seed=N + K + M) if K >= 512 else synthgen.gen_x(M, K, seed=N + M)
    w8, sw, wp, swd = prepared_weight(N, K, seed=7, e8m0=e8m0)
    _, _, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
    fn = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    y = fn(to_dev_bf16(x), wp, swd)
    torch.cuda.synchronize()
    assert_within_tol(y, ref, what=f"N={N} K={K} M={M} e8m0={e8m0}")


@pytest.mark.parametrize("N,K", FULL_SHAPES)
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_full_shapes_all_m(N, K, e8m0):
    w8, sw, wp, swd = prepared_weight(N, K, seed=0, copy=0, e8m0=e8m0)
    cols, ranges = windows(N)
    fn = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    for M in M_LIST:
        note(f"fused full N={N} K={K} M={M} e8m0={e8m0}")
        x = synthgen.gen_x(M, K, seed=M, outliers=(M % 2 == 1))
        _, _, ref = oracle_ref(x, w8, sw, e8m0, ranges)
        y = fn(to_dev_bf16(x), wp, swd)
        torch.cuda.synchronize()
        assert_within_tol(y, ref, cols, what=f"N={N} K={K} M={M} e8m0={e8m0}")


# Shapes that exercise every work split of the launch plan: column groups of C = 16, 8, 4, 2
# columns; 1, 2, 3, 5, 9 and 12 column groups per workgroup; K shared by 4, 2 or 1 MFMA waves;
# and K of 16384 and 12416 (several K rounds, the last one ragged).
PLAN_SHAPES = [(8192, 256), (12288, 256), (6144, 1024), (5120, 512), (4608, 1024), (2048, 512),
               (36864, 128), (49152, 256),
               (2048, 16384), (1024, 12416)]   # long K: four full rounds; 97 K blocks, a ragged last round


@pytest.mark.parametrize("N,K", PLAN_SHAPES)
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_launch_plans(N, K, e8m0):
    w8, sw, wp, swd = prepared_weight(N, K, seed=11, e8m0=e8m0)
    cols, ranges = windows(N, 384)
    fn = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    for M in (1, 7, 16, 32):
        note(f"plan N={N} K={K} C={P.layout_columns(N, K)} M={M} e8m0={e8m0}")
        x = special_x(M, K, seed=M + N) if K >= 512 else synthgen.gen_x(M, K, seed=M + N)
        _, _, ref = oracle_ref(x, w8, sw, e8m0, ranges)
        y = fn(to_dev_bf16(x), wp, swd)
        torch.cuda.synchronize()
        assert_within_tol(y, ref, cols, what=f"N={N} K={K} M={M} e8m0={e8m0}")


@pytest.mark.parametrize("M", [33, 48, 64, 128, 256])
def test_fused_beyond_small_m(M):
    note(f"fused beyond small M={M}")
    N, K = 4096, 2048
    w8, sw, wp, swd = prepared_weight(N, K, seed=0)
    cols, ranges = windows(N, 128)
    x = synthgen.gen_x(M, K, seed=M)
    _, _, ref = oracle_ref(x, w8, sw, False, ranges)
    y = P.smallm_fp8bs_quant_gemm(to_dev_bf16(x), wp, swd)
    torch.cuda.synchronize()
    assert_within_tol(y, ref, cols, what=f"M={M}")


@pytest.mark.parametrize("e8m0", [False, True])
@pytest.mark.parametrize("M", [1, 8, 17, 32])
def test_two_kernel_path(M, e8m0):
    note(f"two-kernel M={M} e8m0={e8m0}")
    N, K = 2048, 4096
    w8, sw, wp, swd = prepared_weight(N, K, seed=2, e8m0=e8m0)
    cols, ranges = windows(N)
    x = special_x(M, K, seed=M + 5)
    q_ref, sx_ref, ref = oracle_ref(x, w8, sw, e8m0, ranges)
    qf = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
    gf = P.smallm_fp8bs_gemm_e8m0 if e8m0 else P.smallm_fp8bs_gemm
    q, sx = qf(to_dev_bf16(x))
    y = gf(q, sx, wp, swd)
    yf = (P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm)(to_dev_bf16(x), wp, swd)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert_within_tol(y, ref, cols, what=f"two-kernel M={M}")
    # same quantised operands, same kernel arithmetic: the two paths agree bit for bit
    assert torch.equal(y.view(torch.int16), yf.view(torch.int16))


TILED_CASES = [
    # (N, K, M, full output?) -- 16-column layouts, M beyond 32: the MFMA-tiled kernel
    (384, 640, 33, True),     # 6 column tiles, 5 K blocks (not a multiple of the prefetch depth)
    (384, 640, 100, True),    # two row tiles, the second ragged
    (4096, 128, 64, True),    # a single K block
    (4096, 2048, 48, False),
    (4096, 2048, 256, False),  # four full row tiles
    (4096, 4736, 77, False),   # 37 K blocks
]


@pytest.mark.parametrize("N,K,M,full", TILED_CASES)
@pytest.mark.parametrize("e8m0", [False, True])
def test_prequantised_gemm_tiled(N, K, M, full, e8m0):
    """GEMM on pre-quantised input beyond the small-M range with a 16-column weight layout: the
    MFMA-tiled kernel, against the oracle GEMM on the oracle's quantised bytes."""
    note(f"tiled prequantised N={N} K={K} M={M} e8m0={e8m0}")
    assert P.layout_columns(N, K) == 16
    w8, sw, wp, swd = prepared_weight(N, K, seed=6, e8m0=e8m0)
    cols, ranges = (np.arange(N), [(0, N)]) if full else windows(N)
    x = special_x(M, K, seed=M + N)
    q_ref, sx_ref, ref = oracle_ref(x, w8, sw, e8m0, ranges)
    qf = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
    gf = P.smallm_fp8bs_gemm_e8m0 if e8m0 else P.smallm_fp8bs_gemm
    q, sx = qf(to_dev_bf16(x))
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    gf(q, sx, wp, swd, y=y)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert_within_tol(y, ref, cols, what=f"tiled N={N} K={K} M={M}")
    # padded row pitches: only the M x N outputs are written
    qp = torch.zeros((M, K + 16), dtype=torch.uint8, device=DEV)
    qp[:, :K] = q
    yp = torch.full((M + 3, N + 8), 5.0, dtype=torch.bfloat16, device=DEV)
    gf(qp[:, :K], sx, wp, swd, y=yp[:M, :N])
    torch.cuda.synchronize()
    assert torch.equal(yp[:M, :N].view(torch.int16), y.view(torch.int16))
    assert torch.all(yp[M:] == 5.0) and torch.all(yp[:, N:] == 5.0)


def test_padded_leading_dimensions():
    note("padded ld")
    M, N, K = 5, 384, 640
    w8, sw, wp, swd = prepared_weight(N, K, seed=9)
    x = synthgen.gen_x(M, K, seed=1)
    _, _, ref = oracle_ref(x, w8, sw, False, [(0, N)])
    xbig = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=DEV)
    xbig[:, :K] = to_dev_bf16(x)
    ybig = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device=DEV)
    P.smallm_fp8bs_quant_gemm(xbig[:, :K], wp, swd, y=ybig[:, :N])
    torch.cuda.synchronize()
    assert_within_tol(ybig[:, :N], ref)
    assert torch.all(ybig[:, N:] == 7.0)


def test_outputs_outside_rows_untouched():
    note("rows untouched")
    M, N, K = 3, 256, 256
    w8, sw, wp, swd = prepared_weight(N, K, seed=4)
    x = synthgen.gen_x(M, K, seed=2)
    y = torch.full((8, N), -3.0, dtype=torch.bfloat16, device=DEV)
    P.smallm_fp8bs_quant_gemm(to_dev_bf16(x), wp, swd, y=y[:M])
    torch.cuda.synchronize()
    assert torch.all(y[M:] == -3.0)


def test_deterministic_and_graph_replay_bitwise():
    note("graph replay")
    M, N, K = 16, 4096, 2048
    w8, sw, wp, swd = prepared_weight(N, K, seed=0)
    x = to_dev_bf16(synthgen.gen_x(M, K, seed=3))
    y1 = P.smallm_fp8bs_quant_gemm(x, wp, swd)
    y2 = P.smallm_fp8bs_quant_gemm(x, wp, swd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    yg = torch.zeros_like(y1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        P.smallm_fp8bs_quant_gemm(x, wp, swd, y=yg)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.smallm_fp8bs_quant_gemm(x, wp, swd, y=yg)
    for i in range(4):
        yg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg.view(torch.int16), y1.view(torch.int16)), f"replay {i}"
        _ = (x.float() * 2).sum()      # unrelated eager work between replays
        torch.cuda.synchronize()


def test_binding_errors_on_device():
    note("binding errors")
    M, N, K = 4, 256, 256
    w8, sw, wp, swd = prepared_weight(N, K, seed=4)
    x = to_dev_bf16(synthgen.gen_x(M, K, seed=2))
    with pytest.raises(P.SmallmError) as e:
        P.smallm_fp8bs_quant_gemm(x, wp, swd, layout_id=123)
    assert e.value.status == P.SMALLM_ERR_LAYOUT
    with pytest.raises(TypeError):
        P.smallm_fp8bs_quant_gemm(x.to(torch.float16), wp, swd)
    with pytest.raises(ValueError):
        P.smallm_fp8bs_quant_gemm(x[:, :K - 128], wp, swd)    # K does not match the weight
    with pytest.raises(TypeError):
        P.smallm_fp8bs_quant_gemm_e8m0(x, wp, swd)             # fp32 scales into the e8m0 entry
    xo = torch.zeros((M, K + 4), dtype=torch.bfloat16, device=DEV)[:, :K]
    with pytest.raises(P.SmallmError) as e:
        P.smallm_fp8bs_quant_gemm(xo, wp, swd)                 # row pitch not 16-byte aligned
    assert e.value.status == P.SMALLM_ERR_ALIGN
