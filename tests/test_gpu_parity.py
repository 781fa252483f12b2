"""GPU parity: the HIP library against the CPU oracle, element by element.

Quantised bytes and scales must be identical to the oracle's; the bf16 output must satisfy
|y - ref| <= 8e-3 * |ref| + 1e-3 * max|ref| for every element, with ref the oracle's fp64 result
built from the same quantised operands.  Every output element is compared, at the benchmark's
full shapes and launch configurations too, on each workload's own inputs (seeds, outlier rows,
graph replay).
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


def assert_within_tol(y_dev: torch.Tensor, ref: np.ndarray, what=""):
    y = bf16_to_np_f64(y_dev)
    tol = REL_TOL * np.abs(ref) + ABS_TOL_FRAC * np.abs(ref).max()
    err = np.abs(y - ref)
    bad = err > tol
    assert np.isfinite(y).all(), what
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, worst err {err.max():.3e}, " \
                          f"at {np.unravel_index(np.argmax(err - tol), err.shape)}"


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


def prepared_weight_nocache(N, K, seed=0, copy=0, e8m0=False):
    w = synthgen.gen_w(N, K, seed=seed, copy=copy)
    w8, sw = oracle.quant_weight(w, e8m0=e8m0)
    return w8, sw, P.smallm_fp8bs_pack_weight(to_dev(w8)), to_dev(sw)


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


@pytest.mark.parametrize("N,K", [(256, 384), (4096, 2048), (5120, 512), (4608, 1024), (2048, 512),
                                 (5120, 4096), (4608, 640), (1024, 12416)])
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
    lay = P.weight_layout(N, K)
    NA, CB, SB = lay["NA"], lay["CB"], lay["SB"]
    plan = P.smallm_fp8bs_launch_plan(1, N, K)
    NWG = plan["nwg"]
    assert NWG * (16 * NA + CB) == N
    KB = K // 128
    region = (16 * NA + CB) * K
    # workgroup w: 16-column fragments (lane 16 chunk + j: column 16 w + j, K bytes [32 chunk, +32) of
    # the block, first 16 at lane * 16, next 16 at 1024 + lane * 16), then the remainder fragments
    # (B column j = c SB + s: column 16 NA NWG + CB w + c, K block f SB + s)
    for w in sorted({0, 1, NWG // 2, NWG - 1}):
        base = w * region
        if NA:
            for kb in sorted({0, KB // 2, KB - 1}):
                frag = packed[base + kb * 2048: base + (kb + 1) * 2048]
                for chunk in range(4):
                    for j in (0, 5, 15):
                        lane = 16 * chunk + j
                        got = np.r_[frag[lane * 16:lane * 16 + 16], frag[1024 + lane * 16:1024 + lane * 16 + 16]]
                        k0 = kb * 128 + 32 * chunk
                        assert np.array_equal(got, w8[16 * w + j, k0:k0 + 32]), (w, kb, lane)
        if CB:
            nb = CB * SB
            fb = nb * 128
            bbase = base + NA * KB * 2048
            for f in sorted({0, KB // SB - 1}):
                frag = packed[bbase + f * fb: bbase + (f + 1) * fb]
                for chunk in range(4):
                    for j in sorted({0, nb - 1, nb // 2}):
                        idx = chunk * nb + j
                        got = np.r_[frag[idx * 16:idx * 16 + 16], frag[fb // 2 + idx * 16:fb // 2 + idx * 16 + 16]]
                        n = 16 * NA * NWG + CB * w + j // SB
                        k0 = (f * SB + j % SB) * 128 + 32 * chunk
                        assert np.array_equal(got, w8[n, k0:k0 + 32]), (w, f, idx)


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


def every_amax_value_pair_groups():
    """1x128 groups holding, for every positive finite bf16 amax, that amax and then every bf16 x
    with |x| <= amax, both signs, 127 to a group (the last group of an amax padded with zeros):
    about 8.4 million groups, 1.07e9 values."""
    parts = []
    for ab in range(1, 0x7F80):
        v = np.arange(ab + 1, dtype=np.uint16)
        v = np.concatenate([v, v | np.uint16(0x8000)])
        n = (len(v) + 126) // 127
        g = np.zeros((n, 128), dtype=np.uint16)
        g[:, 0] = ab
        g[:, 1:].reshape(-1)[:len(v)] = v
        parts.append(g)
    return np.concatenate(parts)


@pytest.mark.gpu
def test_quant_every_amax_value_pair():
    """The standalone quantiser (fp32 group scales) against the oracle over every pair of a bf16
    amax and a bf16 x with |x| <= amax: codes and scales bit-exact.  This runs the kernel's own
    instruction sequence over the whole domain the CPU proof of the quotient recipe covers."""
    note("quant every amax/value pair")
    groups = every_amax_value_pair_groups()
    per = 256 * 512                                   # groups per call: 256 rows x K = 65536
    for c0 in range(0, len(groups), per):
        chunk = groups[c0:c0 + per]
        if len(chunk) < per:
            chunk = np.concatenate([chunk, np.zeros((per - len(chunk), 128), dtype=np.uint16)])
        x = chunk.reshape(256, 65536)
        q_ref, sx_ref = oracle.quant_act(x)
        q, sx = P.smallm_fp8bs_quant(to_dev_bf16(x))
        torch.cuda.synchronize()
        assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32)), f"scales, groups from {c0}"
        assert np.array_equal(q.cpu().numpy(), q_ref), f"codes, groups from {c0}"
        print(f"  groups {min(c0 + per, len(groups))} of {len(groups)} checked", flush=True)


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


def fused_fn(e8m0):
    return P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm


@pytest.mark.parametrize("N,K", SMALL_SHAPES)
@pytest.mark.parametrize("M", [1, 5, 16, 23, 32])
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_small_shapes_full_output(N, K, M, e8m0):
    note(f"fused small N={N} K={K} M={M} e8m0={e8m0}")
    x = special_x(M, K, seed=N + K + M) if K >= 512 else synthgen.gen_x(M, K, seed=N + M)
    w8, sw, wp, swd = prepared_weight(N, K, seed=7, e8m0=e8m0)
    _, _, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
    y = fused_fn(e8m0)(to_dev_bf16(x), wp, swd)
    torch.cuda.synchronize()
    assert_within_tol(y, ref, what=f"N={N} K={K} M={M} e8m0={e8m0}")


@pytest.mark.parametrize("N,K", FULL_SHAPES)
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_full_shapes_all_m(N, K, e8m0):
    """The pages' shapes at every M of the unit-test list, whole outputs."""
    w8, sw, wp, swd = prepared_weight(N, K, seed=0, copy=0, e8m0=e8m0)
    for M in M_LIST:
        note(f"fused full N={N} K={K} M={M} e8m0={e8m0}")
        x = synthgen.gen_x(M, K, seed=M, outliers=(M % 2 == 1))
        _, _, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
        y = fused_fn(e8m0)(to_dev_bf16(x), wp, swd)
        torch.cuda.synchronize()
        assert_within_tol(y, ref, what=f"N={N} K={K} M={M} e8m0={e8m0}")


# ---- the benchmark's workloads on their own inputs (activations seed 0, weight copies 0..23) ----

def test_config_single_call_m4_4096x2048():
    """M = 4, N = 4096, K = 2048, activations and weights at seed 0 (weight copy 0)."""
    note("config single call M=4 4096x2048 seed 0")
    N, K, M = 4096, 2048, 4
    w8, sw, wp, swd = prepared_weight(N, K, seed=0, copy=0)
    x = synthgen.gen_x(M, K, seed=0)
    q_ref, sx_ref, ref = oracle_ref(x, w8, sw, False, [(0, N)])
    q_dbg = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    sx_dbg = torch.zeros((M, K // 128), dtype=torch.float32, device=DEV)
    y = P.smallm_fp8bs_quant_gemm(to_dev_bf16(x), wp, swd, q_dbg=q_dbg, sx_dbg=sx_dbg)
    torch.cuda.synchronize()
    assert np.array_equal(q_dbg.cpu().numpy(), q_ref)
    assert np.array_equal(sx_dbg.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert_within_tol(y, ref, what="single call")


@pytest.mark.parametrize("copy", [0, 23])
def test_config_m_sweep_5120x4096(copy):
    """N = 5120, K = 4096, M in {1, 4, 8, 16, 32}, activations at seed 0, the first and last of the
    benchmark's 24 weight copies."""
    N, K = 5120, 4096
    w8, sw, wp, swd = prepared_weight(N, K, seed=0, copy=copy)
    for M in (1, 4, 8, 16, 32):
        note(f"config sweep 5120x4096 copy={copy} M={M}")
        x = synthgen.gen_x(M, K, seed=0)
        _, _, ref = oracle_ref(x, w8, sw, False, [(0, N)])
        y = P.smallm_fp8bs_quant_gemm(to_dev_bf16(x), wp, swd)
        torch.cuda.synchronize()
        assert_within_tol(y, ref, what=f"5120x4096 copy {copy} M={M}")


@pytest.mark.parametrize("N,K", [(4608, 4096), (4096, 2048)])
def test_config_outlier_rows_graph_replay(N, K):
    """M in {1, 4, 8, 16, 32} with 5 % outlier rows, the calls replayed from a captured HIP graph
    over three weight copies; every replayed output is checked against the oracle."""
    copies = (0, 1, 2)
    ws = [prepared_weight_nocache(N, K, seed=0, copy=c) for c in copies]
    for M in (1, 4, 8, 16, 32):
        note(f"config outliers graph N={N} K={K} M={M}")
        x = synthgen.gen_x(M, K, seed=0, outliers=True)
        xd = to_dev_bf16(x)
        refs = [oracle_ref(x, w8, sw, False, [(0, N)])[2] for (w8, sw, _, _) in ws]
        ys = [torch.zeros((M, N), dtype=torch.bfloat16, device=DEV) for _ in copies]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for (_, _, wp, swd), y in zip(ws, ys):
                P.smallm_fp8bs_quant_gemm(xd, wp, swd, y=y)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for (_, _, wp, swd), y in zip(ws, ys):
                P.smallm_fp8bs_quant_gemm(xd, wp, swd, y=y)
        for rep in range(2):
            for y in ys:
                y.fill_(-5.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for c, y, ref in zip(copies, ys, refs):
                assert_within_tol(y, ref, what=f"N={N} K={K} M={M} copy {c} replay {rep}")
            _ = (xd.float() * 3).sum()     # unrelated eager work between replays
            torch.cuda.synchronize()


@pytest.mark.parametrize("M", [33, 48, 64, 128, 256])
def test_config_beyond_small_m(M):
    """M = 33 .. 256 on 4096 x 2048: the fused entry and quant + the GEMM on pre-quantised input."""
    note(f"config beyond small M={M}")
    N, K = 4096, 2048
    w8, sw, wp, swd = prepared_weight(N, K, seed=0)
    x = synthgen.gen_x(M, K, seed=0)
    q_ref, _, ref = oracle_ref(x, w8, sw, False, [(0, N)])
    y = P.smallm_fp8bs_quant_gemm(to_dev_bf16(x), wp, swd)
    q, sx = P.smallm_fp8bs_quant(to_dev_bf16(x))
    y2 = P.smallm_fp8bs_gemm(q, sx, wp, swd)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert_within_tol(y, ref, what=f"fused M={M}")
    assert_within_tol(y2, ref, what=f"prequantised M={M}")


@pytest.mark.parametrize("e8m0", [False, True])
@pytest.mark.parametrize("M", [33, 64, 128, 256])
@pytest.mark.parametrize("N,K", [(5120, 4096), (4608, 4096), (4096, 2048), (2048, 4096)])
def test_beyond_small_m_every_layout(N, K, M, e8m0):
    """Past the small-M cap on each packed layout (16-column groups; 16 + 4, 16 + 2 and 8-column
    remainder groups): the fused entry (quantisation into a workspace, then the tiled GEMM) over
    the full output against the oracle, bit-equal to the two launches through the C entry points,
    and the fused kernel's 32-row chunks (no workspace) within the same tolerance."""
    note(f"beyond small M N={N} K={K} M={M} e8m0={e8m0}")
    w8, sw, wp, swd = prepared_weight(N, K, seed=9, e8m0=e8m0)
    x = synthgen.gen_x(M, K, seed=M + 3, outliers=True)
    q_ref, sx_ref, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
    xd = to_dev_bf16(x)
    y = fused_fn(e8m0)(xd, wp, swd)
    qf = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
    gf = P.smallm_fp8bs_gemm_e8m0 if e8m0 else P.smallm_fp8bs_gemm
    q, sx = qf(xd)
    y2 = gf(q, sx, wp, swd)
    # the fused kernel in 32-row chunks: the C entry without a workspace
    y3 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    fn = P.lib().smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.lib().smallm_fp8bs_quant_gemm
    st = fn(P._ptr(xd), xd.stride(0), P._ptr(wp), P.smallm_fp8bs_weight_layout_id(N, K), P._ptr(swd), P._ptr(y3),
            N, M, N, K, None, None, P._stream())
    assert st == 0
    torch.cuda.synchronize()
    assert P.smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K) > 0
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert_within_tol(y, ref, what=f"fused N={N} K={K} M={M} e8m0={e8m0}")
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert_within_tol(y3, ref, what=f"fused chunks N={N} K={K} M={M} e8m0={e8m0}")


@pytest.mark.parametrize("N,K", [(4096, 2048), (2048, 4096)])
def test_config_e8m0_beside_fp32(N, K):
    """Power-of-two scales (weights rounded, activations rounded up, as e8m0 bytes) at M in
    {1, 8, 32}, and the fp32-scale path on the same activations and master weights."""
    w = synthgen.gen_w(N, K, seed=0, copy=0)
    for M in (1, 8, 32):
        note(f"config e8m0 N={N} K={K} M={M}")
        x = synthgen.gen_x(M, K, seed=0)
        ys = {}
        for e8m0 in (False, True):
            w8, sw = oracle.quant_weight(w, e8m0=e8m0)
            wp = P.smallm_fp8bs_pack_weight(to_dev(w8))
            q_ref, sx_ref, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
            q_dbg = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
            sx_dbg = torch.zeros((M, K // 128), dtype=torch.uint8 if e8m0 else torch.float32, device=DEV)
            y = fused_fn(e8m0)(to_dev_bf16(x), wp, to_dev(sw), q_dbg=q_dbg, sx_dbg=sx_dbg)
            torch.cuda.synchronize()
            assert np.array_equal(q_dbg.cpu().numpy(), q_ref)
            assert np.array_equal(sx_dbg.cpu().numpy().view(np.uint8), sx_ref.view(np.uint8))
            assert_within_tol(y, ref, what=f"N={N} K={K} M={M} e8m0={e8m0}")
            ys[e8m0] = bf16_to_np_f64(y)
        # the two scale types quantise differently; their outputs agree to a few percent of the largest
        rel = np.abs(ys[True] - ys[False]).max() / np.abs(ys[False]).max()
        assert rel < 0.15, rel


# ---- every variant of the packed layout and the launch ----

# (N, K): 16-column groups only (N a multiple of 4096, and the fallback), 16-column groups plus a
# remainder of 2 / 4 / 8 columns, a remainder only; rounds of 1, 2 and 4 K blocks per wave; many
# rounds per wave (K = 16384) and a ragged last round (97 K blocks)
PLAN_SHAPES = [(8192, 256), (384, 640), (4608, 640), (5120, 1024), (6144, 1024), (4608, 4096), (1024, 2048),
               (512, 4096), (2048, 16384), (1024, 12416), (5120, 2048), (2560, 1536)]


@pytest.mark.parametrize("N,K", PLAN_SHAPES)
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_launch_plans(N, K, e8m0):
    w8, sw, wp, swd = prepared_weight(N, K, seed=11, e8m0=e8m0)
    for M in (1, 7, 16, 17, 32):
        note(f"plan N={N} K={K} layout={P.weight_layout(N, K)} M={M} e8m0={e8m0}")
        x = special_x(M, K, seed=M + N) if K >= 512 else synthgen.gen_x(M, K, seed=M + N)
        _, _, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
        y = fused_fn(e8m0)(to_dev_bf16(x), wp, swd)
        torch.cuda.synchronize()
        assert_within_tol(y, ref, what=f"N={N} K={K} M={M} e8m0={e8m0}")


@pytest.mark.parametrize("N,K", [(512, 4096), (1024, 4096), (2048, 4096), (5120, 4096)])
@pytest.mark.parametrize("e8m0", [False, True])
def test_huge_group_over_zero_weight_block(N, K, e8m0):
    """A row whose one activation group has an amax near the bf16 maximum sits over a weight block
    that is all zero; the other groups and blocks are ordinary.  In the remainder fragments, which
    chain several K blocks in one MFMA, the huge group's products with the other blocks' columns must
    contribute nothing: the true contribution of that group is exactly zero."""
    note(f"huge group over zero block N={N} K={K} e8m0={e8m0}")
    lay = P.weight_layout(N, K)
    w = synthgen.gen_w(N, K, seed=13, copy=0)
    kb_huge = 2
    # the zero block: the remainder columns' first 128-row block (or block 0 without a remainder)
    n0 = 16 * lay["NA"] * P.smallm_fp8bs_launch_plan(1, N, K)["nwg"] if lay["CB"] else 0
    n0 = n0 // 128 * 128
    w[n0:n0 + 128, kb_huge * 128:(kb_huge + 1) * 128] = 0.0
    w8, sw = oracle.quant_weight(w, e8m0=e8m0)
    wp = P.smallm_fp8bs_pack_weight(to_dev(w8))
    for M in (1, 3):
        x = synthgen.gen_x(M, K, seed=17)
        big = synthgen.f32_to_bf16_bits(
            synthgen.bf16_bits_to_f32(x[0, kb_huge * 128:(kb_huge + 1) * 128]) * np.float32(1e36))
        x[0, kb_huge * 128:(kb_huge + 1) * 128] = big
        assert np.isfinite(synthgen.bf16_bits_to_f32(x)).all()
        _, _, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
        y = fused_fn(e8m0)(to_dev_bf16(x), wp, to_dev(sw))
        torch.cuda.synchronize()
        # columns over the zero block: compared on their own scale as well
        assert_within_tol(y, ref, what=f"N={N} K={K} M={M} e8m0={e8m0}")
        cols = slice(n0, n0 + 128)
        assert_within_tol(y[:, cols], ref[:, cols], what=f"zero-block columns N={N} K={K} M={M} e8m0={e8m0}")


@pytest.mark.parametrize("e8m0", [False, True])
@pytest.mark.parametrize("M", [1, 8, 17, 32])
def test_two_kernel_path(M, e8m0):
    note(f"two-kernel M={M} e8m0={e8m0}")
    N, K = 2048, 4096
    w8, sw, wp, swd = prepared_weight(N, K, seed=2, e8m0=e8m0)
    x = special_x(M, K, seed=M + 5)
    q_ref, sx_ref, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
    qf = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
    gf = P.smallm_fp8bs_gemm_e8m0 if e8m0 else P.smallm_fp8bs_gemm
    q, sx = qf(to_dev_bf16(x))
    y = gf(q, sx, wp, swd)
    yf = fused_fn(e8m0)(to_dev_bf16(x), wp, swd)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert_within_tol(y, ref, what=f"two-kernel M={M}")
    # same quantised operands, same kernel arithmetic: the two paths agree bit for bit
    assert torch.equal(y.view(torch.int16), yf.view(torch.int16))


PREQ_CASES = [
    # (N, K, M): the GEMM on pre-quantised input beyond the small-M range
    (384, 640, 33), (384, 640, 100), (4096, 128, 64), (4096, 2048, 48), (4096, 2048, 256),
    (4096, 4736, 77), (5120, 4096, 40), (2048, 4096, 96), (4608, 4096, 65), (4608, 640, 200),
    (5120, 2048, 129), (1024, 12416, 48),
    # the largest K the tiled kernel takes (128 K blocks: four batches of row scales at 64 rows)
    (256, 16384, 256), (384, 16384, 33),
]


@pytest.mark.parametrize("N,K,M", PREQ_CASES)
@pytest.mark.parametrize("e8m0", [False, True])
def test_prequantised_gemm_beyond_small_m(N, K, M, e8m0):
    """GEMM on pre-quantised input beyond M = 32, against the oracle GEMM on the oracle's bytes,
    with padded row pitches (padding never written)."""
    note(f"prequantised N={N} K={K} M={M} e8m0={e8m0}")
    w8, sw, wp, swd = prepared_weight(N, K, seed=6, e8m0=e8m0)
    x = special_x(M, K, seed=M + N)
    q_ref, sx_ref, ref = oracle_ref(x, w8, sw, e8m0, [(0, N)])
    qf = P.smallm_fp8bs_quant_e8m0 if e8m0 else P.smallm_fp8bs_quant
    gf = P.smallm_fp8bs_gemm_e8m0 if e8m0 else P.smallm_fp8bs_gemm
    q, sx = qf(to_dev_bf16(x))
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    gf(q, sx, wp, swd, y=y)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert_within_tol(y, ref, what=f"prequantised N={N} K={K} M={M}")
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
