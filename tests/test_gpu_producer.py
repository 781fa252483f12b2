"""GPU parity of the producer (RMSNorm with the per-1x128 quantisation of its bf16 output)
against the CPU oracle, and of the producer followed by the GEMM on pre-quantised input.

y (bf16), q (e4m3) and sx (fp32 bits or e8m0 bytes) must be identical to the oracle's.  The
oracle takes the mean square exactly; the kernel sums exact squares in fp64 per lane and as
double-double sums across lanes, so the two can differ only for a row whose exact mean lies
within about 2^-48 (relative) of an fp32 rounding boundary.  Every test row is checked to be
far from that (a margin of 2^-40, from the correctly rounded fp64 sum), so the comparison is
exact.  The GEMM output is held to the same tolerance as the fused path.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import precision_gemm_x128_amd as P
import synthgen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_TOL = 8e-3
ABS_TOL_FRAC = 1e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16).copy()).to(DEV).view(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def producer_inputs(M, H, seed):
    """gen_x rows (outlier rows included) plus special rows: all zeros with signed zeros, a
    single non-zero value, tiny values (bf16 subnormals), large values, one huge outlier."""
    x = synthgen.gen_x(M, H, seed=seed, outliers=True)
    f = synthgen.bf16_bits_to_f32(x)
    specials = [
        lambda r: np.where(np.arange(H) % 3 == 0, 0x8000, 0).astype(np.uint16),
        lambda r: np.where(np.arange(H) == H // 2, 0x4040, 0).astype(np.uint16),
        lambda r: synthgen.f32_to_bf16_bits(f[r] * np.float32(1e-39)),
        lambda r: synthgen.f32_to_bf16_bits(f[r] * np.float32(1e15)),
        lambda r: np.where(np.arange(H) == 7, 0x4B00, x[r]).astype(np.uint16),   # 8388608 amid O(1)
    ]
    for i, mk in enumerate(specials):
        if i + 1 < M:
            x[i + 1] = mk(i + 1)
    rng = np.random.default_rng([seed, 77])
    w = synthgen.f32_to_bf16_bits(rng.normal(1.0, 0.3, H).astype(np.float32))
    w[::97] = synthgen.f32_to_bf16_bits(-np.abs(synthgen.bf16_bits_to_f32(w[::97])))
    return x, w


def assert_rows_clear_of_fp32_boundaries(x):
    """The exact mean square of every row is at least 2^-40 (relative) away from any fp32
    rounding boundary (checked on the correctly rounded fp64 sum, whose error is 2^-53)."""
    H = x.shape[1]
    xf = synthgen.bf16_bits_to_f32(x).astype(np.float64)
    for m in range(x.shape[0]):
        mean = math.fsum((xf[m] * xf[m]).tolist()) / H
        if mean == 0.0 or mean < 2.0 ** -120:
            continue
        e = math.frexp(mean)[1] - 1                        # 2^e <= mean < 2^(e+1)
        ulp = 2.0 ** (e - 23)
        k = mean / ulp                                     # midpoints at k + 1/2
        d = abs((k - math.floor(k)) - 0.5) * ulp / mean
        assert d > 2.0 ** -40, f"row {m}: mean square within {d:.3g} of an fp32 boundary"


@pytest.mark.parametrize("M,H", [(1, 4096), (4, 2048), (7, 128), (17, 7168), (32, 4096), (33, 16384),
                                 (300, 1024)])
@pytest.mark.parametrize("e8m0", [False, True])
def test_rmsnorm_quant_bitexact(M, H, e8m0):
    note(f"rmsnorm_quant M={M} H={H} e8m0={e8m0}")
    x, w = producer_inputs(M, H, seed=M * 31 + H)
    assert_rows_clear_of_fp32_boundaries(x)
    eps = 1e-6
    y_ref, q_ref, sx_ref = oracle.rmsnorm_quant(x, w, eps, e8m0=e8m0)
    fn = P.smallm_fp8bs_rmsnorm_quant_e8m0 if e8m0 else P.smallm_fp8bs_rmsnorm_quant
    y, q, sx = fn(to_dev_bf16(x), to_dev_bf16(w), eps)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), y_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy().view(np.uint8 if e8m0 else np.uint32),
                          sx_ref.view(np.uint8 if e8m0 else np.uint32))


def test_rmsnorm_only_and_padded_pitches():
    """q = NULL: a plain RMSNorm (no quantisation written).  Row pitches beyond H: the padding
    columns of y and q are never written."""
    note("rmsnorm only / padded pitches")
    M, H = 5, 2048
    x, w = producer_inputs(M, H, seed=5)
    assert_rows_clear_of_fp32_boundaries(x)
    y_ref, q_ref, sx_ref = oracle.rmsnorm_quant(x, w, 1e-5)
    xp = torch.zeros((M, H + 64), dtype=torch.bfloat16, device=DEV)
    xp[:, :H] = to_dev_bf16(x)
    yb = torch.full((M, H + 128), 7.0, dtype=torch.bfloat16, device=DEV)
    y, q, sx = P.smallm_fp8bs_rmsnorm_quant(xp[:, :H], to_dev_bf16(w), 1e-5, y=yb[:, :H], emit_q=False)
    torch.cuda.synchronize()
    assert q is None and sx is None
    assert np.array_equal(bits(yb[:, :H].contiguous()), y_ref)
    assert torch.all(yb[:, H:] == 7.0)
    qb = torch.full((M, H + 32), 0x5A, dtype=torch.uint8, device=DEV)
    sxb = torch.zeros((M, H // 128), dtype=torch.float32, device=DEV)
    P.smallm_fp8bs_rmsnorm_quant(xp[:, :H], to_dev_bf16(w), 1e-5, q=qb[:, :H], sx=sxb, emit_y=False)
    torch.cuda.synchronize()
    assert np.array_equal(qb[:, :H].cpu().numpy(), q_ref)
    assert torch.all(qb[:, H:] == 0x5A)
    assert np.array_equal(sxb.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))


def test_rmsnorm_quant_graph_replay_bitwise():
    note("rmsnorm_quant graph replay")
    M, H = 8, 4096
    x, w = producer_inputs(M, H, seed=9)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    y0, q0, s0 = P.smallm_fp8bs_rmsnorm_quant(xd, wd, 1e-6)
    torch.cuda.synchronize()
    y, q, s = torch.empty_like(y0), torch.empty_like(q0), torch.empty_like(s0)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        P.smallm_fp8bs_rmsnorm_quant(xd, wd, 1e-6, y=y, q=q, sx=s)
    torch.cuda.current_stream().wait_stream(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.smallm_fp8bs_rmsnorm_quant(xd, wd, 1e-6, y=y, q=q, sx=s)
    for rep in range(4):
        y.zero_(); q.zero_(); s.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), rep
        assert torch.equal(q, q0) and torch.equal(s.view(torch.int32), s0.view(torch.int32)), rep


@pytest.mark.parametrize("M", [1, 16, 32])
@pytest.mark.parametrize("e8m0", [False, True])
def test_producer_then_prequantised_gemm(M, e8m0):
    """The producer's q and sx feed the GEMM on pre-quantised input (the consumer): the output
    is within tolerance of the oracle's GEMM on the oracle's producer bytes, and the fused path
    on the producer's y gives the same quantised operands."""
    note(f"producer -> gemm M={M} e8m0={e8m0}")
    N, K = 1024, 4096
    x, wn = producer_inputs(M, K, seed=40 + M)
    assert_rows_clear_of_fp32_boundaries(x)
    y_ref, q_ref, sx_ref = oracle.rmsnorm_quant(x, wn, 1e-6, e8m0=e8m0)
    wt = synthgen.gen_w(N, K, seed=8)
    w8, sw = oracle.quant_weight(wt, e8m0=e8m0)
    wp = P.smallm_fp8bs_pack_weight(torch.from_numpy(w8).to(DEV))
    swd = torch.from_numpy(sw).to(DEV)
    prod = P.smallm_fp8bs_rmsnorm_quant_e8m0 if e8m0 else P.smallm_fp8bs_rmsnorm_quant
    y, q, sx = prod(to_dev_bf16(x), to_dev_bf16(wn), 1e-6)
    gemm = P.smallm_fp8bs_gemm_e8m0 if e8m0 else P.smallm_fp8bs_gemm
    out = gemm(q, sx, wp, swd)
    fused = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    q_dbg = torch.zeros_like(q)
    sx_dbg = torch.zeros_like(sx)
    out_f = fused(y, wp, swd, q_dbg=q_dbg, sx_dbg=sx_dbg)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert torch.equal(q_dbg, q) and torch.equal(sx_dbg.view(torch.uint8), sx.view(torch.uint8))
    ref = oracle.gemm(q_ref, sx_ref, w8, sw, e8m0=e8m0)
    for o, what in ((out, "pre-quantised"), (out_f, "fused")):
        yv = o.float().cpu().numpy().astype(np.float64)
        tol = REL_TOL * np.abs(ref) + ABS_TOL_FRAC * np.abs(ref).max()
        assert np.isfinite(yv).all() and not (np.abs(yv - ref) > tol).any(), what


def test_producer_binding_errors():
    note("producer binding errors")
    x = to_dev_bf16(synthgen.gen_x(2, 256, seed=1))
    w = to_dev_bf16(np.full(256, 0x3F80, dtype=np.uint16))
    with pytest.raises(P.SmallmError) as e:
        P.smallm_fp8bs_rmsnorm_quant(x, w, 0.0)
    assert e.value.status == P.SMALLM_ERR_INVALID
    with pytest.raises(ValueError):
        P.smallm_fp8bs_rmsnorm_quant(x, w[:128], 1e-6)
    with pytest.raises(TypeError):
        P.smallm_fp8bs_rmsnorm_quant(x.to(torch.float16), w, 1e-6)
