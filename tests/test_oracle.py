"""Pins for the CPU oracle (runs without a GPU).

Every check here ties the oracle to something other than itself: the hand-worked fixture in
tests/golden (derived from the e4m3 definition and the 1x128 / 128x128 group rules of the
pages), torch's independent float8_e4m3fn cast, brute-force nearest-value search, exact
rational arithmetic, numpy matmul of dequantised operands, closed forms and invariants.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_handworked.json")


# ---------------------------------------------------------------------------------------------
# helpers independent of the oracle
# ---------------------------------------------------------------------------------------------

def parse_value(s: str) -> Fraction:
    s = s.strip()
    neg = s.startswith("-")
    body = s[1:] if neg else s
    if "2^" in body:
        if "*" in body:
            a, b = body.split("*")
            v = Fraction(a) * Fraction(2) ** int(b[2:])
        else:
            v = Fraction(2) ** int(body[2:])
    else:
        v = Fraction(body)
    return -v if neg else v


def is_negative_zero_str(s: str) -> bool:
    return s.strip() == "-0"


def bf16_bits_of(v: Fraction, neg_zero=False) -> int:
    """Exact bf16 bit pattern of a value that must be representable in bf16."""
    f = np.float32(float(v))
    if neg_zero:
        f = np.float32(-0.0)
    bits = int(np.array([f], dtype=np.float32).view(np.uint32)[0])
    assert bits & 0xFFFF == 0, f"{v} not exactly representable in bf16"
    return bits >> 16


def e4m3_table_torch() -> np.ndarray:
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def brute_force_e4m3(v: float) -> int:
    """Nearest finite e4m3 value by exhaustive search over all codes, ties to the even code,
    saturating; independent of the oracle's binary search."""
    table = e4m3_table_torch()
    a = abs(v)
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    if a >= 448.0:
        return sign | 0x7E
    best, bestd = None, None
    for c in range(0x7F):  # non-negative finite codes
        d = abs(table[c] - a)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return sign | best


def round_fraction_to_f32(v: Fraction) -> Fraction:
    """Exact IEEE binary32 round-to-nearest-even of a rational (normal and subnormal range)."""
    if v == 0:
        return Fraction(0)
    neg = v < 0
    a = -v if neg else v
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    return -r if neg else r


# ---------------------------------------------------------------------------------------------
# codec
# ---------------------------------------------------------------------------------------------

def test_decode_matches_torch_all_codes(oracle_lib):
    t = e4m3_table_torch()
    for c in range(256):
        d = oracle.e4m3_decode(c)
        if (c & 0x7F) == 0x7F:
            assert math.isnan(d) and math.isnan(t[c])
        else:
            assert d == t[c], hex(c)
            assert math.copysign(1.0, d) == math.copysign(1.0, t[c])


def test_roundtrip_every_finite_code(oracle_lib):
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)


def test_encode_matches_torch_on_every_bf16(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = synthgen.bf16_bits_to_f32(bits)
    fin = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    v = vals[fin]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(f)) for f in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_encode_ties_and_neighbours_vs_brute_force_and_torch(oracle_lib):
    t = e4m3_table_torch()
    pts = []
    for c in range(0x7E):
        mid = (t[c] + t[c + 1]) / 2.0
        m32 = np.float32(mid)
        assert float(m32) == mid  # every midpoint is an fp32 value
        for f in (np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(1000))):
            pts.append(float(f))
            pts.append(-float(f))
    ref = torch.tensor(pts, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for f, r in zip(pts, ref):
        got = oracle.e4m3_encode(f)
        assert got == brute_force_e4m3(f), f
        assert got == r, f


def test_encode_saturates_and_keeps_sign(oracle_lib):
    for f in (448.0, 449.0, 463.99, 464.0, 500.0, 1e6, 3.4e38):
        assert oracle.e4m3_encode(f) == 0x7E
        assert oracle.e4m3_encode(-f) == 0xFE
    for f in (-0.0, -1e-30, -2.0 ** -10, -1e-4):
        assert oracle.e4m3_encode(f) == 0x80


def test_golden_encode_cases(oracle_lib):
    g = json.load(open(GOLDEN))
    for case in g["encode"]:
        v = parse_value(case["value"])
        f = -0.0 if is_negative_zero_str(case["value"]) else float(v)
        assert oracle.e4m3_encode(f) == int(case["code"], 16), case


def test_bf16_from_double_ties_and_double_rounding(oracle_lib):
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80        # tie -> even (down)
    assert oracle.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82    # tie -> even (up)
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # no double rounding
    assert oracle.bf16_from_double(-2.5) == 0xC020
    assert oracle.bf16_from_double(0.0) == 0x0000
    assert oracle.bf16_from_double(-0.0) == 0x8000
    rng = np.random.default_rng(5)
    for v in rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000):
        b = oracle.bf16_from_double(float(v))
        got = Fraction(float(synthgen.bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0]))
        fv = Fraction(float(v))
        e = math.frexp(abs(float(v)))[1]
        half_ulp = Fraction(2) ** (e - 8) / 2
        assert abs(got - fv) <= half_ulp


# ---------------------------------------------------------------------------------------------
# activation quantisation
# ---------------------------------------------------------------------------------------------

def build_group(spec, G=1):
    x = np.zeros((1, 128 * G), dtype=np.uint16)
    fill = spec.get("fill", "0")
    x[:] = bf16_bits_of(parse_value(fill), neg_zero=is_negative_zero_str(fill))
    for k, v in spec.get("set", {}).items():
        x[0, int(k)] = bf16_bits_of(parse_value(v), neg_zero=is_negative_zero_str(v))
    return x


def expected_codes(spec):
    q = np.full(128, int(spec.get("fill", "0x00"), 16), dtype=np.uint8)
    for k, v in spec.get("set", {}).items():
        q[int(k)] = int(v, 16)
    return q


def test_golden_groups_fp32(oracle_lib):
    g = json.load(open(GOLDEN))
    for case in g["groups_fp32"]:
        x = build_group(case["x"])
        q, sx = oracle.quant_act(x)
        assert Fraction(float(sx[0, 0])) == parse_value(case["sx"]), case["name"]
        assert np.array_equal(q[0], expected_codes(case["q"])), case["name"]


def test_golden_groups_e8m0(oracle_lib):
    g = json.load(open(GOLDEN))
    for case in g["groups_e8m0"]:
        x = build_group(case["x"])
        q, sx = oracle.quant_act(x, e8m0=True)
        assert sx[0, 0] == int(case["sx_byte"], 16), case["name"]
        assert np.array_equal(q[0], expected_codes(case["q"])), case["name"]


def exact_quant_group_fp32(xvals):
    """Exact-rational rendering of the 1x128 rule: sx = RN32(amax/448), q = enc(RN32(x/sx))."""
    amax = max(abs(Fraction(float(v))) for v in xvals)
    if amax == 0:
        return Fraction(0), [0x80 if math.copysign(1.0, float(v)) < 0 else 0 for v in xvals]
    sx = round_fraction_to_f32(amax / 448)
    codes = []
    for v in xvals:
        quo = round_fraction_to_f32(Fraction(float(v)) / sx)
        fq = float(quo)
        if quo == 0 and math.copysign(1.0, float(v)) < 0:
            fq = -0.0
        codes.append(brute_force_e4m3(fq))
    return sx, codes


def test_quant_fp32_vs_exact_rationals(oracle_lib):
    x = synthgen.gen_x(2, 256, seed=11)
    q, sx = oracle.quant_act(x)
    xf = synthgen.bf16_bits_to_f32(x)
    for m in range(2):
        for g in range(2):
            s_ref, codes = exact_quant_group_fp32(xf[m, 128 * g:128 * g + 128])
            assert Fraction(float(sx[m, g])) == s_ref
            assert list(q[m, 128 * g:128 * g + 128]) == codes


def test_quant_fp32_vs_torch_cast(oracle_lib):
    for seed, outl in ((0, False), (3, True), (7, True)):
        x = synthgen.gen_x(9, 1024, seed=seed, outliers=outl)
        q, sx = oracle.quant_act(x)
        xt = torch.from_numpy(synthgen.bf16_bits_to_f32(x).copy()).reshape(9, 8, 128)
        amax = xt.abs().amax(dim=-1, keepdim=True)
        s = amax / 448.0
        qt = (xt / s).to(torch.float8_e4m3fn).view(torch.uint8).reshape(9, 1024).numpy()
        assert np.array_equal(sx, s.reshape(9, 8).numpy())
        assert np.array_equal(q, qt)


def test_quant_division_reading_is_observable(oracle_lib):
    """The quotient is x / sx (one IEEE division), not x * (1/sx): find groups where the two
    readings give different bytes and check the oracle follows the division."""
    x = synthgen.gen_x(32, 4096, seed=1)
    q, sx = oracle.quant_act(x)
    xt = torch.from_numpy(synthgen.bf16_bits_to_f32(x).copy()).reshape(32, 32, 128)
    s = torch.from_numpy(sx.copy()).reshape(32, 32, 1)
    by_div = (xt / s).to(torch.float8_e4m3fn).view(torch.uint8).reshape(32, 4096).numpy()
    by_rcp = (xt * (1.0 / s)).to(torch.float8_e4m3fn).view(torch.uint8).reshape(32, 4096).numpy()
    differ = by_div != by_rcp
    assert differ.sum() > 0
    assert np.array_equal(q[differ], by_div[differ])


def test_quant_invariants(oracle_lib):
    x = synthgen.gen_x(17, 2048, seed=4, outliers=True)
    q, sx = oracle.quant_act(x)
    xf = synthgen.bf16_bits_to_f32(x).astype(np.float64).reshape(17, 16, 128)
    qd = oracle.e4m3_decode_array(q).reshape(17, 16, 128)
    qb = q.reshape(17, 16, 128)
    xbits = x.reshape(17, 16, 128)
    # sign of every code equals the sign bit of its input
    assert np.array_equal(qb >> 7, (xbits >> 15).astype(np.uint8))
    # the amax element of each group encodes to +-448
    idx = np.abs(xf).argmax(axis=-1)
    amax_codes = np.take_along_axis(qb, idx[..., None], axis=-1)[..., 0]
    assert np.all((amax_codes & 0x7F) == 0x7E)
    # reconstruction error within half an e4m3 step of the quotient (plus fp32 rounding)
    quo = xf / sx.astype(np.float64)[..., None]
    step = np.where(np.abs(qd) < 2.0 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(np.abs(qd), 2.0 ** -6))) - 3))
    assert np.all(np.abs(qd - quo) <= step / 2 + np.abs(quo) * 2.0 ** -22)


def test_outlier_groups(oracle_lib):
    x = synthgen.gen_x(16, 1024, seed=2, outliers=True)
    rows = synthgen.outlier_rows(16, seed=2)
    assert len(rows) == 1
    q, sx = oracle.quant_act(x)
    r = rows[0]
    assert np.all(sx[r] == np.float32(1000.0) / np.float32(448.0))
    xf = synthgen.bf16_bits_to_f32(x[r])
    assert np.sum(np.abs(xf) == 1000.0) == 8


def test_e8m0_activation_exponent_all_bf16(oracle_lib):
    """Smallest E with amax <= 448 * 2^E, over every positive finite bf16 amax."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    vals = synthgen.bf16_bits_to_f32(bits).astype(np.float64)
    for a in vals[::7]:
        E = oracle.e8m0_ceil_exponent(float(a))
        if E > -127:
            assert a <= 448.0 * 2.0 ** E and a > 448.0 * 2.0 ** (E - 1), a
        else:
            assert a <= 448.0 * 2.0 ** -127
        # agrees with ceil(log2(a / 448)) computed in 60-digit decimal
        r = Fraction(float(a)) / 448
        if r.numerator & (r.numerator - 1) == 0 and r.denominator & (r.denominator - 1) == 0:
            c = r.numerator.bit_length() - r.denominator.bit_length()   # exact power of two
        else:
            getcontext().prec = 60
            l2 = (Decimal(float(a)) / Decimal(448)).ln() / Decimal(2).ln()
            c = int(l2.to_integral_value(rounding="ROUND_CEILING"))
        assert E == max(c, -127)


def test_e8m0_activation_quant_exact_scaling(oracle_lib):
    x = synthgen.gen_x(5, 1024, seed=9, outliers=True)
    q, sx = oracle.quant_act(x, e8m0=True)
    xf = synthgen.bf16_bits_to_f32(x).astype(np.float64).reshape(5, 8, 128)
    E = sx.astype(np.int64) - 127
    scaled = xf * np.exp2(-E.astype(np.float64))[..., None]
    assert np.all(np.abs(scaled) <= 448.0)
    ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q.reshape(5, 8, 128), ref)


# ---------------------------------------------------------------------------------------------
# weight quantisation
# ---------------------------------------------------------------------------------------------

def test_weight_quant_fp32_vs_torch(oracle_lib):
    w = synthgen.gen_w(256, 384, seed=0, copy=3)
    w[0:128, 128:256] = 0.0                      # one all-zero block
    w8, sw = oracle.quant_weight(w)
    wt = torch.from_numpy(w).reshape(2, 128, 3, 128).permute(0, 2, 1, 3)
    amax = wt.abs().amax(dim=(-1, -2), keepdim=True)
    s = amax / 448.0
    assert np.array_equal(sw, s.reshape(2, 3).numpy())
    qt = torch.where(s > 0, wt / torch.where(s > 0, s, torch.ones_like(s)), wt * 0.0)
    qt = qt.to(torch.float8_e4m3fn).view(torch.uint8).permute(0, 2, 1, 3).reshape(256, 384).numpy()
    assert np.array_equal(w8, qt)
    assert sw[0, 1] == 0.0 and np.all(w8[0:128, 128:256] == 0)


def test_weight_e8m0_exponent_golden_and_log_domain(oracle_lib):
    g = json.load(open(GOLDEN))
    for case in g["weight_e8m0_exponent"]:
        a = float(np.float32(float(Fraction(case["amax"]))))
        assert oracle.e8m0_round_exponent(a) == case["E"], case
    getcontext().prec = 60
    rng = np.random.default_rng(3)
    for a in np.abs(rng.standard_normal(500).astype(np.float32)) * np.float32(0.05) + np.float32(1e-6):
        E = oracle.e8m0_round_exponent(float(a))
        l2 = (Decimal(float(a)) / Decimal(448)).ln() / Decimal(2).ln()
        assert abs(l2 - E) <= Decimal("0.5"), (a, E, l2)


def test_weight_quant_e8m0_saturates(oracle_lib):
    w = np.zeros((128, 128), dtype=np.float32)
    w[0, 0] = np.float32(0.07)
    w[1, 1] = np.float32(-0.035)
    w8, sw = oracle.quant_weight(w, e8m0=True)
    assert sw[0, 0] == 127 - 13
    assert w8[0, 0] == 0x7E                     # 0.07 * 2^13 = 573.44 -> 448
    assert w8[1, 1] == 0xF9                     # -0.035 * 2^13 = -286.72 -> -288 (step 32)
    e8 = synthgen.gen_w(256, 256, seed=1)
    w8, sw = oracle.quant_weight(e8, e8m0=True)
    wd = oracle.e4m3_decode_array(w8).reshape(2, 128, 2, 128) * np.exp2(
        sw.astype(np.float64) - 127)[:, None, :, None]
    scale = np.repeat(np.repeat(np.exp2(sw.astype(np.float64) - 127), 128, 0), 128, 1)
    scaled = e8.astype(np.float64) / scale
    err = np.abs(wd.reshape(256, 256) - e8)
    ok = np.abs(scaled) <= 448.0
    # unsaturated values: within half an e4m3 step (relative 2^-4, or 2^-10 absolute near zero)
    assert np.all(err[ok] <= np.maximum(np.abs(e8[ok]) * 2.0 ** -4, 2.0 ** -10 * scale[ok]))
    # saturated values decode to exactly +-448 * scale
    assert np.all(np.abs(wd.reshape(256, 256)[~ok]) == 448.0 * scale[~ok])


# ---------------------------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------------------------

def dequant_matmul(q, sx, w8, sw, e8m0=False):
    """Brute force: decode both operands to fp64, apply their scales, numpy matmul."""
    M, K = q.shape
    N = w8.shape[0]
    if e8m0:
        sxf = np.exp2(sx.astype(np.float64) - 127)
        swf = np.exp2(sw.astype(np.float64) - 127)
    else:
        sxf = sx.astype(np.float64)
        swf = sw.astype(np.float64)
    A = oracle.e4m3_decode_array(q) * np.repeat(sxf, 128, axis=1)
    B = oracle.e4m3_decode_array(w8) * np.repeat(np.repeat(swf, 128, axis=0), 128, axis=1)
    return A @ B.T


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 256, 384), (2, 384, 256)])
@pytest.mark.parametrize("e8m0", [False, True])
def test_gemm_vs_dequantised_matmul(oracle_lib, M, N, K, e8m0):
    x = synthgen.gen_x(M, K, seed=M + N)
    w = synthgen.gen_w(N, K, seed=K)
    q, sx = oracle.quant_act(x, e8m0=e8m0)
    w8, sw = oracle.quant_weight(w, e8m0=e8m0)
    ref = oracle.gemm(q, sx, w8, sw, e8m0=e8m0)
    bf = dequant_matmul(q, sx, w8, sw, e8m0=e8m0)
    assert np.allclose(ref, bf, rtol=1e-12, atol=1e-12 * np.abs(bf).max())
    # a transposed or mis-indexed operand would not survive this asymmetric check
    assert not np.allclose(ref[:, :128], dequant_matmul(q, sx, w8[::-1].copy(), sw[::-1].copy(), e8m0)[:, :128])


def test_gemm_closed_form_single_block(oracle_lib):
    """K = 128: Y = sx * sw * sum_k dec(q) dec(w), computed here in exact rationals."""
    x = synthgen.gen_x(2, 128, seed=21)
    w = synthgen.gen_w(128, 128, seed=22)
    q, sx = oracle.quant_act(x)
    w8, sw = oracle.quant_weight(w)
    ref = oracle.gemm(q, sx, w8, sw)
    for m in range(2):
        for n in (0, 5, 127):
            s = sum(Fraction(oracle.e4m3_decode(int(q[m, k]))) * Fraction(oracle.e4m3_decode(int(w8[n, k])))
                    for k in range(128))
            mag = sum(abs(Fraction(oracle.e4m3_decode(int(q[m, k]))) * Fraction(oracle.e4m3_decode(int(w8[n, k]))))
                      for k in range(128))
            scale = Fraction(float(sx[m, 0])) * Fraction(float(sw[0, 0]))
            exact = scale * s
            # fp64 accumulation of 128 terms: the error stays far below 2^-44 of the absolute sum
            assert abs(Fraction(ref[m, n]) - exact) <= scale * mag * Fraction(1, 2 ** 44)


def test_gemm_unit_weights_gives_row_sums(oracle_lib):
    x = synthgen.gen_x(3, 384, seed=8)
    q, sx = oracle.quant_act(x)
    w8 = np.full((128, 384), 0x38, dtype=np.uint8)      # every weight 1.0
    sw = np.ones((1, 3), dtype=np.float32)
    ref = oracle.gemm(q, sx, w8, sw)
    rows = (oracle.e4m3_decode_array(q) * np.repeat(sx.astype(np.float64), 128, axis=1)).sum(axis=1)
    assert np.allclose(ref, rows[:, None], rtol=1e-13)
    assert np.all(ref == ref[:, :1])


def test_gemm_e8m0_is_exact_dyadic(oracle_lib):
    x = synthgen.gen_x(2, 256, seed=31)
    w = synthgen.gen_w(128, 256, seed=32)
    q, sx = oracle.quant_act(x, e8m0=True)
    w8, sw = oracle.quant_weight(w, e8m0=True)
    ref = oracle.gemm(q, sx, w8, sw, e8m0=True)
    for m in range(2):
        for n in (0, 77):
            exact = sum(Fraction(oracle.e4m3_decode(int(q[m, k]))) * Fraction(2) ** (int(sx[m, k // 128]) - 127)
                        * Fraction(oracle.e4m3_decode(int(w8[n, k]))) * Fraction(2) ** (int(sw[0, k // 128]) - 127)
                        for k in range(256))
            assert Fraction(ref[m, n]) == exact


def test_quant_gemm_column_window_and_bf16(oracle_lib):
    x = synthgen.gen_x(4, 256, seed=41)
    w = synthgen.gen_w(384, 256, seed=42)
    w8, sw = oracle.quant_weight(w)
    y, ref, q, sx = oracle.quant_gemm(x, w8, sw)
    q2, sx2 = oracle.quant_act(x)
    assert np.array_equal(q, q2) and np.array_equal(sx, sx2)
    full = oracle.gemm(q2, sx2, w8, sw)
    assert np.array_equal(ref, full)
    assert np.array_equal(y, oracle.round_bf16(full))
    y2, ref2, _, _ = oracle.quant_gemm(x, w8, sw, n0=128, n1=256, threads=2)
    assert np.array_equal(ref2[:, 128:256], full[:, 128:256])
    assert np.all(ref2[:, :128] == 0) and np.all(ref2[:, 256:] == 0)


# ---------------------------------------------------------------------------------------------
# RMSNorm producer (mean square exact then rounded to fp32, correctly rounded fp32 rsqrt,
# fp32 products, bf16 output, then the 1x128 quantisation)
# ---------------------------------------------------------------------------------------------

def round_fraction_to_bf16_bits(v: Fraction) -> int:
    """Exact bf16 round-to-nearest-even of a rational (8 significant bits, quantum 2^-133 at the
    bottom), as a bit pattern; independent of the oracle's bf16 rounding."""
    neg = v < 0
    a = -v if neg else v
    if a == 0:
        return 0x8000 if neg else 0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    bits = int(np.array([np.float32(float(r))], dtype=np.float32).view(np.uint32)[0]) >> 16
    return bits | (0x8000 if neg else 0)


def decimal_rsqrt_f32(v: float) -> Fraction:
    """RN32(1 / sqrt(v)) from an 80-digit decimal square root and exact rational rounding."""
    getcontext().prec = 80
    d = Decimal(1) / Decimal(v).sqrt()
    return round_fraction_to_f32(Fraction(d))


def rmsnorm_by_fractions(x_bits, w_bits, eps32):
    """The producer's RMSNorm in exact rationals, row by row (slow; small shapes only)."""
    M, H = x_bits.shape
    xs = synthgen.bf16_bits_to_f32(x_bits)
    ws = synthgen.bf16_bits_to_f32(w_bits)
    y = np.zeros((M, H), dtype=np.uint16)
    for m in range(M):
        ss = sum(Fraction(float(a)) ** 2 for a in xs[m])
        ms = round_fraction_to_f32(ss / H)
        v = round_fraction_to_f32(ms + Fraction(float(eps32)))
        r = decimal_rsqrt_f32(float(v))
        for i in range(H):
            t = round_fraction_to_f32(Fraction(float(xs[m, i])) * r)
            u = round_fraction_to_f32(t * Fraction(float(ws[i])))
            y[m, i] = round_fraction_to_bf16_bits(u)
            if u == 0 and math.copysign(1.0, float(xs[m, i])) * math.copysign(1.0, float(ws[i])) < 0:
                y[m, i] = 0x8000
    return y


def test_rmsnorm_unit_row_returns_the_weight(oracle_lib):
    # all-ones row: mean square 1, eps far below half an ulp of 1, so r = 1 and y = w exactly
    rng = np.random.default_rng([5, 1])
    w = synthgen.f32_to_bf16_bits(rng.normal(0.0, 2.0, 256).astype(np.float32))
    x = np.full((2, 256), 0x3F80, dtype=np.uint16)
    y, r = oracle.rmsnorm(x, w, 2.0 ** -40)
    assert np.all(r == 1.0)
    assert np.array_equal(y, np.stack([w, w]))


def test_rmsnorm_hand_worked_3_4_row(oracle_lib):
    # x = (3, 4, 0, ..., 0), H = 128: sum of squares 25, mean 25/128 = 0.1953125 exactly;
    # eps = 2^-30 is below half an ulp (2^-27) of it, so v = 25/128 and r = RN32(sqrt(5.12))
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 0] = 0x4040   # 3.0
    x[0, 1] = 0x4080   # 4.0
    w = np.full(128, 0x3F80, dtype=np.uint16)
    assert oracle.mean_square_f32(x[0]) == 0.1953125
    y, r = oracle.rmsnorm(x, w, 2.0 ** -30)
    getcontext().prec = 80
    r_ref = round_fraction_to_f32(Fraction(Decimal("5.12").sqrt()))
    assert Fraction(float(r[0])) == r_ref
    assert float(r[0]) == pytest.approx(2.2627417, abs=3e-7)
    assert y[0, 0] == round_fraction_to_bf16_bits(round_fraction_to_f32(3 * r_ref))
    assert y[0, 1] == round_fraction_to_bf16_bits(round_fraction_to_f32(4 * r_ref))
    assert y[0, 0] == 0x40D9 and y[0, 1] == 0x4111   # 6.78125 and 9.0625
    assert np.all(y[0, 2:] == 0)


@pytest.mark.parametrize("H", [128, 384])
def test_rmsnorm_matches_exact_rational_reference(oracle_lib, H):
    rng = np.random.default_rng([7, H])
    x = synthgen.gen_x(3, H, seed=H, outliers=True)
    x[2, :] = synthgen.f32_to_bf16_bits(synthgen.bf16_bits_to_f32(x[2, :]) * np.float32(1e-20))
    w = synthgen.f32_to_bf16_bits(rng.normal(1.0, 0.3, H).astype(np.float32))
    eps = np.float32(1e-6)
    y, _ = oracle.rmsnorm(x, w, float(eps))
    assert np.array_equal(y, rmsnorm_by_fractions(x, w, eps))


def test_rmsnorm_rsqrt_against_decimal_on_edge_values(oracle_lib):
    vals = [2.0 ** -126, 2.0 ** -20, 0.1953125, 1.0, 2.0, 3.0, 1e-6, 12345.678, 2.0 ** 100,
            float(np.float32(3.4e38))]
    rng = np.random.default_rng([9, 9])
    vals += [float(np.float32(v)) for v in rng.uniform(1e-7, 1e7, 40)]
    for v in vals:
        v = float(np.float32(v))
        assert Fraction(oracle.rsqrt_f32(v)) == decimal_rsqrt_f32(v), v


def test_rmsnorm_permutation_and_power_of_two_scale_invariance(oracle_lib):
    rng = np.random.default_rng([11, 2])
    x = synthgen.gen_x(4, 512, seed=3)
    w = synthgen.f32_to_bf16_bits(rng.normal(1.0, 0.5, 512).astype(np.float32))
    y, _ = oracle.rmsnorm(x, w, 1e-6)
    perm = rng.permutation(512)
    yp, _ = oracle.rmsnorm(np.ascontiguousarray(x[:, perm]), w[perm], 1e-6)
    assert np.array_equal(yp, y[:, perm])            # the mean is exact: order does not matter
    xs = synthgen.f32_to_bf16_bits(synthgen.bf16_bits_to_f32(x) * np.float32(32.0))
    ys, _ = oracle.rmsnorm(xs, w, 1e-6 * 1024.0)
    assert np.array_equal(ys, y)                      # x * 2^5 with eps * 2^10: same output


def test_rmsnorm_quant_zero_row_keeps_signs(oracle_lib):
    x = np.zeros((1, 256), dtype=np.uint16)
    x[0, 1::2] = 0x8000                               # -0.0 at odd positions
    w = np.full(256, 0x3F80, dtype=np.uint16)
    w[::4] = 0xBF80                                   # -1.0 at every fourth position
    y, q, sx = oracle.rmsnorm_quant(x, w, 1e-6)
    sign = (np.arange(256) % 2 == 1) ^ (np.arange(256) % 4 == 0)
    assert np.array_equal(y[0], np.where(sign, 0x8000, 0).astype(np.uint16))
    assert np.array_equal(q[0], np.where(sign, 0x80, 0).astype(np.uint8))
    assert np.all(sx == 0)
    _, q8, sx8 = oracle.rmsnorm_quant(x, w, 1e-6, e8m0=True)
    assert np.array_equal(q8[0], q[0]) and np.all(sx8 == 0)   # E = -127 for an all-zero group
