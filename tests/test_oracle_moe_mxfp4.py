"""Pins for the oracle of the MoE layer with MXFP4 expert weights (runs without a GPU).

* The e2m1 and e8m0 decoders against the values the OCP Microscaling Formats (MX) v1.0
  specification tabulates (tests/golden/mxfp4_handworked.json), and against torch's e4m3 cast
  (every e2m1 value is an e4m3 value).
* A hand-worked dequantisation with two rows, two 32-element scale groups per row, both nibbles
  of a byte and the scale extremes.
* The whole layer against the already pinned FP8 block-scale MoE oracle: MXFP4 experts whose
  32-element scales vary inside a 128x128 block are rewritten as e4m3 bytes with one power-of-two
  block scale (the bytes come from torch's cast of the tabulated e2m1 values), so both layers
  must agree bit for bit.  A transposed scale array, a swapped nibble order or a wrong scale group
  breaks the agreement.
* The down projection is linear in its scales: one more unit on every w2 scale byte doubles the
  output exactly and leaves h alone.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_handworked.json")


def _num(s: str) -> float:
    if s == "nan":
        return math.nan
    if s.startswith("-2^") or s.startswith("2^"):
        neg = s.startswith("-")
        v = math.ldexp(1.0, int(s.split("^")[1]))
        return -v if neg else v
    if s == "-0":
        return -0.0
    return float(Fraction(s))


def _same(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


G = json.load(open(GOLDEN))
E2M1 = [_num(v) for v in G["e2m1"]]


def test_e2m1_decode_matches_the_ocp_table():
    for c in range(16):
        assert _same(oracle.e2m1_decode(c), E2M1[c]), c


def test_e2m1_values_are_e4m3_values():
    vals = torch.tensor(E2M1, dtype=torch.float32)
    back = vals.to(torch.float8_e4m3fn).to(torch.float32)
    assert torch.equal(back, vals)
    for c in range(16):
        assert oracle.e4m3_decode(oracle.e4m3_encode(E2M1[c])) == E2M1[c]


def test_e8m0_decode_matches_the_ocp_table():
    for b, v in G["e8m0"].items():
        assert _same(oracle.e8m0_decode(int(b)), _num(v)), b


def test_dequant_handworked():
    D = G["dequant"]
    R, K = D["R"], D["K"]
    w4 = np.zeros((R, K // 2), dtype=np.uint8)
    for d in D["bytes"]:
        w4[d["r"], d["i"]] = int(d["b"], 16)
    s = np.array(D["scales"], dtype=np.uint8)
    got = oracle.dequant_mxfp4(w4, s)
    want = np.zeros((R, K))
    listed = set()
    for d in D["expect"]:
        want[d["r"], d["k"]] = _num(d["v"])
        listed.add((d["r"], d["k"]))
    for r in range(R):
        for k in range(K):
            assert _same(got[r, k], want[r, k]) or ((r, k) not in listed and got[r, k] == 0.0), (r, k)


def _as_fp8(w4: np.ndarray, s: np.ndarray):
    """The same values as e4m3 bytes [R, K] and fp32 128x128 block scales: block scale 2^(m - 127)
    with m the smallest scale byte of the block; element = e2m1 value (from the table) times
    2^(b - m), cast by torch."""
    R, K = w4.shape[0], 2 * w4.shape[1]
    codes = np.empty((R, K), dtype=np.uint8)
    codes[:, 0::2] = w4 & 15
    codes[:, 1::2] = w4 >> 4
    b = np.repeat(s.astype(np.int64), 32, axis=1)
    m = s.astype(np.int64).reshape(R // 128, 128, K // 128, 4).min(axis=(1, 3))
    mfull = np.repeat(np.repeat(m, 128, axis=0), 128, axis=1)
    v = np.array(E2M1, dtype=np.float64)[codes] * np.exp2(b - mfull)
    assert np.abs(v).max() <= 448.0
    t = torch.from_numpy(v.astype(np.float32))
    w8 = t.to(torch.float8_e4m3fn)
    assert torch.equal(w8.to(torch.float32), t)          # exact: the values are e4m3 values
    sw = np.exp2(m - 127.0).astype(np.float32)
    return w8.view(torch.uint8).numpy(), sw


@pytest.mark.parametrize("T,S,E,H,I,seed", [(3, 2, 4, 256, 128, 1), (5, 3, 6, 384, 256, 2)])
def test_layer_matches_fp8_oracle_on_equal_values(oracle_lib, T, S, E, H, I, seed):
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=seed, shared=False)
    x = synthgen.gen_x(T, H, seed=seed)
    w13, s13, w2, s2 = {}, {}, {}, {}
    f13, fs13, f2, fs2 = {}, {}, {}, {}
    for e in range(E):
        w13[e], s13[e] = synthgen.gen_moe_expert_mxfp4(2 * I, H, seed, 2 * e)
        w2[e], s2[e] = synthgen.gen_moe_expert_mxfp4(H, I, seed, 2 * e + 1)
        f13[e], fs13[e] = _as_fp8(w13[e], s13[e])
        f2[e], fs2[e] = _as_fp8(w2[e], s2[e])
        assert len(set(s13[e].ravel().tolist())) > 1   # scales vary inside the blocks
    h4, ref4 = oracle.moe_mxfp4(x, ids, tw, w13, s13, w2, s2, E=E)
    h8, ref8 = oracle.moe(x, ids, tw, f13, fs13, f2, fs2, E=E)
    assert np.array_equal(h4, h8)
    assert np.array_equal(ref4, ref8)
    assert np.abs(ref4).max() > 0


def test_layer_is_linear_in_the_down_scales(oracle_lib):
    T, S, E, H, I = 4, 2, 3, 256, 128
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=9, shared=False)
    x = synthgen.gen_x(T, H, seed=9)
    w13, s13, w2, s2 = {}, {}, {}, {}
    for e in range(E):
        w13[e], s13[e] = synthgen.gen_moe_expert_mxfp4(2 * I, H, 9, 2 * e)
        w2[e], s2[e] = synthgen.gen_moe_expert_mxfp4(H, I, 9, 2 * e + 1)
    h, ref = oracle.moe_mxfp4(x, ids, tw, w13, s13, w2, s2, E=E)
    s2b = {e: (s2[e] + 1).astype(np.uint8) for e in s2}
    hb, refb = oracle.moe_mxfp4(x, ids, tw, w13, s13, w2, s2b, E=E)
    assert np.array_equal(h, hb)
    assert np.array_equal(refb, 2.0 * ref)
