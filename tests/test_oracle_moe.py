"""Pins for the oracle of the FP8 block-scale small-M MoE layer (runs without a GPU).

The oracle is tied to a hand-worked layer (tests/golden/moe_handworked.json), to the already
pinned block-scale GEMM oracle (exact int64 block sums) on activations that quantise losslessly,
to closed forms of silu, and to invariants of the layer's definition (slot order, expert
labels, linearity in the top-k weights, ignored ids, a repeated expert).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe_handworked.json")


def _value(s: str) -> float:
    return float(Fraction(s))


def golden_layer():
    G = json.load(open(GOLDEN))
    H, I, E, T, S = G["H"], G["I"], G["E"], G["T"], G["S"]
    x = np.zeros((T, H), dtype=np.float32)
    for d in G["x"]:
        x[d["t"], d["k"]] = _value(d["v"])
    w13 = np.zeros((E, 2 * I, H), dtype=np.uint8)
    w2 = np.zeros((E, H, I), dtype=np.uint8)
    for d in G["w13"]:
        w13[d["e"], d["row"], d["k"]] = int(d["code"], 16)
    for d in G["w2"]:
        w2[d["e"], d["row"], d["k"]] = int(d["code"], 16)
    sw13 = np.array([[[_value(v)] for v in G["sw13"][str(e)]] for e in range(E)], np.float32)
    sw2 = np.array([[[_value(G["sw2"][str(e)])]] for e in range(E)], np.float32)
    ids = np.array(G["ids"], dtype=np.int32)
    tw = np.array([[_value(v) for v in r] for r in G["tw"]], dtype=np.float32)
    return G, synthgen.f32_to_bf16_bits(x), ids, tw, w13, sw13, w2, sw2


def test_moe_handworked_layer(oracle_lib):
    G, x, ids, tw, w13, sw13, w2, sw2 = golden_layer()
    h, ref = oracle.moe(x, ids, tw, w13, sw13, w2, sw2)
    y = oracle.round_bf16(ref)
    want_h = np.zeros_like(h)
    for d in G["h"]:
        want_h[d["t"], d["s"], d["j"]] = int(d["bits"], 16)
    want_y = np.zeros_like(y)
    for d in G["y"]:
        want_y[d["t"], d["n"]] = int(d["bits"], 16)
    # zeros may carry either sign; every non-zero element is pinned bit for bit
    assert np.array_equal(h & 0x7FFF == 0, want_h == 0)
    assert np.array_equal(np.where(h & 0x7FFF, h, 0), want_h)
    assert np.array_equal(y & 0x7FFF == 0, want_y == 0)
    assert np.array_equal(np.where(y & 0x7FFF, y, 0), want_y)


def test_silu_closed_forms(oracle_lib):
    l3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4, and silu(z) - silu(-z) = z since sigmoid(z) + sigmoid(-z) = 1
    s = oracle.silu(np.array([0.0, l3, -l3, 40.0, -40.0, 2.5]))
    assert s[0] == 0.0
    assert s[1] == pytest.approx(0.75 * l3, rel=1e-15)
    assert s[2] == pytest.approx(-0.25 * l3, rel=1e-15)
    assert s[3] == pytest.approx(40.0, rel=1e-15)
    assert abs(s[4]) < 1e-15
    z = np.linspace(-30, 30, 241)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)
    assert np.all(np.isfinite(oracle.silu(np.array([-1e4, 1e4]))))


def test_moe_gate_up_matches_block_scale_gemm_oracle(oracle_lib):
    """On activations made of e4m3 values with a 448 in every 1x128 group, the activation
    quantiser is lossless (sx = 1, q = enc(x)), so the pinned int64 block-sum GEMM must give the
    same gate and up outputs as the dequantised fp64 product."""
    rng = np.random.default_rng([40, 1])
    T, H, I = 3, 512, 256
    table = np.array([oracle.e4m3_decode(b) for b in range(256)])
    finite = np.array([b for b in range(256) if np.isfinite(table[b])], dtype=np.uint8)
    codes = rng.choice(finite, size=(T, H))
    xv = table[codes].astype(np.float32)
    xv[:, ::128] = 448.0
    x = synthgen.f32_to_bf16_bits(xv)
    q, sx = oracle.quant_act(x)
    assert np.all(sx == 1.0)
    w8, sw = oracle.quant_weight(synthgen.gen_w(2 * I, H, seed=40))
    ref = oracle.gemm(q, sx, w8, sw)
    g, u = oracle.moe_gate_up(oracle.bf16_to_f32(x).astype(np.float64), oracle.dequant_weight(w8, sw))
    scale = np.abs(ref).max()
    assert np.allclose(g, ref[:, :I], rtol=1e-12, atol=1e-13 * scale)
    assert np.allclose(u, ref[:, I:], rtol=1e-12, atol=1e-13 * scale)


def _random_layer(seed, T=3, S=4, E=6, H=256, I=128):
    x = synthgen.gen_x(T, H, seed=seed)
    w13, sw13, w2, sw2 = [], [], [], []
    for e in range(E):
        a, b = oracle.quant_weight(synthgen.gen_w(2 * I, H, seed=seed, copy=2 * e))
        c, d = oracle.quant_weight(synthgen.gen_w(H, I, seed=seed, copy=2 * e + 1))
        w13.append(a), sw13.append(b), w2.append(c), sw2.append(d)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=seed)
    return x, ids, tw, np.array(w13), np.array(sw13), np.array(w2), np.array(sw2)


def test_moe_down_projection_orientation(oracle_lib):
    """w2 a permutation matrix (row n has its 1.0 at column pi(n)), one slot with weight 1:
    y[n] = h[pi(n)], which fails if w2 is read transposed."""
    T, H, I = 2, 128, 128
    x = synthgen.gen_x(T, H, seed=41)
    w13, sw13 = oracle.quant_weight(synthgen.gen_w(2 * I, H, seed=41))
    pi = np.random.default_rng([41, 3]).permutation(I)
    assert np.any(pi[pi] != np.arange(I))             # not an involution
    w2 = np.zeros((H, I), dtype=np.uint8)
    w2[np.arange(H), pi] = 0x38
    sw2 = np.ones((1, 1), dtype=np.float32)
    ids = np.zeros((T, 1), dtype=np.int32)
    tw = np.ones((T, 1), dtype=np.float32)
    h, ref = oracle.moe(x, ids, tw, [w13], [sw13], [w2], [sw2])
    hv = oracle.bf16_to_f32(h[:, 0, :]).astype(np.float64)
    assert np.array_equal(ref, hv[:, pi])


def test_moe_invariants(oracle_lib):
    x, ids, tw, w13, sw13, w2, sw2 = _random_layer(42)
    T, S = ids.shape
    E = len(sw13)
    h, ref = oracle.moe(x, ids, tw, w13, sw13, w2, sw2)
    scale = np.abs(ref).max()
    assert scale > 0
    # slot order does not matter
    perm = np.random.default_rng([42, 5]).permutation(S)
    hp, rp = oracle.moe(x, ids[:, perm], tw[:, perm], w13, sw13, w2, sw2)
    assert np.array_equal(hp, h[:, perm])
    assert np.allclose(rp, ref, rtol=0, atol=1e-14 * scale)
    # expert labels do not matter
    lab = np.random.default_rng([42, 6]).permutation(E)
    inv = np.argsort(lab)
    hl, rl = oracle.moe(x, lab[ids], tw, w13[inv], sw13[inv], w2[inv], sw2[inv])
    assert np.array_equal(hl, h) and np.array_equal(rl, ref)
    # linear in the top-k weights (doubling is exact)
    _, r2 = oracle.moe(x, ids, tw * np.float32(2), w13, sw13, w2, sw2)
    assert np.array_equal(r2, 2 * ref)
    # ids outside [0, E) add nothing and leave h zero
    bad = ids.copy()
    bad[0, 1] = -1
    bad[1, 0] = E
    hb, rb = oracle.moe(x, bad, tw, w13, sw13, w2, sw2)
    drop = tw.copy()
    drop[0, 1] = 0
    drop[1, 0] = 0
    _, rd = oracle.moe(x, ids, drop, w13, sw13, w2, sw2)
    assert np.all(hb[0, 1] == 0) and np.all(hb[1, 0] == 0)
    assert np.allclose(rb, rd, rtol=0, atol=1e-14 * scale)
    # one expert in two slots equals one slot carrying the summed weight
    dup = ids.copy()
    dup[2, 1] = dup[2, 0]
    tdup = tw.copy()
    tdup[2, 0], tdup[2, 1] = 0.25, 0.5
    one = tdup.copy()
    one[2, 0], one[2, 1] = 0.75, 0.0
    hd, r_dup = oracle.moe(x, dup, tdup, w13, sw13, w2, sw2)
    _, r_one = oracle.moe(x, dup, one, w13, sw13, w2, sw2)
    assert np.array_equal(hd[2, 0], hd[2, 1])
    assert np.allclose(r_dup, r_one, rtol=0, atol=1e-14 * scale)


def test_moe_routing_generator_shape():
    ids, tw = synthgen.gen_moe_routing(5, 11, 513, seed=1)
    assert ids.shape == (5, 11) and ids.dtype == np.int32 and tw.dtype == np.float32
    assert np.all(ids[:, 10] == 512) and np.all(tw[:, 10] == 1.0)
    assert np.all(ids[:, :10] < 512) and np.all(ids[:, :10] >= 0)
    for t in range(5):
        assert len(set(ids[t].tolist())) == 11
    assert np.allclose(tw[:, :10].sum(axis=1), 1.0, atol=1e-6)


def test_moe_expert_generator_draws_finite_normal_like_codes():
    w8, sw = synthgen.gen_moe_expert(256, 512, seed=1, e=3)
    assert w8.shape == (256, 512) and sw.shape == (2, 4) and sw.dtype == np.float32
    assert not np.any((w8 & 0x7F) == 0x7F)                  # no NaN code
    w8b, swb = synthgen.gen_moe_expert(256, 512, seed=1, e=3)
    assert np.array_equal(w8, w8b) and np.array_equal(sw, swb)
    v = np.abs(np.array([oracle.e4m3_decode(b) for b in range(256)])[w8])
    # |v| = |z| * 448 / 4.5: the median of |z| is 0.674, so the median code value is near 67
    assert 40 < np.median(v) < 100 and v.max() <= 448
