"""Seeded synthetic inputs for the small-M FP8 block-scale GEMM.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic (no quantisation, no scales, no products).  Both the GPU library's tests/benchmark
and the CPU oracle take their inputs from here.

Recipe (the pages' workloads are Qwen3.5-397B-A17B TP4 projection shapes run on 1-32 decode or
verify rows, see sglang "[AMD] Small-M FP8 block-scale GEMM with fused activation quant for
gfx950 (Qwen3.5)", sections Modifications and Kernel microbenchmarks; trained weights are not
used, these synthetic draws stand in for them):

* X, bf16 [M, K]: z ~ N(0, 1) in fp32, each 1x128 group multiplied by f = 2^u with
  u ~ U(-4, 4) drawn once per (row, group); x = bf16_rne(fp32(z * f)).  numpy PCG64 seeded with
  the tuple (seed, 0).
* Outlier rows (optional): ceil(0.05 * M) rows picked by a seeded permutation; in every 1x128
  group of those rows one uniformly chosen position is set to +-1000 (exact in bf16) with a
  random sign.  Seed tuple (seed, 0, 1).
* W, fp32 [N, K]: w ~ N(0, 0.02), weight copy i drawn with seed tuple (seed, 1, i).  The fp8
  weight and its block scales are derived from it by a quantiser (oracle or library), never
  here.
* MoE routing (sglang "[AMD] gfx950 small-batch MoE: expert-count gate for the small sort and
  FP8 block-scale small-M kernel", Kernel microbenchmarks: E = 513 experts, 11 slots per token):
  read as 512 routed experts plus one shared expert; see gen_moe_routing.  Expert weights
  arrive quantised (e4m3 with fp32 128x128 block scales), so they are drawn as bytes directly:
  see gen_moe_expert (w13 of expert e with index 2 e, w2 with index 2 e + 1).
"""
from __future__ import annotations

import math

import numpy as np


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Used only to produce bf16 inputs; inputs here are always finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_x(M: int, K: int, seed: int = 0, outliers: bool = False) -> np.ndarray:
    """bf16 activations as uint16 bit patterns, shape [M, K]."""
    assert K % 128 == 0
    rng = np.random.default_rng([seed, 0])
    z = rng.standard_normal((M, K), dtype=np.float32)
    u = rng.uniform(-4.0, 4.0, size=(M, K // 128))
    f = np.exp2(u).astype(np.float32)
    v = (z.reshape(M, K // 128, 128) * f[:, :, None]).astype(np.float32).reshape(M, K)
    x = f32_to_bf16_bits(v)
    if outliers and M > 0:
        orng = np.random.default_rng([seed, 0, 1])
        n_out = math.ceil(0.05 * M)
        rows = orng.permutation(M)[:n_out]
        G = K // 128
        pos = orng.integers(0, 128, size=(n_out, G))
        sgn = orng.integers(0, 2, size=(n_out, G))
        one_k = np.uint16(0x447A)  # 1000.0 in bf16
        for i, r in enumerate(rows):
            for g in range(G):
                x[r, 128 * g + pos[i, g]] = one_k | (np.uint16(0x8000) if sgn[i, g] else np.uint16(0))
    return x


def gen_w(N: int, K: int, seed: int = 0, copy: int = 0) -> np.ndarray:
    """fp32 master weights ~ N(0, 0.02), shape [N, K]."""
    rng = np.random.default_rng([seed, 1, copy])
    return rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)


def outlier_rows(M: int, seed: int = 0) -> np.ndarray:
    """The rows gen_x(..., outliers=True) turns into outlier rows."""
    orng = np.random.default_rng([seed, 0, 1])
    return orng.permutation(M)[: math.ceil(0.05 * M)]


def gen_moe_routing(T: int, S: int, E: int, seed: int = 0, shared: bool = True):
    """Synthetic top-k routing: (ids int32 [T, S], tw float32 [T, S]).

    With shared=True the last slot of every token holds expert E - 1 (the always-on shared expert)
    with weight 1, and the other S - 1 slots hold distinct experts drawn uniformly from [0, E - 1)
    with weights v / sum(v), v ~ U(0.05, 1).  With shared=False all S slots are routed that way
    over [0, E).  Seed tuple (seed, 2)."""
    rng = np.random.default_rng([seed, 2])
    routed = S - 1 if shared else S
    pool = E - 1 if shared else E
    assert 0 <= routed <= pool
    ids = np.empty((T, S), dtype=np.int32)
    tw = np.empty((T, S), dtype=np.float32)
    for t in range(T):
        ids[t, :routed] = rng.permutation(pool)[:routed]
        v = rng.uniform(0.05, 1.0, size=routed)
        tw[t, :routed] = (v / v.sum()).astype(np.float32)
        if shared:
            ids[t, routed] = E - 1
            tw[t, routed] = 1.0
    return ids, tw


def _e4m3_normal_exponent_law(spread: float = 4.5) -> np.ndarray:
    """Probabilities of the 16 exponent fields of |v| for v = z * 448 / spread, z ~ N(0, 1)
    (a normal weight block whose largest value maps near 448), from the normal law."""
    c = 448.0 / spread

    def mass(lo, hi):   # P(lo <= |z| * c < hi)
        return math.erf(hi / c / math.sqrt(2)) - math.erf(lo / c / math.sqrt(2))

    p = [mass(0.0, 2.0 ** -6)]
    p += [mass(2.0 ** (e - 7), 2.0 ** (e - 6)) for e in range(1, 15)]
    p += [mass(256.0, 1e300)]
    p = np.array(p)
    return p / p.sum()


def gen_moe_expert(R: int, K: int, seed: int, e: int):
    """Expert e's e4m3 matrix [R, K] as bytes plus fp32 128x128 block scales.

    The bytes are drawn to look like a quantised normal weight block: sign uniform, exponent
    field from _e4m3_normal_exponent_law (through a 2^16-entry table), mantissa uniform (folded
    to 0..6 in the top binade, so no NaN code).  Scales: 4.5 * sigma / 448 with sigma = 0.02 * U(0.8, 1.2) per block.  Seed tuple
    (seed, 3, e), so any expert can be drawn on its own."""
    rng = np.random.default_rng([seed, 3, e])
    p = _e4m3_normal_exponent_law()
    counts = np.floor(p * 65536).astype(np.int64)
    counts[int(np.argmax(counts))] += 65536 - counts.sum()
    table = np.repeat(np.arange(16, dtype=np.uint8), counts)          # 2^16-entry sampling table
    ex = table[rng.integers(0, 65536, size=(R, K), dtype=np.uint16)]
    b = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    man = b & 7
    man = np.where(ex == 15, man % 7, man).astype(np.uint8)
    sign = b >> 7
    w8 = (sign << 7) | (ex << 3) | man
    sigma = 0.02 * rng.uniform(0.8, 1.2, size=(R // 128, K // 128))
    sw = (4.5 * sigma / 448.0).astype(np.float32)
    return w8.astype(np.uint8), sw


def _e2m1_normal_magnitude_law(spread: float = 2.5) -> np.ndarray:
    """Probabilities of the 8 e2m1 magnitude codes 0..7 (values 0, 0.5, 1, 1.5, 2, 3, 4, 6) for
    |v| with v = z * 6 / spread, z ~ N(0, 1), binned at the midpoints between those values (a
    normal group of 32 whose largest value lands near 6)."""
    c = 6.0 / spread
    edges = [0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, math.inf]

    def mass(lo, hi):
        top = 1.0 if hi == math.inf else math.erf(hi / c / math.sqrt(2))
        return top - math.erf(lo / c / math.sqrt(2))

    p = np.array([mass(edges[i], edges[i + 1]) for i in range(8)])
    return p / p.sum()


def gen_moe_expert_mxfp4(R: int, K: int, seed: int, e: int):
    """Expert e's MXFP4 matrix [R, K]: fp4x2 bytes [R, K/2] (even K element in the low nibble) and
    e8m0 scale bytes [R, K/32], one per 32 consecutive K elements of a row.

    Codes: sign uniform, magnitude from _e2m1_normal_magnitude_law (through a 2^16-entry table).
    Scales: byte 120 + U{-1, 0, 1} (2^-8 .. 2^-6, so 6 * scale spans the 0.02-sigma weights of
    gen_moe_expert).  Seed tuple (seed, 4, e), so any expert can be drawn on its own."""
    rng = np.random.default_rng([seed, 4, e])
    p = _e2m1_normal_magnitude_law()
    counts = np.floor(p * 65536).astype(np.int64)
    counts[int(np.argmax(counts))] += 65536 - counts.sum()
    table = np.repeat(np.arange(8, dtype=np.uint8), counts)
    mag = table[rng.integers(0, 65536, size=(R, K), dtype=np.uint16)]
    sign = rng.integers(0, 2, size=(R, K), dtype=np.uint8)
    codes = (sign << 3) | mag
    w4 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = (120 + rng.integers(-1, 2, size=(R, K // 32))).astype(np.uint8)
    return w4, s
