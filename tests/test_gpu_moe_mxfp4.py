"""GPU parity of the MoE layer with MXFP4 expert weights against the CPU oracle.

Bars as for the FP8 block-scale layer (bf16 x bf16-exact weight products accumulated in fp32, an
fp32 silu and a bf16 intermediate, against an fp64 dequantised reference):
  * h, for every valid (token, slot) pair: |h - h_ref| <= 2^-7 |h_ref| + 1e-3 max|h_ref|, and at
    most 1 % of the elements may differ in their bits at all;
  * y: |y - ref| <= 8e-3 |ref| + 1e-3 max|ref| for every element, and the relative L2 error at
    most 5e-3 (the bar of the unit test on sglang "[AMD] Small-M MXFP4 fused-MoE kernel for gfx950
    (Qwen)", Modifications).
Shapes are that page's: E = 513 experts, 10 routed slots plus the shared expert, hidden 4096,
per-rank intermediate 256 (TP4) and 512 (TP2), and its unit test's 1 / 3 / 16 / 40 tokens; plus
small, ragged and degenerate cases, both ends of the scale range the contract allows, and graph
replay.  Experts no case routes to hold random codes with NaN scales (byte 0xFF), so reading a
wrong expert shows up as NaN.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import precision_gemm_x128_amd as P
import synthgen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WSEED = 17


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Bank4:
    """All E MXFP4 experts of one (E, H, I) shape on the device.  Experts a case uses hold
    synthgen.gen_moe_expert_mxfp4 draws (expert e: w13 index 2 e, w2 index 2 e + 1, seed WSEED);
    the others hold random codes and NaN scales."""

    def __init__(self, E, H, I):
        self.E, self.H, self.I = E, H, I
        g = torch.Generator(device=DEV)
        g.manual_seed(2000 + E + H + I)
        self.w13 = torch.randint(0, 256, (E, 2 * I, H // 2), dtype=torch.uint8, device=DEV, generator=g)
        self.w2 = torch.randint(0, 256, (E, H, I // 2), dtype=torch.uint8, device=DEV, generator=g)
        self.s13 = torch.full((E, 2 * I, H // 32), 255, dtype=torch.uint8, device=DEV)
        self.s2 = torch.full((E, H, I // 32), 255, dtype=torch.uint8, device=DEV)
        self.cpu = {}
        self.dirty = True

    def set_expert(self, e, a, b, c, d):
        self.cpu[e] = (a, b, c, d)
        self.w13[e].copy_(torch.from_numpy(a))
        self.s13[e].copy_(torch.from_numpy(b))
        self.w2[e].copy_(torch.from_numpy(c))
        self.s2[e].copy_(torch.from_numpy(d))
        self.dirty = True

    def expert(self, e):
        if e not in self.cpu:
            a, b = synthgen.gen_moe_expert_mxfp4(2 * self.I, self.H, WSEED, 2 * e)
            c, d = synthgen.gen_moe_expert_mxfp4(self.H, self.I, WSEED, 2 * e + 1)
            self.set_expert(e, a, b, c, d)
        return self.cpu[e]

    def packed(self, ids):
        for e in sorted(set(int(v) for v in np.asarray(ids).ravel() if 0 <= v < self.E)):
            self.expert(e)
        if self.dirty:
            self.w13p, self.s13p = P.smallm_fp8bs_moe_mxfp4_pack(self.w13, self.s13, True)
            self.w2p, self.s2p = P.smallm_fp8bs_moe_mxfp4_pack(self.w2, self.s2, False)
            torch.cuda.synchronize()
            self.dirty = False
        return self.w13p, self.s13p, self.w2p, self.s2p

    def oracle_maps(self, ids):
        used = sorted(set(int(v) for v in np.asarray(ids).ravel() if 0 <= v < self.E))
        return tuple({e: self.cpu[e][i] for e in used} for i in range(4))


_BANKS = {}


def bank(E, H, I):
    key = (E, H, I)
    if key not in _BANKS:
        _BANKS.clear()
        torch.cuda.empty_cache()
        _BANKS[key] = Bank4(E, H, I)
    return _BANKS[key]


def to_dev_bf16(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def run_layer(x_bits, ids, tw, B, h_fill=None):
    w13p, s13p, w2p, s2p = B.packed(ids)
    x = to_dev_bf16(x_bits)
    idd = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
    twd = torch.from_numpy(np.ascontiguousarray(tw, dtype=np.float32)).to(DEV)
    T, S = ids.shape
    ws = P.moe_workspace(T, S, B.H, B.I)
    if h_fill is not None:
        P.moe_h_view(ws, T, S, B.I).view(torch.int16).fill_(h_fill)
    y, h = P.smallm_fp8bs_moe_mxfp4(x, idd, twd, w13p, s13p, w2p, s2p, workspace=ws)
    torch.cuda.synchronize()
    return (y.view(torch.int16).cpu().numpy().view(np.uint16),
            h.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, S, B.I))


def check_against_oracle(x_bits, ids, tw, B, what):
    y, h = run_layer(x_bits, ids, tw, B)
    w13, s13, w2, s2 = B.oracle_maps(ids)
    h_ref, ref = oracle.moe_mxfp4(x_bits, ids, tw, w13, s13, w2, s2, E=B.E)
    valid = (ids >= 0) & (ids < B.E)
    hv = oracle.bf16_to_f32(h[valid]).astype(np.float64)
    hr = oracle.bf16_to_f32(h_ref[valid]).astype(np.float64)
    assert np.isfinite(hv).all(), what
    herr = np.abs(hv - hr)
    htol = 2.0 ** -7 * np.abs(hr) + 1e-3 * np.abs(hr).max()
    assert not (herr > htol).any(), f"{what}: h out of tolerance, worst {herr.max():.3e}"
    assert np.mean(h[valid] != h_ref[valid]) <= 1e-2, f"{what}: too many h bit differences"
    yv = oracle.bf16_to_f32(y).astype(np.float64)
    assert np.isfinite(yv).all(), what
    err = np.abs(yv - ref)
    tol = 8e-3 * np.abs(ref) + 1e-3 * np.abs(ref).max()
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} outputs out of tolerance, worst {err.max():.3e}"
    rel_l2 = np.linalg.norm(yv - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel_l2 <= 5e-3, f"{what}: rel L2 {rel_l2:.3e}"
    return y, h, ref


def test_mxfp4_pack_round_trip_and_positions():
    note("mxfp4 pack round trip")
    E, H, I = 3, 256, 384
    g = torch.Generator(device=DEV)
    g.manual_seed(6)
    w13 = torch.randint(0, 256, (E, 2 * I, H // 2), dtype=torch.uint8, device=DEV, generator=g)
    s13 = torch.randint(0, 256, (E, 2 * I, H // 32), dtype=torch.uint8, device=DEV, generator=g)
    w2 = torch.randint(0, 256, (E, H, I // 2), dtype=torch.uint8, device=DEV, generator=g)
    s2 = torch.randint(0, 256, (E, H, I // 32), dtype=torch.uint8, device=DEV, generator=g)
    p13, q13 = P.smallm_fp8bs_moe_mxfp4_pack(w13, s13, True)
    p2, q2 = P.smallm_fp8bs_moe_mxfp4_pack(w2, s2, False)
    u13, v13 = P.smallm_fp8bs_moe_mxfp4_unpack(p13, q13, True)
    u2, v2 = P.smallm_fp8bs_moe_mxfp4_unpack(p2, q2, False)
    assert torch.equal(u13, w13) and torch.equal(v13, s13) and torch.equal(u2, w2) and torch.equal(v2, s2)
    # fragment (tile, K block kb) of expert e: lane l holds row j = l % 16 of the tile at K elements
    # 32 (l // 16) + [0, 32), i.e. row-major bytes 64 kb + 16 (l // 16) + [0, 16), and its scale
    # byte sits at packed scale index fragment * 64 + l; w13 tile rows are gate rows 8 q + j (j < 8)
    # and up rows I + 8 q + j - 8
    a13, b13 = w13.cpu().numpy(), p13.cpu().numpy().reshape(E, -1)
    c13, d13 = s13.cpu().numpy(), q13.cpu().numpy().reshape(E, -1)
    a2, b2 = w2.cpu().numpy(), p2.cpu().numpy().reshape(E, -1)
    c2, d2 = s2.cpu().numpy(), q2.cpu().numpy().reshape(E, -1)
    rng = np.random.default_rng(2)
    for _ in range(200):
        e, l = int(rng.integers(E)), int(rng.integers(64))
        j, c = l % 16, l // 16
        q, kb = int(rng.integers(2 * I // 16)), int(rng.integers(H // 128))
        row = 8 * q + j if j < 8 else I + 8 * q + j - 8
        frag = q * (H // 128) + kb
        assert np.array_equal(b13[e, frag * 1024 + l * 16:frag * 1024 + l * 16 + 16],
                              a13[e, row, 64 * kb + 16 * c:64 * kb + 16 * c + 16])
        assert d13[e, frag * 64 + l] == c13[e, row, 4 * kb + c]
        q2, kb2 = int(rng.integers(H // 16)), int(rng.integers(I // 128))
        frag2 = q2 * (I // 128) + kb2
        assert np.array_equal(b2[e, frag2 * 1024 + l * 16:frag2 * 1024 + l * 16 + 16],
                              a2[e, 16 * q2 + j, 64 * kb2 + 16 * c:64 * kb2 + 16 * c + 16])
        assert d2[e, frag2 * 64 + l] == c2[e, 16 * q2 + j, 4 * kb2 + c]


FULL_CASES = [(1, 256), (3, 256), (16, 256), (40, 256), (1, 512), (20, 512)]


@pytest.mark.parametrize("T,I", FULL_CASES)
def test_mxfp4_full_shape(T, I):
    note(f"mxfp4 full shape T={T} I={I}")
    E, S, H = 513, 11, 4096
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(40, S, E, seed=I + 1)
    x = synthgen.gen_x(40, H, seed=I + 1)
    check_against_oracle(x[:T], ids[:T], tw[:T], B, f"T={T} I={I}")


SMALL_CASES = [
    # (T, S, E, H, I, shared, seed)
    (48, 4, 16, 1024, 256, False, 1),     # every expert shared by many tokens
    (33, 3, 8, 512, 384, False, 2),       # third row tile with one token, 3 K blocks in phase 2
    (5, 6, 40, 1152, 128, True, 3),       # 9 K blocks: waves with one and two blocks
    (16, 2, 4, 128, 128, False, 4),       # one K block: seven of eight waves idle in phase 1
    (1, 1, 1, 256, 256, False, 5),        # one pair
    (48, 1, 1, 384, 128, False, 6),       # all 48 tokens on one expert
    (2, 16, 64, 256, 128, False, 7),      # 16 slots
    (48, 16, 4096, 256, 128, False, 9),   # largest T, S and E: 768 pairs, item grid, full expert table
    (3, 2, 3, 16384, 256, False, 10),     # largest hidden size: 128 K blocks in phase 1
    (3, 2, 3, 1024, 2048, False, 12),     # largest intermediate: 16 K blocks in phase 2
    (40, 11, 64, 4096, 256, True, 8),     # 40 tokens over few experts: two and three row tiles
    (2, 16, 100, 512, 256, False, 13),    # 32 pairs: the largest per-pair grid in phase 1
    (11, 3, 100, 512, 256, False, 14),    # 33 pairs: the smallest item grid in phase 1
]


@pytest.mark.parametrize("T,S,E,H,I,shared,seed", SMALL_CASES)
def test_mxfp4_small_shapes(T, S, E, H, I, shared, seed):
    note(f"mxfp4 small T={T} S={S} E={E} H={H} I={I}")
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=seed, shared=shared)
    x = synthgen.gen_x(T, H, seed=seed)
    check_against_oracle(x, ids, tw, B, f"T={T} S={S} E={E} H={H} I={I}")


def test_mxfp4_scale_range_ends():
    """Scale bytes 252 (2^125) on every w13 group and 2 (2^-125) on every w2 group, the ends the
    contract allows, with activations scaled by 2^-110 so that every value stays finite."""
    note("mxfp4 scale range ends")
    T, S, E, H, I = 3, 2, 3, 256, 128
    B = bank(E, H, I)
    B.cpu.clear()
    for e in range(E):
        a, _ = synthgen.gen_moe_expert_mxfp4(2 * I, H, 31, 2 * e)
        c, _ = synthgen.gen_moe_expert_mxfp4(H, I, 31, 2 * e + 1)
        B.set_expert(e, a, np.full((2 * I, H // 32), 252, np.uint8), c, np.full((H, I // 32), 2, np.uint8))
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=31, shared=False)
    x = synthgen.gen_x(T, H, seed=31)
    xs = synthgen.f32_to_bf16_bits(synthgen.bf16_bits_to_f32(x) * np.float32(2.0 ** -110))
    _, _, ref = check_against_oracle(xs, ids, tw, B, "scale range ends")
    assert 1e-35 < np.abs(ref).max() < 1e30
    _BANKS.clear()


def _as_mxfp4(values):
    """Exact MXFP4 encoding of an fp64 matrix [R, K] whose every 32-wide group is a power of two
    times e2m1 values: (fp4x2 bytes [R, K/2], e8m0 scales [R, K/32]), by search over the scale
    bytes; all-zero groups get byte 127.  Raises if a group has no exact encoding."""
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    R, K = values.shape
    codes = np.zeros((R, K), dtype=np.uint8)
    scales = np.full((R, K // 32), 127, dtype=np.uint8)
    for r in range(R):
        for g in range(K // 32):
            v = values[r, 32 * g:32 * g + 32]
            if not v.any():
                continue
            for b in range(2, 253):
                m = np.abs(v) / 2.0 ** (b - 127)
                if all(x in e2m1 for x in m):
                    scales[r, g] = b
                    for i, x in enumerate(m):
                        codes[r, 32 * g + i] = e2m1.index(x) | (8 if v[i] < 0 else 0)
                    break
            else:
                raise ValueError(f"row {r} group {g} has no exact MXFP4 encoding")
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), scales


def test_mxfp4_handworked_layer_on_gpu():
    """The hand-worked layer of tests/golden/moe_handworked.json with its weights re-expressed
    exactly in MXFP4 (every weight there is an e2m1 value times a power of two): the dequantised
    weights are the same numbers, so h and y must be the hand-worked bits."""
    note("mxfp4 hand-worked layer")
    from test_oracle_moe import golden_layer
    G, x, ids, tw, w13, sw13, w2, sw2 = golden_layer()
    E = w13.shape[0]
    d13 = [oracle.dequant_weight(w13[e], sw13[e]) for e in range(E)]
    d2 = [oracle.dequant_weight(w2[e], sw2[e]) for e in range(E)]
    enc13 = [_as_mxfp4(d) for d in d13]
    enc2 = [_as_mxfp4(d) for d in d2]
    for e in range(E):    # the encodings dequantise to the same values
        assert np.array_equal(oracle.dequant_mxfp4(*enc13[e]), d13[e])
        assert np.array_equal(oracle.dequant_mxfp4(*enc2[e]), d2[e])
    st = lambda lst, i: torch.from_numpy(np.stack([t[i] for t in lst])).to(DEV)
    w13p, s13p = P.smallm_fp8bs_moe_mxfp4_pack(st(enc13, 0), st(enc13, 1), True)
    w2p, s2p = P.smallm_fp8bs_moe_mxfp4_pack(st(enc2, 0), st(enc2, 1), False)
    y, h = P.smallm_fp8bs_moe_mxfp4(to_dev_bf16(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV),
                                    w13p, s13p, w2p, s2p)
    torch.cuda.synchronize()
    y = y.view(torch.int16).cpu().numpy().view(np.uint16)
    h = h.view(torch.int16).cpu().numpy().view(np.uint16).reshape(G["T"], G["S"], G["I"])
    for d in G["h"]:
        assert h[d["t"], d["s"], d["j"]] == int(d["bits"], 16), d
    for d in G["y"]:
        assert y[d["t"], d["n"]] == int(d["bits"], 16), d
    assert np.count_nonzero(h & 0x7FFF) == len(G["h"]) and np.count_nonzero(y & 0x7FFF) == len(G["y"])


@pytest.mark.parametrize("T,S", [(6, 5), (30, 11)])   # 30 pairs: pair grid; 330: item grid
def test_mxfp4_ignores_invalid_ids_and_adds_repeated_experts(T, S):
    note(f"mxfp4 invalid and repeated ids T={T} S={S}")
    E, H, I = 24, 512, 256
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=11, shared=False)
    ids[0, 1] = -1
    ids[1, 0] = E
    ids[2, 3] = 1 << 30
    ids[3, :] = -5
    ids[4, 2] = ids[4, 0]
    ids[5, 4] = ids[5, 1]
    y, h = run_layer(synthgen.gen_x(T, H, seed=11), ids, tw, B, h_fill=0x7FC1)
    untouched = ~((ids >= 0) & (ids < E))
    assert np.all(h[untouched] == 0x7FC1)
    assert np.all(y[3] & 0x7FFF == 0)
    assert np.array_equal(h[4, 2], h[4, 0]) and np.array_equal(h[5, 4], h[5, 1])
    check_against_oracle(synthgen.gen_x(T, H, seed=11), ids, tw, B, "invalid and repeated ids")


def test_mxfp4_deterministic_and_graph_replay_bitwise():
    note("mxfp4 graph replay")
    T, S, E, H, I = 12, 11, 513, 4096, 256
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=21)
    w13p, s13p, w2p, s2p = B.packed(ids)
    x = to_dev_bf16(synthgen.gen_x(T, H, seed=21))
    idd = torch.from_numpy(ids).to(DEV)
    twd = torch.from_numpy(tw).to(DEV)
    assert P.smallm_fp8bs_moe_splits(T, S) > 1          # the split form is captured
    y1, h1 = P.smallm_fp8bs_moe_mxfp4(x, idd, twd, w13p, s13p, w2p, s2p)
    y2, h2 = P.smallm_fp8bs_moe_mxfp4(x, idd, twd, w13p, s13p, w2p, s2p)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    yg = torch.zeros_like(y1)
    ws = P.moe_workspace(T, S, H, I)
    hg = P.moe_h_view(ws, T, S, I)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        P.smallm_fp8bs_moe_mxfp4(x, idd, twd, w13p, s13p, w2p, s2p, workspace=ws, y=yg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.smallm_fp8bs_moe_mxfp4(x, idd, twd, w13p, s13p, w2p, s2p, workspace=ws, y=yg)
    for i in range(4):
        yg.zero_()
        hg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg.view(torch.int16), y1.view(torch.int16)), f"replay {i}"
        assert torch.equal(hg.view(torch.int16), h1.view(torch.int16)), f"replay {i}"
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()


def test_mxfp4_binding_errors_on_device():
    note("mxfp4 binding errors")
    T, S, E, H, I = 2, 2, 4, 256, 128
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=3, shared=False)
    w13p, s13p, w2p, s2p = B.packed(ids)
    x = to_dev_bf16(synthgen.gen_x(T, H, seed=3))
    idd = torch.from_numpy(ids).to(DEV)
    twd = torch.from_numpy(tw).to(DEV)
    with pytest.raises(P.SmallmError) as e:
        P.smallm_fp8bs_moe_mxfp4(x, idd, twd, w13p, s13p, w2p, s2p, layout_id=P.smallm_fp8bs_moe_layout_id())
    assert e.value.status == P.SMALLM_ERR_LAYOUT
    with pytest.raises(ValueError):
        P.smallm_fp8bs_moe_mxfp4(x, idd, twd, w13p, s13p[:, :, :1].contiguous(), w2p, s2p)
    with pytest.raises(ValueError):      # e4m3-shaped w13 (K bytes, not K/2) is refused
        P.smallm_fp8bs_moe_mxfp4(x, idd, twd, torch.zeros((E, 2 * I, H), dtype=torch.uint8, device=DEV),
                                 s13p, w2p, s2p)
