"""GPU parity of the FP8 block-scale small-M MoE layer against the CPU oracle.

Bars (the layer's arithmetic is bf16 x e4m3 products accumulated in fp32 with an fp32 silu and a
bf16 intermediate, against an fp64 dequantised reference):
  * h, for every valid (token, slot) pair: |h - h_ref| <= 2^-7 |h_ref| + 1e-3 max|h_ref| (one
    bf16 rounding of a value the fp32 accumulation moved by far less than an ulp can land one ulp
    away), and at most 1 % of the elements may differ in their bits at all;
  * y: |y - ref| <= 8e-3 |ref| + 1e-3 max|ref| for every element, and the relative L2 error at
    most 5e-3 (the bar the MXFP4 small-M MoE test states on sglang "[AMD] Small-M MXFP4 fused-MoE
    kernel for gfx950 (Qwen)", Modifications).
Shapes are those of the pages' microbenchmarks (sglang "[AMD] gfx950 small-batch MoE: expert-count
gate for the small sort and FP8 block-scale small-M kernel", Kernel microbenchmarks: E = 513,
11 slots, hidden 4096, intermediate 256 at TP4 and 128 at TP8, up to 20 / 48 tokens) plus small,
ragged and degenerate cases.  Experts no case routes to hold random bytes, so reading a wrong
expert shows up as garbage or NaN.
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
WSEED = 7


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Bank:
    """All E experts of one (E, H, I) shape on the device, packed.  Experts a case uses hold
    synthgen.gen_moe_expert draws (expert e: w13 index 2 e, w2 index 2 e + 1, seed WSEED); the
    others hold random bytes and scales."""

    def __init__(self, E, H, I):
        self.E, self.H, self.I = E, H, I
        g = torch.Generator(device=DEV)
        g.manual_seed(1000 + E + H + I)
        self.w13 = torch.randint(0, 256, (E, 2 * I, H), dtype=torch.uint8, device=DEV, generator=g)
        self.w2 = torch.randint(0, 256, (E, H, I), dtype=torch.uint8, device=DEV, generator=g)
        self.sw13 = torch.rand((E, 2 * I // 128, H // 128), device=DEV, generator=g)
        self.sw2 = torch.rand((E, H // 128, I // 128), device=DEV, generator=g)
        self.cpu = {}
        self.dirty = True

    def expert(self, e):
        if e not in self.cpu:
            a, b = synthgen.gen_moe_expert(2 * self.I, self.H, WSEED, 2 * e)
            c, d = synthgen.gen_moe_expert(self.H, self.I, WSEED, 2 * e + 1)
            self.cpu[e] = (a, b, c, d)
            self.w13[e].copy_(torch.from_numpy(a))
            self.sw13[e].copy_(torch.from_numpy(b))
            self.w2[e].copy_(torch.from_numpy(c))
            self.sw2[e].copy_(torch.from_numpy(d))
            self.dirty = True
        return self.cpu[e]

    def packed(self, ids):
        for e in sorted(set(int(v) for v in np.asarray(ids).ravel() if 0 <= v < self.E)):
            self.expert(e)
        if self.dirty:
            self.w13p = P.smallm_fp8bs_moe_pack(self.w13, True)
            self.w2p = P.smallm_fp8bs_moe_pack(self.w2, False)
            torch.cuda.synchronize()
            self.dirty = False
        return self.w13p, self.sw13, self.w2p, self.sw2

    def oracle_maps(self, ids):
        used = sorted(set(int(v) for v in np.asarray(ids).ravel() if 0 <= v < self.E))
        w13 = {e: self.cpu[e][0] for e in used}
        sw13 = {e: self.cpu[e][1] for e in used}
        w2 = {e: self.cpu[e][2] for e in used}
        sw2 = {e: self.cpu[e][3] for e in used}
        return w13, sw13, w2, sw2


_BANKS = {}


def bank(E, H, I):
    key = (E, H, I)
    if key not in _BANKS:
        _BANKS.clear()          # one bank at a time keeps device memory bounded
        torch.cuda.empty_cache()
        _BANKS[key] = Bank(E, H, I)
    return _BANKS[key]


def to_dev_bf16(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def run_layer(x_bits, ids, tw, B, h_fill=None):
    w13p, sw13, w2p, sw2 = B.packed(ids)
    x = to_dev_bf16(x_bits)
    idd = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
    twd = torch.from_numpy(np.ascontiguousarray(tw, dtype=np.float32)).to(DEV)
    T, S = ids.shape
    ws = P.moe_workspace(T, S, B.H, B.I)
    if h_fill is not None:
        P.moe_h_view(ws, T, S, B.I).view(torch.int16).fill_(h_fill)
    y, h = P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2, workspace=ws)
    torch.cuda.synchronize()
    return (y.view(torch.int16).cpu().numpy().view(np.uint16),
            h.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, S, B.I))


def check_against_oracle(x_bits, ids, tw, B, what):
    y, h = run_layer(x_bits, ids, tw, B)
    w13, sw13, w2, sw2 = B.oracle_maps(ids)
    h_ref, ref = oracle.moe(x_bits, ids, tw, w13, sw13, w2, sw2, E=B.E)
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


def test_moe_pack_round_trip_and_interleave():
    note("moe pack round trip")
    E, H, I = 3, 256, 384
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    w13 = torch.randint(0, 256, (E, 2 * I, H), dtype=torch.uint8, device=DEV, generator=g)
    w2 = torch.randint(0, 256, (E, H, I), dtype=torch.uint8, device=DEV, generator=g)
    p13 = P.smallm_fp8bs_moe_pack(w13, True)
    p2 = P.smallm_fp8bs_moe_pack(w2, False)
    assert torch.equal(P.smallm_fp8bs_moe_unpack(p13, True), w13)
    assert torch.equal(P.smallm_fp8bs_moe_unpack(p2, False), w2)
    # fragment (tile q, K block kb) of expert e: lane l holds row j = l % 16 of the tile at K bytes
    # 32 (l // 16) + [0, 16) (first KiB) and + [16, 32) (second KiB); w13 tile rows are gate rows
    # 8 q + j (j < 8) and up rows I + 8 q + j - 8
    a13, b13 = w13.cpu().numpy(), p13.cpu().numpy().reshape(E, -1)
    a2, b2 = w2.cpu().numpy(), p2.cpu().numpy().reshape(E, -1)
    rng = np.random.default_rng(1)
    for _ in range(200):
        e = int(rng.integers(E))
        q, kb, l, half = int(rng.integers(2 * I // 16)), int(rng.integers(H // 128)), int(rng.integers(64)), int(rng.integers(2))
        j, c = l % 16, l // 16
        row = 8 * q + j if j < 8 else I + 8 * q + j - 8
        off = (q * (H // 128) + kb) * 2048 + half * 1024 + l * 16
        k0 = kb * 128 + 32 * c + 16 * half
        assert np.array_equal(b13[e, off:off + 16], a13[e, row, k0:k0 + 16])
        q2, kb2 = int(rng.integers(H // 16)), int(rng.integers(I // 128))
        off2 = (q2 * (I // 128) + kb2) * 2048 + half * 1024 + l * 16
        k2 = kb2 * 128 + 32 * c + 16 * half
        assert np.array_equal(b2[e, off2:off2 + 16], a2[e, 16 * q2 + j, k2:k2 + 16])


FULL_CASES = [
    # (T, I): the pages' TP4 (I = 256, cap 20 tokens) and TP8 (I = 128, cap 48 tokens) shapes; a
    # case takes the first T tokens of one routing per shape, so the cases share their experts
    (1, 256), (3, 256), (8, 256), (20, 256),
    (1, 128), (17, 128), (48, 128),
]


@pytest.mark.parametrize("T,I", FULL_CASES)
def test_moe_full_shape(T, I):
    note(f"moe full shape T={T} I={I}")
    E, S, H = 513, 11, 4096
    B = bank(E, H, I)
    Tmax = 20 if I == 256 else 48
    ids, tw = synthgen.gen_moe_routing(Tmax, S, E, seed=I)
    x = synthgen.gen_x(Tmax, H, seed=I)
    check_against_oracle(x[:T], ids[:T], tw[:T], B, f"T={T} I={I}")


SMALL_CASES = [
    # (T, S, E, H, I, shared, seed): collisions, ragged tiles, odd K-block counts
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
    (8, 16, 200, 512, 256, False, 13),    # 128 pairs: the largest unsplit down projection
    (43, 3, 200, 512, 256, False, 14),    # 129 pairs: the smallest split one
    (2, 16, 200, 512, 256, False, 15),    # 32 pairs: the largest per-pair grid in phase 1
    (11, 3, 200, 512, 256, False, 16),    # 33 pairs: the smallest item grid in phase 1
]


@pytest.mark.parametrize("T,S,E,H,I,shared,seed", SMALL_CASES)
def test_moe_small_shapes(T, S, E, H, I, shared, seed):
    note(f"moe small T={T} S={S} E={E} H={H} I={I}")
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=seed, shared=shared)
    x = synthgen.gen_x(T, H, seed=seed)
    check_against_oracle(x, ids, tw, B, f"T={T} S={S} E={E} H={H} I={I}")


@pytest.mark.parametrize("T,S", [(6, 5), (30, 11)])   # 30 pairs: pair grid; 330: item grid
def test_moe_ignores_invalid_ids_and_adds_repeated_experts(T, S):
    note(f"moe invalid and repeated ids T={T} S={S}")
    E, H, I = 24, 512, 256
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=11, shared=False)
    ids[0, 1] = -1
    ids[1, 0] = E
    ids[2, 3] = 1 << 30
    ids[3, :] = -5                      # a token with no valid slot: y row is zero
    ids[4, 2] = ids[4, 0]               # one expert in two slots
    ids[5, 4] = ids[5, 1]
    y, h = run_layer(synthgen.gen_x(T, H, seed=11), ids, tw, B, h_fill=0x7FC1)
    untouched = ~((ids >= 0) & (ids < E))
    assert np.all(h[untouched] == 0x7FC1)
    assert np.all(y[3] & 0x7FFF == 0)
    assert np.array_equal(h[4, 2], h[4, 0]) and np.array_equal(h[5, 4], h[5, 1])
    check_against_oracle(synthgen.gen_x(T, H, seed=11), ids, tw, B, "invalid and repeated ids")


def test_moe_handworked_layer_on_gpu():
    """The hand-worked layer of tests/golden/moe_handworked.json through the library."""
    note("moe hand-worked layer")
    from test_oracle_moe import golden_layer
    G, x, ids, tw, w13, sw13, w2, sw2 = golden_layer()
    w13p = P.smallm_fp8bs_moe_pack(torch.from_numpy(w13).to(DEV), True)
    w2p = P.smallm_fp8bs_moe_pack(torch.from_numpy(w2).to(DEV), False)
    y, h = P.smallm_fp8bs_moe(to_dev_bf16(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV),
                              w13p, torch.from_numpy(sw13).to(DEV), w2p, torch.from_numpy(sw2).to(DEV))
    torch.cuda.synchronize()
    y = y.view(torch.int16).cpu().numpy().view(np.uint16)
    h = h.view(torch.int16).cpu().numpy().view(np.uint16).reshape(G["T"], G["S"], G["I"])
    for d in G["h"]:
        assert h[d["t"], d["s"], d["j"]] == int(d["bits"], 16), d
    for d in G["y"]:
        assert y[d["t"], d["n"]] == int(d["bits"], 16), d
    assert np.count_nonzero(h & 0x7FFF) == len(G["h"]) and np.count_nonzero(y & 0x7FFF) == len(G["y"])


def test_moe_deterministic_and_graph_replay_bitwise():
    note("moe graph replay")
    T, S, E, H, I = 12, 11, 513, 4096, 256
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=21)
    w13p, sw13, w2p, sw2 = B.packed(ids)
    x = to_dev_bf16(synthgen.gen_x(T, H, seed=21))
    idd = torch.from_numpy(ids).to(DEV)
    twd = torch.from_numpy(tw).to(DEV)
    y1, h1 = P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2)
    y2, h2 = P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert P.smallm_fp8bs_moe_splits(T, S) > 1          # the split form is captured
    yg = torch.zeros_like(y1)
    ws = P.moe_workspace(T, S, H, I)
    hg = P.moe_h_view(ws, T, S, I)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2, workspace=ws, y=yg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2, workspace=ws, y=yg)
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


def test_moe_split_partials_summed_by_the_last_workgroup():
    # Above 128 pairs two workgroups share each output tile; the one that finishes last reads the
    # other's fp32 partial (written through to the device coherence point) and writes y.  A graph
    # of 48 calls alternating between two inputs over one workspace must give every call the
    # output of an eager call on its own input, bit for bit: a partial read before it landed, or
    # one left over from the previous call (the other input), would show as a mismatch.
    note("moe split partials, 48 calls in a graph")
    T, S, E, H, I = 24, 11, 513, 4096, 128
    assert P.smallm_fp8bs_moe_splits(T, S) > 1
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=31)
    w13p, sw13, w2p, sw2 = B.packed(ids)
    idd = torch.from_numpy(ids).to(DEV)
    twd = torch.from_numpy(tw).to(DEV)
    xs = [to_dev_bf16(synthgen.gen_x(T, H, seed=31 + k)) for k in range(2)]
    refs = [P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2)[0] for x in xs]
    torch.cuda.synchronize()
    assert not torch.equal(refs[0].view(torch.int16), refs[1].view(torch.int16))
    n = 48
    ws = P.moe_workspace(T, S, H, I)
    ys = torch.zeros((n, T, H), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        P.smallm_fp8bs_moe(xs[0], idd, twd, w13p, sw13, w2p, sw2, workspace=ws, y=ys[0])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            P.smallm_fp8bs_moe(xs[i % 2], idd, twd, w13p, sw13, w2p, sw2, workspace=ws, y=ys[i])
    for rep in range(3):
        ys.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(n):
            assert torch.equal(ys[i].view(torch.int16), refs[i % 2].view(torch.int16)), f"replay {rep} call {i}"


def test_moe_binding_errors_on_device():
    note("moe binding errors")
    T, S, E, H, I = 2, 2, 4, 256, 128
    B = bank(E, H, I)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=3, shared=False)
    w13p, sw13, w2p, sw2 = B.packed(ids)
    x = to_dev_bf16(synthgen.gen_x(T, H, seed=3))
    idd = torch.from_numpy(ids).to(DEV)
    twd = torch.from_numpy(tw).to(DEV)
    with pytest.raises(P.SmallmError) as e:
        P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2, layout_id=1)
    assert e.value.status == P.SMALLM_ERR_LAYOUT
    with pytest.raises(TypeError):
        P.smallm_fp8bs_moe(x, idd.long(), twd, w13p, sw13, w2p, sw2)
    with pytest.raises(ValueError):
        P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13[:, :1].contiguous(), w2p, sw2)
    small = torch.empty(P.smallm_fp8bs_moe_workspace_bytes(T, S, H, I) - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(P.SmallmError) as e:
        P.smallm_fp8bs_moe(x, idd, twd, w13p, sw13, w2p, sw2, workspace=small)
    assert e.value.status == P.SMALLM_ERR_SHAPE
    xt = to_dev_bf16(synthgen.gen_x(49, H, seed=3))
    ids49, tw49 = synthgen.gen_moe_routing(49, S, E, seed=3, shared=False)
    with pytest.raises(P.SmallmError) as e:
        P.smallm_fp8bs_moe(xt, torch.from_numpy(ids49).to(DEV), torch.from_numpy(tw49).to(DEV),
                           w13p, sw13, w2p, sw2)
    assert e.value.status == P.SMALLM_ERR_SHAPE
