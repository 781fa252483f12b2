"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every symbol the
header declares, and rejects bad arguments before enqueueing anything."""
import ctypes
import os
import re

import pytest

import precision_gemm_x128_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smallm_fp8bs.h")


def header_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(smallm_fp8bs_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_what_binding_lists():
    assert header_symbols() == sorted(P.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = P.lib()
    for name in header_symbols():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {P.LIB_PATH}").read()
    for name in header_symbols():
        assert re.search(rf"\bT {name}\b", out), name


def test_launch_plans_balance_the_cus():
    # the pages' shapes: 256 workgroups, each streaming the same weight bytes (one per CU)
    for (N, K), (na, cb, sb, r) in {(5120, 4096): (1, 4, 4, 4), (4608, 4096): (1, 2, 4, 4),
                                    (4096, 2048): (1, 0, 1, 2), (2048, 4096): (0, 8, 2, 4)}.items():
        p = P.smallm_fp8bs_launch_plan(16, N, K)
        assert (p["nwg"], p["NA"], p["CB"], p["SB"], p["R"]) == (256, na, cb, sb, r)
        assert p["nwg"] * (16 * p["NA"] + p["CB"]) == N
        # waves split K: R blocks each (a power of two), rounds of at most 4, every block covered
        K_blocks = K // 128
        assert p["NW"] == -(-K_blocks // p["R"]) and p["NW"] <= 8 and (p["NW"] - 1) * p["R"] < K_blocks
        assert p["RC"] == min(p["R"], 4) and p["R"] % p["RC"] == 0 and p["RC"] % p["SB"] == 0
        assert P.weight_layout(N, K) == {"NA": na, "CB": cb, "SB": sb}
    assert P.smallm_fp8bs_launch_plan(17, 4096, 2048)["MT"] == 2
    # two 16-row tiles keep the one-tile K split: 8 ranges of 4 blocks on 5120x4096
    p32 = P.smallm_fp8bs_launch_plan(32, 5120, 4096)
    assert (p32["R"], p32["RC"], p32["NW"]) == (4, 4, 8)
    assert P.smallm_fp8bs_launch_plan(16, 4096, 2048)["MT"] == 1
    # N a multiple of 4096: one 16-column group per workgroup, N / 16 workgroups
    p = P.smallm_fp8bs_launch_plan(8, 8192, 256)
    assert (p["nwg"], p["NA"], p["CB"], p["R"], p["NW"]) == (512, 1, 0, 1, 2)
    # shapes without a balanced split fall back to one 16-column group per workgroup
    p = P.smallm_fp8bs_launch_plan(8, 384, 640)
    assert (p["nwg"], p["NA"], p["CB"], p["R"], p["NW"]) == (24, 1, 0, 1, 5)
    p = P.smallm_fp8bs_launch_plan(8, 1024, 12416)   # 97 K blocks: no whole remainder fragments
    assert (p["nwg"], p["NA"], p["CB"], p["R"], p["RC"], p["NW"]) == (64, 1, 0, 16, 4, 7)
    # a remainder group of single K blocks when a wave holds one block
    p = P.smallm_fp8bs_launch_plan(8, 4608, 640)
    assert (p["nwg"], p["NA"], p["CB"], p["SB"], p["R"]) == (256, 1, 2, 1, 1)
    # up to 4 rows on a short K (<= 16 blocks) take ranges of twice the blocks
    p = P.smallm_fp8bs_launch_plan(4, 4096, 2048)
    assert (p["R"], p["RC"], p["NW"]) == (4, 4, 4)
    p = P.smallm_fp8bs_launch_plan(5, 4096, 2048)
    assert (p["R"], p["RC"], p["NW"]) == (2, 2, 8)
    p = P.smallm_fp8bs_launch_plan(1, 384, 640)
    assert (p["R"], p["RC"], p["NW"]) == (2, 2, 3)
    p = P.smallm_fp8bs_launch_plan(1, 4608, 640)     # single-block remainder fragments: unchanged
    assert (p["R"], p["RC"], p["NW"]) == (1, 1, 5)
    p = P.smallm_fp8bs_launch_plan(4, 5120, 4096)    # 32 blocks: unchanged
    assert (p["R"], p["RC"], p["NW"]) == (4, 4, 8)
    assert P.kernel_name(4, 5120, 4096) == "smallm_gemm_kernel<1, 0, 1, true, 4, 4>"
    assert P.kernel_name(32, 4608, 4096) == "smallm_gemm_kernel<2, 0, 1, true, 4, 4>"
    assert P.kernel_name(8, 4096, 2048, 1) == "smallm_gemm_kernel<1, 1, 1, false, 1, 2>"
    assert P.kernel_name(8, 2048, 4096, 3) == "smallm_gemm_kernel<1, 3, 0, true, 2, 4>"


def test_version_layout_and_strerror():
    assert P.smallm_fp8bs_abi_version() == 7
    # 0x46390000 | NA << 12 | CB << 4 | SB
    assert P.smallm_fp8bs_weight_layout_id(4096, 2048) == 0x46391001
    assert P.smallm_fp8bs_weight_layout_id(5120, 4096) == 0x46391044
    assert P.smallm_fp8bs_weight_layout_id(4608, 4096) == 0x46391024
    assert P.smallm_fp8bs_weight_layout_id(2048, 4096) == 0x46390082
    assert P.smallm_fp8bs_weight_layout_id(5120, 2048) == 0x46391042   # 2 K blocks per wave: SB = 2
    assert P.smallm_fp8bs_weight_layout_id(384, 640) == 0x46391001
    assert P.smallm_fp8bs_weight_layout_id(4608, 640) == 0x46391021
    assert P.smallm_fp8bs_weight_layout_id(100, 128) == 0
    for s in range(6):
        assert len(P.strerror(s)) > 0
    assert P.strerror(99) == "unknown status"


def test_workspace_entry_sizes_and_host_checks():
    assert P.smallm_fp8bs_quant_gemm_workspace_bytes(32, 4096, 2048) == 0      # the fused kernel
    assert P.smallm_fp8bs_quant_gemm_workspace_bytes(33, 4096, 2048) == (33 * 2048 + 255) // 256 * 256 + 33 * 16 * 4
    assert P.smallm_fp8bs_quant_gemm_workspace_bytes(41, 4096, 2048) == (41 * 2048 + 255) // 256 * 256 + 41 * 16 * 4
    assert P.smallm_fp8bs_quant_gemm_workspace_bytes(256, 5120, 4096) == 256 * 4096 + 256 * 32 * 4
    assert P.smallm_fp8bs_quant_gemm_workspace_bytes(64, 4096, 128 * 129) == 0   # K past the tiled kernel
    L = P.lib()
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: every case fails a host check
    M, N, K = 64, 4096, 2048
    lid = P.smallm_fp8bs_weight_layout_id(N, K)
    need = P.smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K)
    for fn in (L.smallm_fp8bs_quant_gemm_ws, L.smallm_fp8bs_quant_gemm_e8m0_ws):
        assert fn(fake, K, fake, lid, fake, fake, N, M, N, K, None, need, None) == 1
        assert fn(fake, K, fake, lid, fake, fake, N, M, N, K, fake, need - 1, None) == 2
        assert fn(fake, K, fake, lid, fake, fake, N, M, N, K, ctypes.c_void_p(0x100010), need, None) == 3
        assert fn(fake, K, fake, lid + 1, fake, fake, N, M, N, K, fake, need, None) == 4


def test_read_floor_rejects_bad_arguments_before_launch():
    L = P.lib()
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: every case fails its host check
    assert L.smallm_fp8bs_read_floor(None, 1024, fake, None) == 1
    assert L.smallm_fp8bs_read_floor(fake, 1024, None, None) == 1
    assert L.smallm_fp8bs_read_floor(fake, 0, fake, None) == 2
    assert L.smallm_fp8bs_read_floor(fake, (1 << 30) + 1, fake, None) == 2
    assert L.smallm_fp8bs_read_floor(ctypes.c_void_p(0x10008), 1024, fake, None) == 3


@pytest.mark.parametrize("M,N,K,ldx,expect", [
    (1, 4096, 2048, 2048, 0), (32, 5120, 4096, 4096, 0), (256, 4096, 2048, 2048, 0),
    (0, 4096, 2048, 2048, 2), (257, 4096, 2048, 2048, 2), (4, 4000, 2048, 2048, 2),
    (4, 4096, 2000, 2000, 2), (4, 4096, 2048, 2047, 2), (4, 4096, 2048, 2052, 3),
    (4, 4096, 2048, 2056, 0), (4, 0, 2048, 2048, 2), (4, 4096, -128, 2048, 2),
])
def test_supported(M, N, K, ldx, expect):
    assert P.smallm_fp8bs_supported(M, N, K, ldx) == expect


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


def test_rejections_happen_before_any_launch():
    """Invalid arguments are refused on the host; these calls never reach HIP (no GPU here)."""
    L = P.lib()
    lid = P.smallm_fp8bs_weight_layout_id(4096, 2048)
    f = _fake()
    # null pointers
    assert L.smallm_fp8bs_quant_gemm(None, 2048, f, lid, f, f, 4096, 4, 4096, 2048, None, None, None) == 1
    assert L.smallm_fp8bs_quant_gemm(f, 2048, None, lid, f, f, 4096, 4, 4096, 2048, None, None, None) == 1
    assert L.smallm_fp8bs_gemm(f, 2048, None, f, lid, f, f, 4096, 4, 4096, 2048, None) == 1
    assert L.smallm_fp8bs_quant(None, 2048, f, 2048, f, 4, 2048, None) == 1
    assert L.smallm_fp8bs_pack_weight(None, f, 128, 128, None) == 1
    assert L.smallm_fp8bs_quant_weight(f, 128, None, f, 128, 128, None) == 1
    # shapes
    assert L.smallm_fp8bs_quant_gemm(f, 2048, f, lid, f, f, 4096, 0, 4096, 2048, None, None, None) == 2
    assert L.smallm_fp8bs_quant_gemm(f, 2048, f, lid, f, f, 4096, 257, 4096, 2048, None, None, None) == 2
    assert L.smallm_fp8bs_quant_gemm(f, 2048, f, lid, f, f, 4096, 4, 4100, 2048, None, None, None) == 2
    assert L.smallm_fp8bs_quant_gemm(f, 2048, f, lid, f, f, 4000, 4, 4096, 2048, None, None, None) == 2
    assert L.smallm_fp8bs_quant_gemm_e8m0(f, 2048, f, lid, f, f, 4096, 4, 4096, 2000, None, None, None) == 2
    assert L.smallm_fp8bs_quant(f, 2048, f, 2048, f, 4, 2100, None) == 2
    assert L.smallm_fp8bs_pack_weight(f, f, 100, 128, None) == 2
    # alignment: x base, x row pitch, weight base, odd y, q_dbg
    assert L.smallm_fp8bs_quant_gemm(_fake(0x10008), 2048, f, lid, f, f, 4096, 4, 4096, 2048, None, None, None) == 3
    assert L.smallm_fp8bs_quant_gemm(f, 2052, f, lid, f, f, 4096, 4, 4096, 2048, None, None, None) == 3
    assert L.smallm_fp8bs_quant_gemm(f, 2048, _fake(0x10004), lid, f, f, 4096, 4, 4096, 2048, None, None, None) == 3
    assert L.smallm_fp8bs_quant_gemm(f, 2048, f, lid, f, _fake(0x10001), 4096, 4, 4096, 2048, None, None, None) == 3
    assert L.smallm_fp8bs_quant_gemm(f, 2048, f, lid, f, f, 4096, 4, 4096, 2048, _fake(0x10002), None, None) == 3
    assert L.smallm_fp8bs_gemm(f, 2056, f, f, lid, f, f, 4096, 4, 4096, 2048, None) == 3
    assert L.smallm_fp8bs_quant(f, 2048, f, 2056, f, 4, 2048, None) == 3
    # layout id
    assert L.smallm_fp8bs_quant_gemm(f, 2048, f, lid ^ 1, f, f, 4096, 4, 4096, 2048, None, None, None) == 4
    assert L.smallm_fp8bs_gemm_e8m0(f, 2048, f, f, 0, f, f, 4096, 4, 4096, 2048, None) == 4
    # a weight packed for another shape's layout is refused
    lid5120 = P.smallm_fp8bs_weight_layout_id(5120, 4096)
    assert L.smallm_fp8bs_quant_gemm(f, 4096, f, lid5120, f, f, 4608, 4, 4608, 4096, None, None, None) == 4


def test_producer_rejections_happen_before_any_launch():
    """smallm_fp8bs_rmsnorm_quant(_e8m0): bad pointers, eps, shapes and alignment are refused on
    the host (argument order: x, ldx, w, eps, y, ldy, q, ldq, sx, M, H, stream)."""
    L = P.lib()
    f = _fake()
    for fn in (L.smallm_fp8bs_rmsnorm_quant, L.smallm_fp8bs_rmsnorm_quant_e8m0):
        assert fn(None, 4096, f, 1e-6, f, 4096, f, 4096, f, 4, 4096, None) == 1      # no x
        assert fn(f, 4096, None, 1e-6, f, 4096, f, 4096, f, 4, 4096, None) == 1      # no w
        assert fn(f, 4096, f, 1e-6, None, 0, None, 0, None, 4, 4096, None) == 1      # no output
        assert fn(f, 4096, f, 1e-6, f, 4096, f, 4096, None, 4, 4096, None) == 1      # q without sx
        assert fn(f, 4096, f, 0.0, f, 4096, f, 4096, f, 4, 4096, None) == 1          # eps <= 0
        assert fn(f, 4096, f, -1e-6, f, 4096, f, 4096, f, 4, 4096, None) == 1
        assert fn(f, 4096, f, float("inf"), f, 4096, f, 4096, f, 4, 4096, None) == 1
        assert fn(f, 4096, f, float("nan"), f, 4096, f, 4096, f, 4, 4096, None) == 1
        assert fn(f, 4096, f, 1e-6, f, 4096, f, 4096, f, 0, 4096, None) == 2         # M = 0
        assert fn(f, 4096, f, 1e-6, f, 4096, f, 4096, f, 4, 4000, None) == 2         # H % 128
        assert fn(f, 32768, f, 1e-6, f, 32768, f, 32768, f, 4, 32768, None) == 2    # H too long
        assert fn(f, 4000, f, 1e-6, f, 4096, f, 4096, f, 4, 4096, None) == 2         # ldx < H
        assert fn(f, 4096, f, 1e-6, f, 4000, f, 4096, f, 4, 4096, None) == 2         # ldy < H
        assert fn(f, 4096, f, 1e-6, f, 4096, f, 4000, f, 4, 4096, None) == 2         # ldq < H
        assert fn(_fake(0x10008), 4096, f, 1e-6, f, 4096, f, 4096, f, 4, 4096, None) == 3
        assert fn(f, 4100, f, 1e-6, f, 4096, f, 4096, f, 4, 4096, None) == 3         # x pitch
        assert fn(f, 4096, _fake(0x10002), 1e-6, f, 4096, f, 4096, f, 4, 4096, None) == 3
        assert fn(f, 4096, f, 1e-6, f, 4100, f, 4096, f, 4, 4096, None) == 3         # y pitch
        assert fn(f, 4096, f, 1e-6, f, 4096, f, 4104, f, 4, 4096, None) == 3         # q pitch



def test_moe_rejections_happen_before_any_launch():
    """smallm_fp8bs_moe and the MoE packers refuse bad pointers, shapes, alignment and layout
    tags on the host (moe argument order: x, ldx, ids, tw, T, S, w13, sw13, w2, sw2, layout,
    E, H, I, h, y, ldy, stream)."""
    L = P.lib()
    f = _fake()
    lid = P.smallm_fp8bs_moe_layout_id()
    assert lid == 0x4D4F4510
    wsb = P.smallm_fp8bs_moe_workspace_bytes(4, 11, 4096, 256)
    ok = [f, 4096, f, f, 4, 11, f, f, f, f, lid, 513, 4096, 256, f, wsb, f, 4096, None]

    def call(**kw):
        a = list(ok)
        names = ["x", "ldx", "ids", "tw", "T", "S", "w13", "sw13", "w2", "sw2", "lid", "E", "H", "I",
                 "ws", "wsb", "y", "ldy"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.smallm_fp8bs_moe(*a)

    for name in ("x", "ids", "tw", "w13", "sw13", "w2", "sw2", "ws", "y"):
        assert call(**{name: None}) == 1, name
    assert call(T=0) == 2 and call(T=49) == 2 and call(S=0) == 2 and call(S=17) == 2
    assert call(E=0) == 2 and call(E=4097) == 2
    assert call(H=4000, ldx=4000, ldy=4000) == 2 and call(I=200) == 2 and call(I=4096) == 2
    assert call(H=32768, ldx=32768, ldy=32768) == 2
    assert call(ldx=4000) == 2 and call(ldy=4000) == 2
    assert call(wsb=wsb - 1) == 2
    assert call(x=_fake(0x10008)) == 3 and call(ldx=4100) == 3 and call(ws=_fake(0x10080)) == 3
    assert call(w13=_fake(0x10008)) == 3 and call(w2=_fake(0x10004)) == 3
    assert call(y=_fake(0x10001)) == 3 and call(ids=_fake(0x10002)) == 3 and call(tw=_fake(0x10002)) == 3
    assert call(lid=lid ^ 1) == 4
    # workspace: h rounded to 256 bytes, then NS fp32 partial planes when NS > 1
    assert P.smallm_fp8bs_moe_splits(1, 11) == 1 and P.smallm_fp8bs_moe_splits(11, 11) == 1
    assert P.smallm_fp8bs_moe_splits(12, 11) == 2 and P.smallm_fp8bs_moe_splits(20, 11) == 2
    assert P.smallm_fp8bs_moe_splits(48, 11) == 2 and P.smallm_fp8bs_moe_splits(48, 16) == 2
    assert P.smallm_fp8bs_moe_splits(0, 11) == 0 and P.smallm_fp8bs_moe_splits(4, 17) == 0
    assert P.smallm_fp8bs_moe_workspace_bytes(1, 11, 4096, 256) == 11 * 256 * 2          # 22 x 256 bytes
    assert P.smallm_fp8bs_moe_workspace_bytes(1, 3, 4096, 128) == 768
    # h, the split partials, one arrival counter per 16 output columns (256 counters = 1 KiB)
    assert P.smallm_fp8bs_moe_workspace_bytes(20, 11, 4096, 256) == 220 * 256 * 2 + 2 * 20 * 4096 * 4 + 1024
    assert P.smallm_fp8bs_moe_workspace_bytes(49, 11, 4096, 256) == 0
    assert P.smallm_fp8bs_moe_supported(48, 16, 4096, 16384, 2048) == 0
    assert P.smallm_fp8bs_moe_supported(1, 1, 1, 128, 128) == 0
    for fn in (L.smallm_fp8bs_moe_pack, L.smallm_fp8bs_moe_unpack):
        assert fn(None, f, 2, 256, 128, 1, None) == 1
        assert fn(f, None, 2, 256, 128, 1, None) == 1
        assert fn(f, f, 2, 256, 128, 2, None) == 1          # gate_up must be 0 or 1
        assert fn(f, f, 0, 256, 128, 1, None) == 2
        assert fn(f, f, 2, 200, 128, 0, None) == 2
        assert fn(f, f, 2, 256, 100, 0, None) == 2
        assert fn(_fake(0x10008), f, 2, 256, 128, 1, None) == 3


def test_moe_mxfp4_rejections_happen_before_any_launch():
    """smallm_fp8bs_moe_mxfp4 and its packers refuse bad pointers, shapes, alignment and layout
    tags on the host (argument order: x, ldx, ids, tw, T, S, w13, s13, w2, s2, layout, E, H, I, ws,
    ws bytes, y, ldy, stream); scale pointers need no alignment."""
    L = P.lib()
    f = _fake()
    lid = P.smallm_fp8bs_moe_mxfp4_layout_id()
    assert lid == 0x4D4F4504 and lid != P.smallm_fp8bs_moe_layout_id()
    wsb = P.smallm_fp8bs_moe_workspace_bytes(4, 11, 4096, 256)
    ok = [f, 4096, f, f, 4, 11, f, f, f, f, lid, 513, 4096, 256, f, wsb, f, 4096, None]
    names = ["x", "ldx", "ids", "tw", "T", "S", "w13", "s13", "w2", "s2", "lid", "E", "H", "I",
             "ws", "wsb", "y", "ldy"]

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.smallm_fp8bs_moe_mxfp4(*a)

    for name in ("x", "ids", "tw", "w13", "s13", "w2", "s2", "ws", "y"):
        assert call(**{name: None}) == 1, name
    assert call(T=0) == 2 and call(T=49) == 2 and call(S=17) == 2 and call(E=4097) == 2
    assert call(I=200) == 2 and call(ldy=4000) == 2 and call(wsb=wsb - 1) == 2
    assert call(x=_fake(0x10008)) == 3 and call(w13=_fake(0x10008)) == 3 and call(w2=_fake(0x10004)) == 3
    assert call(ws=_fake(0x10080)) == 3 and call(ids=_fake(0x10002)) == 3
    assert call(lid=P.smallm_fp8bs_moe_layout_id()) == 4
    # the FP8 entry point refuses the MXFP4 tag, and the other way round
    fp8 = [f, 4096, f, f, 4, 11, f, f, f, f, lid, 513, 4096, 256, f, wsb, f, 4096, None]
    assert L.smallm_fp8bs_moe(*fp8) == 4
    for fn in (L.smallm_fp8bs_moe_mxfp4_pack, L.smallm_fp8bs_moe_mxfp4_unpack):
        assert fn(None, f, f, f, 2, 256, 128, 1, None) == 1
        assert fn(f, None, f, f, 2, 256, 128, 1, None) == 1
        assert fn(f, f, None, f, 2, 256, 128, 1, None) == 1
        assert fn(f, f, f, None, 2, 256, 128, 1, None) == 1
        assert fn(f, f, f, f, 2, 256, 128, 2, None) == 1
        assert fn(f, f, f, f, 0, 256, 128, 1, None) == 2
        assert fn(f, f, f, f, 2, 200, 128, 0, None) == 2
        assert fn(f, f, f, f, 2, 256, 100, 0, None) == 2
        assert fn(_fake(0x10008), f, f, f, 2, 256, 128, 1, None) == 3
        assert fn(f, f, _fake(0x10008), f, 2, 256, 128, 1, None) == 3


def test_binding_rejects_wrong_dtypes_without_gpu():
    import torch
    x16 = torch.zeros((4, 256), dtype=torch.float16)
    with pytest.raises(TypeError):
        P.smallm_fp8bs_quant_gemm(x16, torch.zeros((128, 256), dtype=torch.uint8), torch.zeros((1, 2)))
    xb = torch.zeros((4, 256), dtype=torch.bfloat16)  # host tensor: refused, never handed to HIP
    with pytest.raises(ValueError):
        P.smallm_fp8bs_quant(xb)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(P, "_lib", None)
    monkeypatch.setattr(P, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        P.lib()
