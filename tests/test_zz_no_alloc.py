"""The allocation-free MoE entry point (smallm_fp8bs_moe_noalloc, workspace in the library's static
device array) against the workspace entry point smallm_fp8bs_moe on the same inputs, through the
C ABI: bit-identical outputs on two calls in a row, the second with a smaller input (the array
keeps the first call's contents), and a workspace beyond the array's size refused before any
launch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import precision_gemm_x128_amd as P
import synthgen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def layer(E, H, I, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    # e4m3 bytes without the NaN codes, block scales around 2e-3
    w13 = torch.randint(0, 256, (E, 2 * I, H), dtype=torch.uint8, device=DEV, generator=g) & 0xBF
    w2 = torch.randint(0, 256, (E, H, I), dtype=torch.uint8, device=DEV, generator=g) & 0xBF
    sw13 = torch.rand((E, 2 * I // 128, H // 128), device=DEV, generator=g) * 4e-3
    sw2 = torch.rand((E, H // 128, I // 128), device=DEV, generator=g) * 4e-3
    return P.smallm_fp8bs_moe_pack(w13, True), sw13, P.smallm_fp8bs_moe_pack(w2, False), sw2


def inputs(T, S, E, H, seed):
    x = torch.from_numpy(synthgen.gen_x(T, H, seed=seed).view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    ids, tw = synthgen.gen_moe_routing(T, S, E, seed=seed)
    return x, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV)


def noalloc_abi(x, ids, tw, w13p, sw13, w2p, sw2, E, H, I, y):
    """The entry point called directly through the C ABI (ctypes), no binding logic in between."""
    T, S = ids.shape
    L = P.lib()
    return L.smallm_fp8bs_moe_noalloc(
        ctypes.c_void_p(x.data_ptr()), x.stride(0), ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(tw.data_ptr()),
        T, S, ctypes.c_void_p(w13p.data_ptr()), ctypes.c_void_p(sw13.data_ptr()), ctypes.c_void_p(w2p.data_ptr()),
        ctypes.c_void_p(sw2.data_ptr()), P.smallm_fp8bs_moe_layout_id(), E, H, I, ctypes.c_void_p(y.data_ptr()),
        y.stride(0), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_entry_twice_then_smaller():
    E, H, I = 65, 1024, 256
    w13p, sw13, w2p, sw2 = layer(E, H, I, seed=21)
    # first call: 24 tokens x 8 slots (192 pairs: the split down projection and its partial sums),
    # second call: 3 tokens x 4 slots (one split) into the array the first call left behind
    for T, S, seed in ((24, 8, 1), (3, 4, 2)):
        note(f"noalloc T={T} S={S}")
        need = P.smallm_fp8bs_moe_workspace_bytes(T, S, H, I)
        assert 0 < need <= P.MOE_NOALLOC_MAX_BYTES
        x, ids, tw = inputs(T, S, E, H, seed)
        y_ref, _ = P.smallm_fp8bs_moe(x, ids, tw, w13p, sw13, w2p, sw2)
        y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
        assert noalloc_abi(x, ids, tw, w13p, sw13, w2p, sw2, E, H, I, y) == P.SMALLM_OK
        torch.cuda.synchronize()
        assert torch.isfinite(y.float()).all()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"T={T} S={S}"
        # the binding's wrapper gives the same bits
        y2 = P.smallm_fp8bs_moe_noalloc(x, ids, tw, w13p, sw13, w2p, sw2)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y_ref.view(torch.int16))


def test_noalloc_refuses_workspace_beyond_its_array():
    note("noalloc size limit")
    E, H, I = 5, 16384, 2048
    T, S = 48, 16
    assert P.smallm_fp8bs_moe_workspace_bytes(T, S, H, I) > P.MOE_NOALLOC_MAX_BYTES
    # shapes only matter: the call must fail before anything is enqueued
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((T, S), dtype=torch.int32, device=DEV)
    tw = torch.zeros((T, S), dtype=torch.float32, device=DEV)
    w13p = torch.zeros((1, 1), dtype=torch.uint8, device=DEV)
    y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    L = P.lib()
    st = L.smallm_fp8bs_moe_noalloc(
        ctypes.c_void_p(x.data_ptr()), H, ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(tw.data_ptr()), T, S,
        ctypes.c_void_p(w13p.data_ptr()), ctypes.c_void_p(tw.data_ptr()), ctypes.c_void_p(w13p.data_ptr()),
        ctypes.c_void_p(tw.data_ptr()), P.smallm_fp8bs_moe_layout_id(), E, H, I, ctypes.c_void_p(y.data_ptr()), H,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == P.SMALLM_ERR_SHAPE
    assert torch.all(y == 7.0)
