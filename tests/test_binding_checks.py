"""The Python binding is the only guard on sizes the C entry points cannot see: every tensor the
kernels read or write must be a device tensor of the exact shape, dtype and density they assume.
The CPU tests drive the validation helpers directly; the GPU tests call the entry points with one
bad argument at a time and expect the error before anything is launched."""
import pytest
import torch

import precision_gemm_x128_amd as P

GPU = torch.cuda.is_available()


# ---------------------------------------------------------------------------------------------
# the helpers, on the CPU
# ---------------------------------------------------------------------------------------------

def test_need_exact_rejects_host_tensors():
    with pytest.raises(ValueError, match="device tensor"):
        P._need_exact(torch.zeros((4, 8), dtype=torch.float32), (torch.float32,), (4, 8), "sx_dbg")


def test_need_exact_rejects_non_tensors_and_wrong_dtype():
    with pytest.raises(TypeError, match="must be a torch.Tensor"):
        P._need_exact([[0.0]], (torch.float32,), (1, 1), "sw")
    with pytest.raises(TypeError, match="dtype"):
        P._need_exact(torch.zeros((4, 8), dtype=torch.uint8), (torch.float32,), (4, 8), "sx_dbg")


def test_need_rows_rejects_host_and_wrong_dtype():
    with pytest.raises(ValueError, match="device tensor"):
        P._need_rows(torch.zeros((2, 256), dtype=torch.uint8), 2, 256, "q", torch.device("cpu"))
    with pytest.raises(TypeError, match="dtype"):
        P._need_rows(torch.zeros((2, 256), dtype=torch.float32), 2, 256, "q", torch.device("cpu"))


def test_check_dbg_validates_both_copies():
    # nothing to check without debug outputs
    P._check_dbg(None, None, 4, 256, False, torch.device("cpu"))
    with pytest.raises(ValueError, match="q_dbg"):
        P._check_dbg(torch.zeros((4, 256), dtype=torch.uint8), None, 4, 256, False, torch.device("cpu"))
    with pytest.raises(TypeError, match="dtype"):
        # fp32 scales expected, e8m0 bytes given
        P._check_dbg(None, torch.zeros((4, 2), dtype=torch.uint8), 4, 256, False, torch.device("cpu"))
    with pytest.raises(TypeError, match="dtype"):
        P._check_dbg(None, torch.zeros((4, 2), dtype=torch.float32), 4, 256, True, torch.device("cpu"))


def test_binding_wraps_the_entry_points():
    # every C entry point the header declares is reachable from Python: a wrapper of the same name,
    # or (the workspace variants) through the wrapper that dispatches to it
    via = {"smallm_fp8bs_quant_gemm_ws": "smallm_fp8bs_quant_gemm",
           "smallm_fp8bs_quant_gemm_e8m0_ws": "smallm_fp8bs_quant_gemm_e8m0",
           "smallm_fp8bs_strerror": "strerror"}
    for name in P.EXPORTS:
        assert callable(getattr(P, via.get(name, name), None)), name


def test_need_rejects_host_activations():
    with pytest.raises(ValueError, match="device tensor"):
        P._need(torch.zeros((4, 256), dtype=torch.bfloat16), (torch.bfloat16,), "x")


# ---------------------------------------------------------------------------------------------
# the entry points, on the GPU (every call below must fail in the binding, before a launch)
# ---------------------------------------------------------------------------------------------

def _operands(M=4, N=512, K=1024, e8m0=False):
    dev = "cuda:0"
    x = torch.randn((M, K), device=dev).to(torch.bfloat16)
    wp = torch.zeros((N, K), dtype=torch.uint8, device=dev)
    sw = torch.ones((N // 128, K // 128), dtype=torch.uint8 if e8m0 else torch.float32, device=dev)
    return x, wp, sw


@pytest.mark.gpu
@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_rejects_bad_debug_outputs(e8m0):
    M, K = 4, 1024
    x, wp, sw = _operands(M=M, K=K, e8m0=e8m0)
    fn = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    sdt = torch.uint8 if e8m0 else torch.float32
    wrong = torch.float32 if e8m0 else torch.uint8
    bad_q = [torch.zeros((M, K - 128), dtype=torch.uint8, device="cuda:0"),          # short
             torch.zeros((M, 2 * K), dtype=torch.uint8, device="cuda:0")[:, :K],     # strided
             torch.zeros((M, K), dtype=torch.uint8)]                                  # host
    for q in bad_q:
        with pytest.raises((ValueError, TypeError)):
            fn(x, wp, sw, q_dbg=q)
    bad_s = [torch.zeros((M, K // 128), dtype=wrong, device="cuda:0"),
             torch.zeros((M - 1, K // 128), dtype=sdt, device="cuda:0"),
             torch.zeros((M, K // 128), dtype=sdt)]
    for s in bad_s:
        with pytest.raises((ValueError, TypeError)):
            fn(x, wp, sw, sx_dbg=s)


@pytest.mark.gpu
def test_gemm_entries_reject_host_scales():
    M, N, K = 4, 512, 1024
    x, wp, sw = _operands(M, N, K)
    with pytest.raises(ValueError, match="device tensor"):
        P.smallm_fp8bs_quant_gemm(x, wp, sw.cpu())
    q = torch.zeros((M, K), dtype=torch.uint8, device="cuda:0")
    sx = torch.ones((M, K // 128), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError, match="device tensor"):
        P.smallm_fp8bs_gemm(q, sx.cpu(), wp, sw)
    with pytest.raises(ValueError, match="device tensor"):
        P.smallm_fp8bs_gemm(q, sx, wp, sw.cpu())


@pytest.mark.gpu
def test_quant_rejects_bad_outputs():
    M, K = 4, 1024
    x = torch.randn((M, K), device="cuda:0").to(torch.bfloat16)
    with pytest.raises(ValueError):
        P.smallm_fp8bs_quant(x, q=torch.zeros((M, K - 128), dtype=torch.uint8, device="cuda:0"))
    with pytest.raises(TypeError):
        P.smallm_fp8bs_quant(x, sx=torch.zeros((M, K // 128), dtype=torch.uint8, device="cuda:0"))
    with pytest.raises(ValueError):
        P.smallm_fp8bs_quant_e8m0(x, sx=torch.zeros((M, K // 128), dtype=torch.uint8))


@pytest.mark.gpu
def test_moe_rejects_host_scales():
    T, S, E, H, I = 2, 2, 4, 256, 256
    dev = "cuda:0"
    x = torch.randn((T, H), device=dev).to(torch.bfloat16)
    ids = torch.zeros((T, S), dtype=torch.int32, device=dev)
    tw = torch.ones((T, S), dtype=torch.float32, device=dev)
    w13 = torch.zeros((E, 2 * I, H), dtype=torch.uint8, device=dev)
    w2 = torch.zeros((E, H, I), dtype=torch.uint8, device=dev)
    sw13 = torch.ones((E, 2 * I // 128, H // 128), dtype=torch.float32, device=dev)
    sw2 = torch.ones((E, H // 128, I // 128), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="device tensor"):
        P.smallm_fp8bs_moe(x, ids, tw, w13, sw13.cpu(), w2, sw2)
    with pytest.raises(ValueError, match="device tensor"):
        P.smallm_fp8bs_moe(x, ids, tw, w13, sw13, w2, sw2.cpu())
    with pytest.raises(ValueError, match="device tensor"):
        P.smallm_fp8bs_moe(x, ids, tw, w13, sw13, w2, sw2, workspace=torch.zeros(1 << 20, dtype=torch.uint8))


@pytest.mark.gpu
def test_read_floor_streams_without_writing():
    # the roofline reference kernel: reads every byte (ragged sizes too) and leaves the sink alone
    for nbytes in (16, 1 << 20, (20 << 20) + 4096):
        buf = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda:0")
        P.smallm_fp8bs_read_floor(buf)
        torch.cuda.synchronize()
    sink = P._floor_sink[torch.device("cuda:0")]
    assert int(sink.abs().sum().item()) == 0
    with pytest.raises(ValueError):
        P.smallm_fp8bs_read_floor(torch.zeros(64, dtype=torch.uint8))
