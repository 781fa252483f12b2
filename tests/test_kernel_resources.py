"""The GEMM, producer and MoE kernels must not spill: a scratch reload shares the in-order vector-memory counter with
the weight and activation loads, so a single spill would make a wave wait for every load in flight
(and the spill stores are HBM traffic).  Compiles the device code (no GPU needed) and reads the
per-kernel resource summary the compiler writes into the assembly."""
import os
import re
import shutil
import subprocess

import pytest

from precision_gemm_x128_amd import build as B


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()), reason="hipcc not found")
def test_gemm_kernels_use_no_scratch(tmp_path):
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    text = ""
    for i, src in enumerate(B.SRCS):
        out = tmp_path / f"dev{i}.s"
        cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", src, "-o", str(out)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        text += out.read_text()
    kernels = re.findall(r"^(_Z\S*smallm_gemm_kernel\S*):", text, re.M)
    assert len(kernels) >= 64
    others = re.findall(r"^(_Z\S*(?:tiled_gemm_kernel|rmsnorm_quant_kernel)\S*):", text, re.M)
    assert len(others) == 4
    moe = re.findall(r"^(_Z\S*moe_(?:gate_up|down)_kernel\S*):", text, re.M)
    assert len(moe) == 6
    kernels += others + moe
    spills = []
    for k in kernels:
        seg = text[text.index(k + ":"):]
        m = re.search(r"; ScratchSize: (\d+)", seg)
        assert m, k
        if int(m.group(1)) != 0:
            spills.append((k, int(m.group(1))))
    assert not spills, spills
