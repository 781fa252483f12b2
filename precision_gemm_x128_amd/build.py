"""Ahead-of-time build of libsmallm_fp8bs.so (gfx950 only) with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "csrc", "smallm_fp8bs.hip"), os.path.join(HERE, "csrc", "moe_fp8bs.hip")]
LIB = os.path.join(HERE, "libsmallm_fp8bs.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "smallm_fp8bs.h")

# -ffp-contract=off: every multiply/add in the quantiser is the single IEEE operation written.
# No fast-math, fp32 denormals kept (hipcc defaults), correctly rounded fp32 division (default).
# Packed fp32 instructions are disabled for all HIP code on this target.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the HIP library in-tree (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
