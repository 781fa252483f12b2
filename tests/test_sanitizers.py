"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU (no GPU sanitizer is used):

* the oracle's C code, built with gcc -fsanitize=address,undefined, driven through every entry
  point on edge inputs (K = 128, ragged column windows, all-zero, subnormal and huge groups, e8m0
  extremes, every e4m3 code);
* the HIP library with the sanitizers on its host code only (argument checks, layout and launch
  plan logic, status strings), running the host ABI tests against it;
* a control: the same gcc flags on a planted out-of-bounds write, which must be reported, so a
  clean run means something.

Each run is a child Python process with the sanitizer runtime preloaded (the interpreter itself
is not instrumented); leak checking is off, any report aborts the child."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-std=c11"]


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(script, preload, timeout=600):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, OMP_NUM_THREADS="4")
    return subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                          timeout=timeout, cwd=ROOT)


def _reported(res):
    text = res.stdout + res.stderr
    return "AddressSanitizer" in text or "runtime error:" in text


@pytest.fixture(scope="module")
def asan_rt():
    rt = _gcc_runtime("libasan.so")
    if rt is None or shutil.which("gcc") is None:
        pytest.skip("gcc with libasan not available")
    return rt


def test_sanitizer_control_reports_planted_overflow(tmp_path, asan_rt):
    src = tmp_path / "bad.c"
    src.write_text("void bad(int n) { int a[4]; volatile int *p = a; for (int i = 0; i <= n; ++i) p[i] = i; }\n")
    so = tmp_path / "libbad.so"
    subprocess.check_call(["gcc", *GCC_SAN, str(src), "-o", str(so)])
    res = _run_child(f"import ctypes; ctypes.CDLL({str(so)!r}).bad(4)", asan_rt, timeout=120)
    assert res.returncode != 0 and _reported(res), res.stderr[-2000:]


ORACLE_EXERCISE = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle
    oracle._LIB = {lib!r}
    L = oracle.lib()
    rng = np.random.default_rng(7)

    # scalar codecs over their whole domains and specials
    for b in range(256):
        oracle.e4m3_decode(b)
    for v in [0.0, -0.0, 1e-30, -1e-30, 2.0 ** -9, 2.0 ** -10, 447.9, 448.0, 464.0, 1e6, -1e6,
              float('inf'), -float('inf')] + list(rng.standard_normal(2000) * 100):
        oracle.e4m3_encode(float(v))
        oracle.bf16_from_double(float(v))
    for a in [0.0, 1e-45, 1e-40, 2.0 ** -133, 1e-300, 1.0, 448.0, 449.0, 3.3e38, 1e300, float('inf')]:
        oracle.e8m0_ceil_exponent(a)
        oracle.e8m0_round_exponent(a)
    oracle.bf16_to_f32(np.arange(0, 65536, dtype=np.uint16))

    def bits(x):
        return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)

    # activation groups: zero, subnormal, huge, mixed; K = 128 and ragged row counts
    for M, K in [(1, 128), (3, 384), (17, 256)]:
        x = rng.standard_normal((M, K)).astype(np.float32)
        x[0, :128] = 0.0
        if M > 1:
            x[1, :128] = 1e-39
        if M > 2:
            x[2, :128] = 3.3e38
        for e8 in (False, True):
            q, sx = oracle.quant_act(bits(x), e8m0=e8)
    # weight blocks: zero block, tiny and huge blocks
    for N, K in [(128, 128), (256, 384)]:
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        w[:128, :128] = 0.0
        if K > 128:
            w[:128, 128:256] = 1e-40
        for e8 in (False, True):
            w8, sw = oracle.quant_weight(w, e8m0=e8)
            x = rng.standard_normal((5, K)).astype(np.float32)
            q, sx = oracle.quant_act(bits(x), e8m0=e8)
            for n0, n1 in [(0, N), (5, min(130, N)), (N - 1, N), (7, 7)]:
                for th in (0, 1):
                    ref = oracle.gemm(q, sx, w8, sw, e8m0=e8, n0=n0, n1=n1, threads=th)
            oracle.round_bf16(ref)
            oracle.quant_gemm(bits(x), w8, sw, e8m0=e8, n0=3, n1=N - 2, threads=2)
            try:
                oracle.gemm(q, sx, w8, sw, e8m0=e8, n0=5, n1=N + 2)   # out of range: refused
                raise SystemExit("an out-of-range column window was accepted")
            except ValueError:
                pass
    print("oracle exercise done")
""")


def test_oracle_clean_under_asan_ubsan(tmp_path, asan_rt):
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", *GCC_SAN, os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(lib), "-lm"])
    res = _run_child(ORACLE_EXERCISE.format(root=ROOT, lib=str(lib)), asan_rt)
    assert res.returncode == 0 and not _reported(res), (res.stdout[-2000:], res.stderr[-4000:])
    assert "oracle exercise done" in res.stdout


HOST_ABI_RUN = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    import precision_gemm_x128_amd as P
    P.LIB_PATH = {lib!r}
    import pytest
    sys.exit(pytest.main([{test!r}, "-q", "-p", "no:cacheprovider"]))
""")


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_host_abi_clean_under_asan_ubsan(tmp_path):
    import glob
    rts = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang ASan runtime not found")
    from precision_gemm_x128_amd import build as B
    lib = tmp_path / "libsmallm_fp8bs_san.so"
    # host code only: every sanitizer flag goes to the host compilation (-Xarch_host)
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-O3",)] + [
        "-O1", "-g",
        "-Xarch_host", "-fsanitize=address",
        "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined",
        "-Xarch_host", "-fno-omit-frame-pointer",
        "-shared-libsan"]
    res = subprocess.run([HIPCC, *flags, *B.SRCS, "-o", str(lib)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    run = HOST_ABI_RUN.format(root=ROOT, lib=str(lib), test=os.path.join(ROOT, "tests", "test_abi_host.py"))
    out = _run_child(run, rts[-1])
    assert out.returncode == 0 and not _reported(out), (out.stdout[-3000:], out.stderr[-4000:])
