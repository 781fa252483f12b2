"""Checks on the compiled device code (no GPU needed): the compiler's assembly for gfx950 is read
per kernel.

* No kernel spills: a scratch reload shares the in-order vector-memory counter with the weight and
  activation loads, so a single spill would make a wave wait for every load in flight (and the
  spill stores are HBM traffic).
* No MFMA result reaches a non-MFMA reader through a branch within 12 wait states.  A matrix
  instruction writes its destination several passes after it issues, and the reader must be that
  many instructions behind.  Inside one basic block the compiler counts them; on a path through a
  branch it has been seen to place the reader two instructions after the MFMA, which read stale
  registers on the GPU.  12 covers the longest instruction used here (16 passes, CDNA3/CDNA4 ISA
  dependency tables)."""
import os
import re
import shutil
import subprocess

import pytest

from precision_gemm_x128_amd import build as B

HAVE_HIPCC = shutil.which(B.hipcc()) is not None or os.path.exists(B.hipcc())
WAIT_STATES = 12


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    tmp = tmp_path_factory.mktemp("asm")
    text = ""
    for i, src in enumerate(B.SRCS):
        out = tmp / f"dev{i}.s"
        cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", src, "-o", str(out)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        text += out.read_text()
    return text


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not found")
def test_gemm_kernels_use_no_scratch(device_asm):
    text = device_asm
    kernels = re.findall(r"^(_Z\S*smallm_gemm_kernel\S*):", text, re.M)
    assert len(kernels) >= 64
    others = re.findall(r"^(_Z\S*rmsnorm_quant_kernel\S*):", text, re.M)
    assert len(others) == 2
    moe = re.findall(r"^(_Z\S*moe_(?:gate_up_pairs|gate_up_items|down)_kernel\S*):", text, re.M)
    assert len(moe) == 10
    tiled = re.findall(r"^(_Z\S*tiled_gemm_kernel\S*):", text, re.M)
    assert len(tiled) == 28
    kernels += others + moe + tiled
    spills = []
    for k in kernels:
        seg = text[text.index(k + ":"):]
        m = re.search(r"; ScratchSize: (\d+)", seg)
        assert m, k
        if int(m.group(1)) != 0:
            spills.append((k, int(m.group(1))))
    assert not spills, spills


def _vregs(tok):
    m = re.match(r"-?v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"-?v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(inst):
    return [o.strip() for o in inst.split(None, 1)[1].split(",")] if " " in inst else []


def _functions(text):
    funcs, fn = {}, None
    for ln in text.split("\n"):
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            fn = m.group(1)
            funcs[fn] = []
            continue
        if fn is None:
            continue
        s = ln.split(";")[0].strip()
        if not s:
            continue
        if s.startswith(".LBB") and s.endswith(":"):
            funcs[fn].append(("label", s[:-1]))
        elif not s.startswith("."):
            funcs[fn].append(("inst", s))
            if s.startswith("s_endpgm"):
                fn = None
    return funcs


def mfma_cross_block_reads(text, limit=WAIT_STATES):
    """Every (kernel, mfma, reader, wait states) where a non-MFMA instruction reads an MFMA's
    destination, or an MFMA reads it as an A/B operand, fewer than `limit` wait states after it on
    a path that crosses a branch or label."""
    found = []
    for fn, items in _functions(text).items():
        labels = {name: i for i, (k, name) in enumerate(items) if k == "label"}

        def succ(i):
            k, s = items[i]
            out = []
            if k == "inst":
                if s.startswith("s_branch"):
                    return [labels[s.split()[1]]]
                if s.startswith("s_cbranch"):
                    out.append(labels[s.split()[1]])
                if s.startswith("s_endpgm") or s.startswith("s_setpc"):
                    return []
            if i + 1 < len(items):
                out.append(i + 1)
            return out

        for i, (k, s) in enumerate(items):
            if k != "inst" or not s.startswith("v_mfma"):
                continue
            dst = _vregs(_operands(s)[0])
            stack = [(j, 0, False) for j in succ(i)]
            seen = set()
            while stack:
                j, dist, crossed = stack.pop()
                if dist >= limit or (j, dist, crossed) in seen:
                    continue
                seen.add((j, dist, crossed))
                kk, t = items[j]
                if kk == "label":
                    stack += [(n, dist, True) for n in succ(j)]
                    continue
                ops = _operands(t)
                if t.startswith("v_mfma"):
                    ab = set().union(*[_vregs(o) for o in ops[1:3]])
                    if crossed and dst & ab:
                        found.append((fn, s, t, dist))
                    if dst & _vregs(ops[0]) and not dst & ab:
                        continue
                    w = dist + 1
                elif t.startswith("s_nop"):
                    w = dist + int(t.split()[1]) + 1
                else:
                    if crossed and t[:2] in ("v_", "ds", "gl", "bu") and dst & set().union(set(), *[_vregs(o) for o in ops]):
                        found.append((fn, s, t, dist))
                        continue
                    w = dist + 1
                branch = t.startswith("s_cbranch") or t.startswith("s_branch")
                stack += [(n, w, crossed or branch) for n in succ(j)]
    return found


def test_hazard_check_finds_a_planted_case():
    # an MFMA whose result is read two instructions after a branch to the reader's block
    text = """_Zdemo:
	v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0
	s_cbranch_vccz .LBB0_2
	s_nop 7
	s_nop 7
.LBB0_2:
	s_waitcnt vmcnt(0)
	v_mul_f32_e32 v0, v12, v0
	s_endpgm
"""
    hits = mfma_cross_block_reads(text)
    assert len(hits) == 1 and hits[0][3] == 2
    # the same read behind enough wait states on every path is accepted
    safe = text.replace("s_cbranch_vccz .LBB0_2\n", "s_nop 7\n\ts_nop 7\n\ts_cbranch_vccz .LBB0_2\n")
    assert mfma_cross_block_reads(safe) == []


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not found")
def test_no_mfma_result_read_early_across_a_branch(device_asm):
    hits = mfma_cross_block_reads(device_asm)
    assert not hits, [(f[:80], m[:50], r[:50], d) for f, m, r, d in hits[:10]]
