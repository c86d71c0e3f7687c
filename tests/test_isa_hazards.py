"""Hazards the compiler cannot see, checked in the gfx950 assembly of the
attention kernels (built here with the library's own flags; no GPU needed).

The kernels issue a few instructions as inline asm: the direct HBM -> LDS
loads (which set M0 with a scalar add, so they write SCC) and the dK/dV
MFMAs with accumulation-register accumulators.  The compiler's hazard
recognizer does not look inside inline asm, so the kernels keep the
distances themselves, and these scans check that they do:
  - no SCC read (s_cselect, s_cbranch_scc*, s_addc / s_subb, s_cmovk) takes
    the value an asm block left in SCC: a compiler write of SCC must come
    first (an undeclared SCC clobber once made a select read the M0 add's
    carry);
  - no inline-asm instruction reads, in the very next slot, the result of a
    transcendental VALU op (gfx950 needs one wait state there, which the
    compiler inserts only for its own instructions);
  - every asm MFMA's A, B and C registers were last written by a VALU
    instruction at least two wait states earlier;
  - no kernel spills to scratch.
"""

import os
import re
import shutil
import subprocess

import pytest

from prefix_tree_attention_amd import build as libbuild

SOURCES = ["fwd_bf16.hip", "bwd_bf16.hip"]


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    if not os.path.exists(libbuild.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    out = {}
    for src in SOURCES:
        s = d / (src + ".s")
        cmd = [libbuild.HIPCC, *[f for f in libbuild.COMMON if f != "-fPIC"], *libbuild.HIP_FLAGS,
               "--cuda-device-only", "-S", os.path.join(libbuild.CSRC, src), "-o", str(s)]
        subprocess.run(cmd, check=True, capture_output=True)
        out[src] = s.read_text().split("\n")
    return out


def _kernels(lines):
    """(name, [(text, in_asm)]) per kernel function."""
    res, cur, name, in_asm = [], None, None, False
    for ln in lines:
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            name, cur, in_asm = m.group(1), [], False
            continue
        if cur is None:
            continue
        if ln.startswith(".Lfunc_end"):
            res.append((name, cur))
            cur = None
            continue
        t = ln.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        cur.append((t.split(";")[0].strip(), in_asm))
    return res


def _regs(op):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", op):
        if m.group(1):
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _operands(t):
    parts = t.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


TRANS = re.compile(r"^v_(exp|log|rcp|rsq|sqrt|sin|cos)_")
SCC_READ = re.compile(r"^s_(cselect|cbranch_scc|addc|subb|cmovk|cmov_)")
# scalar ops that write SCC (the ones that can appear here)
SCC_WRITE = re.compile(r"^s_(add_|sub_|addc|subb|and_|or_|xor_|andn2|orn2|nand|nor|xnor|lshl|lshr|ashr|bfe|"
                       r"cmp_|min_|max_|abs|not_|bitcmp|mul_hi)")


def _is_valu_write(t):
    op = t.split()[0]
    return op.startswith("v_") and not op.startswith(("v_mfma", "v_cmp", "v_readlane", "v_readfirstlane",
                                                       "v_writelane", "v_nop"))


def _wait_states(t):
    m = re.match(r"^s_nop\s+(\d+)", t)
    return int(m.group(1)) + 1 if m else 1


@pytest.mark.parametrize("src", SOURCES)
def test_no_scc_read_after_asm_write(isa, src):
    bad = []
    for name, body in _kernels(isa[src]):
        asm_scc = False
        for t, in_asm in body:
            op = t.split()[0]
            if in_asm:
                if SCC_WRITE.match(op):
                    asm_scc = True
                continue
            if SCC_READ.match(op) and asm_scc:
                bad.append((name[:60], t))
            if SCC_WRITE.match(op) or op.startswith("s_cmp"):
                asm_scc = False
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_no_asm_read_of_fresh_transcendental(isa, src):
    bad = []
    for name, body in _kernels(isa[src]):
        for (pt, _), (t, in_asm) in zip(body, body[1:]):
            if in_asm and TRANS.match(pt.split()[0]):
                dst = _regs(_operands(pt)[0])
                srcs = set().union(*[_regs(o) for o in _operands(t)[1:]]) if len(_operands(t)) > 1 else set()
                if dst & srcs:
                    bad.append((name[:60], pt, t))
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_asm_mfma_operands_two_wait_states_after_valu(isa, src):
    bad, n_mfma = [], 0
    for name, body in _kernels(isa[src]):
        for i, (t, in_asm) in enumerate(body):
            if not (in_asm and t.startswith("v_mfma")):
                continue
            n_mfma += 1
            reads = set().union(*[_regs(o) for o in _operands(t)[1:]])
            ws = 0
            for j in range(i - 1, max(-1, i - 8), -1):
                pt, _ = body[j]
                if _is_valu_write(pt) and _regs(_operands(pt)[0]) & reads and ws < 2:
                    bad.append((name[:60], pt, t, ws))
                ws += _wait_states(pt)
                if ws >= 2:
                    break
    assert not bad, bad[:5]
    if src == "bwd_bf16.hip":
        assert n_mfma > 0  # the dK/dV kernels do issue asm MFMAs


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(isa, src):
    sizes = [int(m.group(1)) for ln in isa[src] for m in [re.match(r"^; ScratchSize: (\d+)", ln.strip())] if m]
    assert sizes and all(s == 0 for s in sizes), sizes
