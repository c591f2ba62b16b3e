"""LDS reads issued through inline asm (the transposed reads and some 16-byte
reads of the attention kernels) return registers that the compiler treats as
written at once; the kernels wait for them with an explicit s_waitcnt.  If
the compiler ever moved or reused such a register before that wait, the
kernel would read stale data (or the load would land in a register that
holds something else by then).

This test compiles the attention kernels to gfx950 assembly and walks each
kernel's instructions in order, tracking the LDS reads in flight: LDS
operations complete in order, so after `s_waitcnt lgkmcnt(k)` at most the k
most recent LDS operations can still be pending.  No instruction may read or
write a register that a pending LDS read still has to fill.  The walk
follows the instruction order, not the branches; after an unconditional
branch the next instruction is not reached from the one before it, so the
walk starts over there with nothing pending.  No GPU is needed.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_top_mla_smla_amd", "csrc")
SOURCES = ["attention_fp8.hip", "attention_bf16.hip", "attention_mx.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vregs(text):
    out = set()
    for a, b, c in VREG.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def _assemble(src):
    out = os.path.join("/tmp", f"smla_isa_{os.getpid()}_{src}.s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c",
           os.path.join(CSRC, src), "--cuda-device-only", "-S", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        text = f.read()
    os.remove(out)
    return text


def _kernels(asm):
    """(name, [instruction lines]) of every kernel in an assembly file."""
    for m in re.finditer(r"^(_Z\w+):(?:\s*;.*)?$", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        body = asm[m.end():end if end > 0 else len(asm)]
        ins = []
        for line in body.splitlines():
            line = line.split(";")[0].strip()
            if line and not line.startswith(".") and not line.endswith(":"):
                ins.append(line)
        yield m.group(1), ins


def hazards(ins):
    """Instructions that touch a register an LDS read in flight still has to fill."""
    lds = []  # (is_read, destination registers) of LDS operations not known to be done, in issue order
    found = []
    for line in ins:
        op = line.split()[0]
        w = re.match(r"s_waitcnt\b.*lgkmcnt\((\d+)\)", line)
        if w:
            k = int(w.group(1))
            lds = lds[len(lds) - k:] if 0 < k < len(lds) else ([] if k == 0 else lds)
            continue
        pending = set()
        for is_read, regs in lds:
            if is_read:
                pending |= regs
        if op.startswith("ds_"):
            operands = line[len(op):]
            if op.startswith("ds_read") or op.startswith("ds_load"):
                dst, _, srcs = operands.partition(",")
                if _vregs(srcs) & pending:
                    found.append(line)
                lds.append((True, _vregs(dst)))
            else:
                if _vregs(operands) & pending:
                    found.append(line)
                lds.append((False, set()))
            continue
        if op in ("s_branch", "s_setpc_b64", "s_endpgm"):
            lds = []
            continue
        if op.startswith("s_"):
            continue
        if _vregs(line[len(op):]) & pending:
            found.append(line)
    return found


def test_hazard_walk_finds_a_copy_before_the_wait():
    ins = ["ds_read_b128 v[4:7], v171 offset:96", "v_mov_b64_e32 v[126:127], v[6:7]", "s_waitcnt lgkmcnt(0)"]
    assert hazards(ins) == ["v_mov_b64_e32 v[126:127], v[6:7]"]
    ok = ["ds_read_b128 v[4:7], v171", "ds_read_b128 v[8:11], v171 offset:16", "s_waitcnt lgkmcnt(1)",
          "v_mov_b32_e32 v1, v4", "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v2, v9"]
    assert hazards(ok) == []
    bad = ["ds_read_b128 v[4:7], v171", "ds_read_b128 v[8:11], v171 offset:16", "s_waitcnt lgkmcnt(1)",
           "v_mov_b32_e32 v2, v9"]
    assert hazards(bad) == ["v_mov_b32_e32 v2, v9"]
    # the block after an unconditional branch is reached from elsewhere
    jump = ["ds_read_b128 v[4:7], v171", "s_branch .LBB0_7", "ds_read_b128 v[8:11], v5", "s_waitcnt lgkmcnt(0)"]
    assert hazards(jump) == []
    fall = ["ds_read_b128 v[4:7], v171", "s_cbranch_scc1 .LBB0_7", "ds_read_b128 v[8:11], v5"]
    assert hazards(fall) == ["ds_read_b128 v[8:11], v5"]


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")
def test_no_register_of_a_pending_lds_read_is_touched():
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        asms = dict(zip(SOURCES, ex.map(_assemble, SOURCES)))
    checked = 0
    problems = []
    for src, asm in asms.items():
        for name, ins in _kernels(asm):
            if not any(i.startswith("ds_read") for i in ins):
                continue
            checked += 1
            for line in hazards(ins)[:3]:
                problems.append(f"{src} {name}: {line}")
    assert checked >= 20, f"only {checked} kernels with LDS reads found"
    assert not problems, "\n".join(problems)
