"""Every HIP kernel keeps its state in registers: no private (scratch)
memory and no VGPR spills.  A register array that the compiler cannot keep
in registers, e.g. one captured by a lambda that is not inlined, moves to
scratch memory and makes a kernel several times slower without changing its
results, so the parity tests would not notice.  The compiler's resource
report for gfx950 gives both figures per kernel.  No GPU is needed."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_top_mla_smla_amd", "csrc")
SOURCES = ["attention_fp8.hip", "attention_bf16.hip", "attention_mx.hip", "attention.hip", "combine.hip",
           "quantize.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _report(src):
    obj = os.path.join("/tmp", f"smla_res_{os.getpid()}_{src}.o")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c",
           os.path.join(CSRC, src), "--cuda-device-only", "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    if os.path.exists(obj):
        os.remove(obj)
    kernels = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark: (ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")
def test_no_kernel_uses_scratch_or_spills():
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        reports = dict(zip(SOURCES, ex.map(_report, SOURCES)))
    n = 0
    bad = []
    for src, kernels in reports.items():
        for name, r in kernels.items():
            n += 1
            if r.get("ScratchSize [bytes/lane]", 0) or r.get("VGPRs Spill", 0):
                bad.append(f"{src} {name}: {r}")
    assert n >= 40, f"only {n} kernels reported"
    assert not bad, "\n".join(bad)
