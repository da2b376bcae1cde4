"""Compiler resource report of the HIP kernels (CPU, no GPU needed): no kernel
may use scratch memory.  A spill in the verification or statistics kernels
costs far more than its instruction count (the hierarchical verification went
from 46 to 76 us per launch when a second inlined draw pushed it into
scratch), so the build is checked for it directly."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_token_verification_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _resources(src):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang",
           "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-c",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, os.path.join(CSRC, src),
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    report, name = {}, None
    for line in out.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            report.setdefault(name, {})[m.group(1).split()[0]] = int(m.group(2))
    return report


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("ld.lld") is None and
                    not os.path.exists("/opt/rocm/llvm/bin/ld.lld"),
                    reason="hipcc is not installed")
@pytest.mark.parametrize("src", ["verify.hip", "rowstats.hip", "byproducts.hip",
                                 "tentative.hip", "lmhead.hip"])
def test_no_kernel_uses_scratch(src):
    rep = _resources(src)
    assert rep, "no kernels reported"
    spilled = {k: v for k, v in rep.items() if v.get("ScratchSize", 0) != 0}
    assert not spilled, spilled
