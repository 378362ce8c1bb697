"""Compiler resource checks on the gfx950 device code (CPU only: hipcc
cross-compiles). Every kernel must keep its working set in registers and LDS:
a per-thread array with a run-time index, or a register spill, moves data to
scratch memory, which costs the sweep tens of microseconds per launch while
still giving correct results, so the parity tests cannot see it."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "partitioned_chip_accumulation_amd", "csrc")


def kernel_resources(source, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-c",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, source),
           "-o", str(tmp_path / "dev.o"), "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kernels, name = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.parametrize("source", ["hist_api.hip", "hist_bench.hip"])
def test_no_scratch_and_no_vgpr_spills(source, tmp_path):
    kernels = kernel_resources(source, tmp_path)
    assert kernels, "no kernel resource remarks parsed"
    bad = {k: v for k, v in kernels.items()
           if v.get("ScratchSize", 0) != 0 or v.get("VGPRs Spill", 0) != 0}
    assert not bad, bad
