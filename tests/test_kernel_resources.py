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


LLVM_BIN = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def parse_remarks(stderr):
    kernels, name = {}, None
    for line in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


def disassemble_by_kernel(listing):
    """Split llvm-objdump's listing into {symbol: [instruction lines]}."""
    out, name = {}, None
    for line in listing.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            name = m.group(1)
            out[name] = []
        elif name and line.startswith("\t"):
            out[name].append(line.strip())
    return out


@pytest.fixture(scope="module", params=["hist_api.hip", "hist_bench.hip"])
def device_build(request, tmp_path_factory):
    """One device-only compile of a source: the resource remarks of every
    kernel and the gfx950 disassembly of its code object."""
    source = request.param
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    bundler = os.path.join(LLVM_BIN, "clang-offload-bundler")
    objdump = os.path.join(LLVM_BIN, "llvm-objdump")
    if not all(os.path.exists(t) for t in (hipcc, bundler, objdump)):
        pytest.skip("ROCm compiler tools not available")
    tmp = tmp_path_factory.mktemp(source.replace(".", "_"))
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-c",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, source),
           "-o", str(tmp / "dev.o"), "-Rpass-analysis=kernel-resource-usage"]
    remarks = parse_remarks(subprocess.run(cmd, capture_output=True, text=True,
                                           check=True).stderr)
    subprocess.run([bundler, "--unbundle", "--type=o", "--input=" + str(tmp / "dev.o"),
                    "--targets=" + TARGET, "--output=" + str(tmp / "co.o")], check=True)
    listing = subprocess.run([objdump, "-d", str(tmp / "co.o")], capture_output=True,
                             text=True, check=True).stdout
    return source, remarks, disassemble_by_kernel(listing)


def test_no_scratch_and_no_vgpr_spills(device_build):
    _, kernels, _ = device_build
    assert kernels, "no kernel resource remarks parsed"
    bad = {k: v for k, v in kernels.items()
           if v.get("ScratchSize", 0) != 0 or v.get("VGPRs Spill", 0) != 0}
    assert not bad, bad


def test_no_run_time_register_indexing(device_build):
    """The 8-bit counters' carry events update one of 32 per-lane counts chosen
    at run time, through a tree of scalar branches whose leaves name their
    registers as constants. A compiler that merges the leaves into one update
    at a run-time register index (GPR indexing mode, or the movrel moves) has
    given wrong counts on a Zipf workload, and only a full-size GPU run would
    show it; no kernel here needs either form, so any occurrence fails."""
    _, _, code = device_build
    assert len(code) >= 10, "no kernels found in the disassembly"
    forms = ("s_set_gpr_idx", "v_movrels", "v_movreld", "v_movrelsd")
    bad = {k: [i for i in ins if i.split()[0].startswith(forms)]
           for k, ins in code.items()}
    bad = {k: v[:3] for k, v in bad.items() if v}
    assert not bad, bad



def test_sweep_kernels_declare_no_static_lds(device_build):
    """The sweep addresses its counters by their offset into the dynamic LDS
    block, with no base added, which holds only while the block starts at
    LDS address 0: the kernel must declare no static LDS of its own."""
    source, kernels, _ = device_build
    if source != "hist_api.hip":
        pytest.skip("the sweep kernels live in the library source")
    sweeps = {k: v for k, v in kernels.items() if "k_sweep" in k}
    assert sweeps, "no sweep kernel in the resource remarks"
    assert all("LDS Size" in v for v in sweeps.values()), sweeps
    bad = {k: v["LDS Size"] for k, v in sweeps.items() if v["LDS Size"] != 0}
    assert not bad, bad
