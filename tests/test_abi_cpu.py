"""C-ABI checks that need no GPU: the library loads, exports every symbol
that include/*.h declares, and rejects bad arguments with the documented
status before touching a device."""
from __future__ import annotations

import ctypes
import glob
import os
import re
import shutil
import subprocess

import pytest

from partitioned_chip_accumulation_amd import hist

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"\b(hist_[a-z_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_headers_declare_the_expected_calls():
    names = declared_functions()
    for must in ["hist_plan", "hist_plan_create", "hist_run", "hist_workspace_size", "hist_plan_destroy",
                 "hist_status_str", "hist_bench_global_atomic", "hist_plan_preview",
                 "hist_run_accumulate", "hist_tune", "hist_tune_workspace_size", "hist_run_static",
                 "hist_predict", "hist_select", "hist_model_calibration",
                 "hist_bench_lds_latency", "hist_bench_handoff", "hist_plan_check",
                 "hist_plan_stream_trace"]:
        assert must in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_declared_symbol(name):
    lib = ctypes.CDLL(hist.LIBRARY)
    assert hasattr(lib, name), name


def test_status_strings():
    lib = hist.library()
    for s in range(5):
        assert lib.hist_status_str(s)
    assert lib.hist_status_str(99) == b"unknown status"


def test_argument_errors_before_any_device_call():
    lib = hist.library()
    n = ctypes.c_uint64(0)
    assert lib.hist_workspace_size(0, 10, None, ctypes.byref(n)) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_workspace_size(10, 10, None, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_workspace_size(10, 2**32, None, ctypes.byref(n)) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_workspace_size(hist.MAX_BINS + 1, 10, None,
                                   ctypes.byref(n)) == hist.HIST_ERR_UNSUPPORTED
    for field, bad in [("path", 7), ("groups", -1), ("range_bins", 6), ("range_bins", 1000),
                       ("counter_bits", 12), ("aggregation", 3), ("lds_copies", 3),
                       ("lds_copies", 32),
                       ("aggregation", -2), ("wg_size", 100), ("xcd_map", 5)]:
        o = hist.PlanOpts()
        o.aggregation = -1
        setattr(o, field, bad)
        assert lib.hist_workspace_size(10, 10, ctypes.byref(o),
                                       ctypes.byref(n)) == hist.HIST_ERR_INVALID_ARG, field
    p = ctypes.c_void_p()
    assert lib.hist_plan(None, 10, 10, None, None, 0) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan(ctypes.byref(p), 0, 10, None, None, 0) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan(ctypes.byref(p), 10, 10, None, 3, 0) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_create(None, 10, 10, None, None, 0) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_create(ctypes.byref(p), 0, 10, None, None, 0) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_create(ctypes.byref(p), 10, 10, None, 3, 0) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_run(None, None, None, 0, 1, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_run_static(None, None, 0, 1, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_run_static(16, None, 5, 8, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_run_static(16, None, 0, 0, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_run_accumulate(None, None, None, 0, 1, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_info(None, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_tune_workspace_size(10, 10, None) == hist.HIST_ERR_INVALID_ARG
    best = hist.PlanOpts()
    cnt = ctypes.c_uint32(0)
    entries = (hist.TuneEntry * hist.TUNE_MAX_ENTRIES)()
    for args in [(10, 10, None, 5, 8, None, 0, 1),      # no input
                 (10, 10, 8, 5, None, None, 0, 1),      # no counts
                 (10, 10, 8, 0, 8, None, 0, 1),         # n == 0
                 (10, 10, 8, 11, 8, None, 0, 1),        # n > max_n
                 (10, 10, 8, 5, 8, None, 0, 0),         # reps == 0
                 (10, 10, 8, 5, 8, None, 0, 1001),      # reps > 1000
                 (10, 10, 8, 5, 8, 4, 4096, 1)]:        # workspace not 256-byte aligned
        assert lib.hist_tune(*args, None, ctypes.byref(best), entries, hist.TUNE_MAX_ENTRIES,
                             ctypes.byref(cnt)) == hist.HIST_ERR_INVALID_ARG, args
    assert lib.hist_tune(10, 10, 8, 5, 8, None, 0, 1, None, None, entries, 1,
                         ctypes.byref(cnt)) == hist.HIST_ERR_INVALID_ARG  # no best
    assert lib.hist_tune(10, 10, 8, 5, 8, None, 0, 1, None, ctypes.byref(best), None, 1,
                         ctypes.byref(cnt)) == hist.HIST_ERR_INVALID_ARG  # no entries
    assert lib.hist_plan_timing_enable(None, 4) == hist.HIST_ERR_INVALID_ARG
    g = ctypes.c_uint32(7)
    assert lib.hist_plan_check(None, None, ctypes.byref(g)) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_plan_stream_trace(None, None, None, 0, ctypes.byref(g)) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_bench_global_atomic(None, None, 0, 1, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_bench_copy(None, None, 16, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_bench_lds_atomic(4, 0, 1, None, 0, None) == hist.HIST_ERR_INVALID_ARG
    assert lib.hist_bench_lds_atomic(0, 0, 0, None, 0, None) == hist.HIST_ERR_INVALID_ARG
    lib.hist_plan_destroy(None)


def test_no_device_is_unsupported_not_a_crash():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = hist.library()
    n = ctypes.c_uint64(0)
    assert lib.hist_workspace_size(65536, 1 << 20, None,
                                   ctypes.byref(n)) == hist.HIST_ERR_UNSUPPORTED
    assert lib.hist_tune_workspace_size(65536, 1 << 20,
                                        ctypes.byref(n)) == hist.HIST_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(hist.LibraryMissing):
        hist.load(str(tmp_path / "missing.so"))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "partitioned_chip_accumulation_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*.*"), recursive=True):
        if path.endswith((".py", ".hip", ".hpp", ".c", ".h")):
            text = open(path).read()
            assert "import oracle" not in text and "from oracle" not in text, path
            assert "oracle_hist" not in text, path


def test_plain_c_client_compiles_links_and_gets_documented_errors(tmp_path):
    """The headers are C: a C99 program includes them, links the library and
    gets the documented statuses for bad arguments (no device needed)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    libdir = os.path.dirname(hist.LIBRARY)
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([gcc, "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-lpca_hist",
                    f"-Wl,-rpath,{libdir}", "-o", exe], check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    lines = out.stdout.split()
    assert out.returncode == 0 and lines[-1] == "ok", out.stdout + out.stderr
    # the ctypes mirrors of the public structs match the C layout
    layout = [int(v) for v in lines[lines.index("layout") + 1:lines.index("layout") + 9]]
    assert layout == [ctypes.sizeof(hist.PlanInfo), ctypes.sizeof(hist.PlanOpts),
                      hist.PlanInfo.max_group_elems.offset, hist.PlanInfo.event_cap.offset,
                      ctypes.sizeof(hist.DeviceDesc), ctypes.sizeof(hist.TuneEntry),
                      hist.TuneEntry.ms.offset, hist.TuneEntry.status.offset]
    layout2 = [int(v) for v in lines[lines.index("layout2") + 1:lines.index("layout2") + 5]]
    assert layout2 == [ctypes.sizeof(hist.ModelCalib), ctypes.sizeof(hist.Prediction),
                       hist.Prediction.predicted_us.offset, hist.Prediction.status.offset]
