"""Python binding of libpca_hist.so (the C ABI in include/hist.h).

Argument marshalling only: every step of the histogram runs in the library's
HIP kernels. PyTorch provides device memory (input, output, workspace) and
the stream (``torch.cuda.current_stream().cuda_stream``, a hipStream_t on
ROCm builds). There is no fallback: if the library is missing or the device
is not gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libpca_hist.so")

HIST_OK, HIST_ERR_INVALID_ARG, HIST_ERR_UNSUPPORTED, HIST_ERR_WORKSPACE, HIST_ERR_HIP = range(5)
PATHS = {"auto": 0, "full": 1, "range": 2, "scatter": 3, "stream": 4}
PATH_NAMES = {v: k for k, v in PATHS.items()}
MAX_PHASES = 7
WINDOW_BINS = 8192  # HIST_WINDOW_BINS
STREAM_TRACE_WORDS = 16
STREAM_TRACE_FIELDS = ("ticket", "start", "produced", "end", "tiles", "blocks", "stints",
                       "flag_wait", "moves_denied", "stint_write", "count", "scans")
MAX_BINS = 1 << 26


class HistError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


class LibraryMissing(ImportError):
    pass


class PlanOpts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("groups", ctypes.c_int32),
                ("range_bins", ctypes.c_int32), ("aggregation", ctypes.c_int32),
                ("wg_size", ctypes.c_int32), ("xcd_map", ctypes.c_int32),
                ("counter_bits", ctypes.c_int32), ("lds_copies", ctypes.c_int32),
                ("pacing", ctypes.c_int32), ("spin_log2", ctypes.c_int32),
                ("window", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("device", ctypes.c_int32),
                ("cu_count", ctypes.c_int32), ("xcd_count", ctypes.c_int32),
                ("num_bins", ctypes.c_uint32), ("range_bins", ctypes.c_uint32),
                ("ranges", ctypes.c_uint32), ("groups", ctypes.c_uint32),
                ("wg_size", ctypes.c_uint32), ("aggregation", ctypes.c_int32),
                ("tile_elems", ctypes.c_uint32), ("counter_bits", ctypes.c_uint32),
                ("max_n", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64),
                ("max_group_elems", ctypes.c_uint64), ("event_cap", ctypes.c_uint32)]


class DeviceDesc(ctypes.Structure):
    _fields_ = [("cu_count", ctypes.c_int32), ("xcd_count", ctypes.c_int32),
                ("lds_bytes", ctypes.c_uint32), ("sweep_waves_per_simd", ctypes.c_uint32)]


class TuneEntry(ctypes.Structure):
    _fields_ = [("opts", PlanOpts), ("ms", ctypes.c_double), ("status", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


TUNE_MAX_ENTRIES = 10


class ModelCalib(ctypes.Structure):
    _fields_ = [("read_gbps", ctypes.c_double), ("copy_gbps", ctypes.c_double),
                ("clock_ghz", ctypes.c_double), ("lds_cycles", ctypes.c_double),
                ("lds_dup_cycles", ctypes.c_double), ("launch_us", ctypes.c_double),
                ("sweep_fixed_us", ctypes.c_double), ("event_cycles", ctypes.c_double),
                ("scatter_fixed_us", ctypes.c_double)]


class Prediction(ctypes.Structure):
    _fields_ = [("opts", PlanOpts), ("predicted_us", ctypes.c_double), ("pass_us", ctypes.c_double),
                ("lds_us", ctypes.c_double), ("events_us", ctypes.c_double),
                ("fixed_us", ctypes.c_double), ("status", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


MODEL_MAX_ENTRIES = 8
SELECT_WORKSPACE_BYTES = 64 * 1024 * 4 + 16384


def mi355x() -> DeviceDesc:
    """MI355X (gfx950) as this library's kernels see it: 256 CUs in 8 XCDs,
    160 KiB of LDS per workgroup, 6 sweep waves per SIMD by registers."""
    return DeviceDesc(256, 8, 163840, 6)


_lib = None


def load(path: str = LIBRARY):
    """Load the library and declare its signatures. Raises LibraryMissing."""
    if not os.path.exists(path):
        raise LibraryMissing(
            f"{path} is not built; run `python -m partitioned_chip_accumulation_amd.build`")
    lib = ctypes.CDLL(path)
    vp, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
    P = ctypes.POINTER
    sigs = {
        "hist_status_str": (ctypes.c_char_p, [i32]),
        "hist_workspace_size": (i32, [u32, u64, P(PlanOpts), P(u64)]),
        "hist_plan": (i32, [P(vp), u32, u64, P(PlanOpts), vp, u64]),
        "hist_plan_create": (i32, [P(vp), u32, u64, P(PlanOpts), vp, u64]),
        "hist_run": (i32, [vp, vp, vp, u64, u32, vp]),
        "hist_run_accumulate": (i32, [vp, vp, vp, u64, u32, vp]),
        "hist_run_static": (i32, [vp, vp, u64, u32, vp]),
        "hist_plan_info": (i32, [vp, P(PlanInfo)]),
        "hist_plan_preview": (i32, [P(DeviceDesc), u32, u64, P(PlanOpts), P(PlanInfo)]),
        "hist_plan_describe": (i32, [vp, ctypes.c_char_p, u64]),
        "hist_tune_workspace_size": (i32, [u32, u64, P(u64)]),
        "hist_tune": (i32, [u32, u64, vp, u64, vp, vp, u64, u32, vp, P(PlanOpts), P(TuneEntry),
                            u32, P(u32)]),
        "hist_model_calibration": (i32, [P(ModelCalib)]),
        "hist_predict": (i32, [P(DeviceDesc), P(ModelCalib), u32, u64, vp, u32, P(PlanOpts),
                               P(Prediction), u32, P(u32)]),
        "hist_select": (i32, [u32, vp, u64, P(ModelCalib), vp, u64, vp, P(PlanOpts),
                              P(Prediction), u32, P(u32)]),
        "hist_plan_timing_enable": (i32, [vp, u32]),
        "hist_plan_timing_read": (i32, [vp, P(ctypes.c_double), P(u32)]),
        "hist_plan_phase_name": (ctypes.c_char_p, [vp, u32]),
        "hist_plan_check": (i32, [vp, vp, P(u32)]),
        "hist_plan_stream_trace": (i32, [vp, vp, P(u32), u32, P(u32)]),
        "hist_plan_destroy": (None, [vp]),
        "hist_bench_global_atomic": (i32, [vp, vp, u64, u32, vp]),
        "hist_bench_read": (i32, [vp, u64, vp, vp]),
        "hist_bench_copy": (i32, [vp, vp, u64, vp]),
        "hist_bench_lds_atomic": (i32, [u32, u32, u32, vp, u32, vp]),
        "hist_bench_lds_latency": (i32, [u32, u32, vp, vp]),
        "hist_bench_handoff": (i32, [u32, u32, u32, vp, vp, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def library():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def status_str(status: int) -> str:
    try:
        return library().hist_status_str(status).decode()
    except LibraryMissing:
        return "library missing"


def _check(status: int, what: str):
    if status != HIST_OK:
        raise HistError(status, what)


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _opts(path="auto", groups=0, range_bins=0, aggregation=-1, wg_size=0, xcd_map=0,
          counter_bits=0, lds_copies=0, pacing=0, spin_log2=0, window=0) -> PlanOpts:
    o = PlanOpts()
    o.path = PATHS[path] if isinstance(path, str) else int(path)
    o.groups, o.range_bins, o.aggregation = int(groups), int(range_bins), int(aggregation)
    o.wg_size, o.xcd_map, o.counter_bits = int(wg_size), int(xcd_map), int(counter_bits)
    o.lds_copies, o.pacing, o.spin_log2 = int(lds_copies), int(pacing), int(spin_log2)
    o.window = int(window)
    return o


def workspace_size(num_bins: int, max_n: int, **opts) -> int:
    o = _opts(**opts)
    n = ctypes.c_uint64(0)
    _check(library().hist_workspace_size(num_bins, max_n, ctypes.byref(o), ctypes.byref(n)),
           "hist_workspace_size")
    return int(n.value)


@dataclass
class Info:
    path: str
    device: int
    cu_count: int
    xcd_count: int
    num_bins: int
    range_bins: int
    ranges: int
    groups: int
    wg_size: int
    aggregation: int
    tile_elems: int
    counter_bits: int
    max_n: int
    workspace_bytes: int
    max_group_elems: int
    event_cap: int


def _info(i: PlanInfo) -> "Info":
    return Info(PATH_NAMES[i.path], i.device, i.cu_count, i.xcd_count, i.num_bins,
                i.range_bins, i.ranges, i.groups, i.wg_size, i.aggregation, i.tile_elems,
                i.counter_bits, i.max_n, i.workspace_bytes, i.max_group_elems, i.event_cap)


def preview(num_bins: int, max_n: int, device: DeviceDesc | None = None, **opts) -> "Info":
    """The plan the library would make on the described device (default: an
    MI355X), computed on the host; needs no GPU."""
    i = PlanInfo()
    _check(library().hist_plan_preview(ctypes.byref(device or mi355x()), int(num_bins),
                                       int(max_n), ctypes.byref(_opts(**opts)), ctypes.byref(i)),
           "hist_plan_preview")
    return _info(i)


class Plan:
    """A histogram plan for ``num_bins`` bins and inputs of up to ``max_n``
    elements on one device; owns its device workspace (a torch tensor)."""

    def __init__(self, num_bins: int, max_n: int, device=None, **opts):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.num_bins, self.max_n = int(num_bins), int(max_n)
        self._plan = ctypes.c_void_p()
        # streams other than the allocation stream that this plan's kernels ran
        # on: the workspace is recorded on each, so the caching allocator does
        # not hand it out again before their work is done
        self._side_streams: set[int] = set()
        lib = library()
        self._run = lib.hist_run
        self._run_acc = lib.hist_run_accumulate
        o = _opts(**opts)
        with torch.cuda.device(self.device):
            n = ctypes.c_uint64(0)
            _check(lib.hist_workspace_size(self.num_bins, self.max_n, ctypes.byref(o),
                                           ctypes.byref(n)), "hist_workspace_size")
            self.workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8,
                                         device=self.device)
            _check(lib.hist_plan(ctypes.byref(self._plan), self.num_bins, self.max_n,
                                 ctypes.byref(o), self.workspace.data_ptr() if n.value else None,
                                 int(n.value)), "hist_plan")

    def run(self, input: torch.Tensor, out: torch.Tensor | None = None,
            accumulate: bool = False, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
        """Histogram of an int32 CUDA tensor into a uint32 tensor of num_bins.
        accumulate=True adds into ``out`` (required then) instead of
        overwriting it: out[b] += #{i : input[i] == b}, modulo 2^32. The
        kernels go to ``stream`` (default: the current stream of the plan's
        device)."""
        if input.dtype != torch.int32 or input.device != self.device:
            raise ValueError("input must be an int32 tensor on the plan's device")
        if not input.is_contiguous():
            raise ValueError("input must be contiguous")
        fresh_out = out is None
        if out is None:
            if accumulate:
                raise ValueError("accumulate=True needs out")
            out = torch.empty(self.num_bins, dtype=torch.int32, device=self.device)
        if out.device != self.device or out.numel() != self.num_bins or \
                out.element_size() != 4 or not out.is_contiguous():
            raise ValueError("out must be a contiguous 4-byte tensor of num_bins on the device")
        n = input.numel()
        fn = self._run_acc if accumulate else self._run
        if stream is not None and stream.device != self.device:
            raise ValueError("stream must be on the plan's device")
        if torch.cuda.current_device() == self.device.index:
            h = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
            st = fn(self._plan, out.data_ptr(), input.data_ptr() if n else None, n,
                    self.num_bins, h)
        else:
            with torch.cuda.device(self.device):
                h = stream.cuda_stream if stream is not None else \
                    torch.cuda.current_stream().cuda_stream
                st = fn(self._plan, out.data_ptr(), input.data_ptr() if n else None, n,
                        self.num_bins, h)
        _check(st, "hist_run_accumulate" if accumulate else "hist_run")
        if stream is not None:
            # Memory from torch's caching allocator belongs to the stream that
            # was current when it was allocated; kernels queued on another
            # stream must be recorded on it, or a later allocation could reuse
            # the memory while they still run.
            h = stream.cuda_stream
            if h not in self._side_streams:
                self.workspace.record_stream(stream)
                self._side_streams.add(h)
            if fresh_out:
                out.record_stream(stream)
        return out.view(torch.uint32) if out.dtype == torch.int32 else out

    __call__ = run

    def info(self) -> Info:
        i = PlanInfo()
        _check(library().hist_plan_info(self._plan, ctypes.byref(i)), "hist_plan_info")
        return _info(i)

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        _check(library().hist_plan_describe(self._plan, buf, len(buf)), "hist_plan_describe")
        return buf.value.decode()

    def timing_enable(self, capacity: int):
        _check(library().hist_plan_timing_enable(self._plan, capacity), "hist_plan_timing_enable")

    def timing_read(self) -> dict[str, tuple[float, int]]:
        ms = (ctypes.c_double * MAX_PHASES)()
        cnt = (ctypes.c_uint32 * MAX_PHASES)()
        _check(library().hist_plan_timing_read(self._plan, ms, cnt), "hist_plan_timing_read")
        lib = library()
        return {lib.hist_plan_phase_name(self._plan, k).decode(): (ms[k], cnt[k])
                for k in range(MAX_PHASES) if cnt[k]}

    def check(self, stream: torch.cuda.Stream | None = None) -> bool:
        """True when a bounded wait of the plan's last runs gave up (STREAM
        plans; always False for the other paths). Waits for the stream."""
        v = ctypes.c_uint32(0)
        with torch.cuda.device(self.device):
            h = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
            _check(library().hist_plan_check(self._plan, h, ctypes.byref(v)), "hist_plan_check")
        return bool(v.value)

    def stream_trace(self, stream: torch.cuda.Stream | None = None):
        """The last run's per-workgroup timeline of a STREAM plan, a
        (workgroups, STREAM_TRACE_WORDS) uint32 array (None for other
        paths); the columns are STREAM_TRACE_FIELDS. Waits for the stream."""
        import numpy as np
        cap = self.info().cu_count * STREAM_TRACE_WORDS
        buf = (ctypes.c_uint32 * cap)()
        wg = ctypes.c_uint32(0)
        with torch.cuda.device(self.device):
            h = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
            _check(library().hist_plan_stream_trace(self._plan, h, buf, cap, ctypes.byref(wg)),
                   "hist_plan_stream_trace")
        if not wg.value:
            return None
        return np.frombuffer(buf, dtype=np.uint32)[:wg.value * STREAM_TRACE_WORDS].reshape(
            wg.value, STREAM_TRACE_WORDS).copy()

    def close(self):
        if self._plan:
            library().hist_plan_destroy(self._plan)
            self._plan = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _opts_dict(o: PlanOpts) -> dict:
    """The keyword options (as Plan takes them) that name a tuned schedule."""
    return {"path": PATH_NAMES[o.path], "counter_bits": int(o.counter_bits),
            "aggregation": int(o.aggregation)}


def tune(input: torch.Tensor, num_bins: int, max_n: int | None = None, reps: int = 3,
         workspace: torch.Tensor | None = None) -> tuple[dict, list[dict]]:
    """Time every candidate schedule on ``input`` (hist_tune) and return the
    fastest one's options, ready for ``Plan(num_bins, max_n, **opts)``, and
    every candidate as {"opts", "ms", "status"} (ms is -1 and status names the
    reason when a candidate was not run). Blocks until the runs are done."""
    if input.dtype != torch.int32 or not input.is_cuda or not input.is_contiguous():
        raise ValueError("input must be a contiguous int32 CUDA tensor")
    n = input.numel()
    max_n = n if max_n is None else int(max_n)
    lib = library()
    with torch.cuda.device(input.device):
        if workspace is None:
            need = ctypes.c_uint64(0)
            _check(lib.hist_tune_workspace_size(int(num_bins), max_n, ctypes.byref(need)),
                   "hist_tune_workspace_size")
            workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8,
                                    device=input.device)
        counts = torch.empty(int(num_bins), dtype=torch.int32, device=input.device)
        best = PlanOpts()
        entries = (TuneEntry * TUNE_MAX_ENTRIES)()
        count = ctypes.c_uint32(0)
        _check(lib.hist_tune(int(num_bins), max_n, input.data_ptr() if n else None, n,
                             counts.data_ptr(), workspace.data_ptr(), workspace.numel(), int(reps),
                             torch.cuda.current_stream().cuda_stream, ctypes.byref(best),
                             entries, TUNE_MAX_ENTRIES, ctypes.byref(count)), "hist_tune")
    rows = [{"opts": _opts_dict(e.opts), "ms": float(e.ms), "status": int(e.status)}
            for e in entries[:count.value]]
    return _opts_dict(best), rows


def _schedule_name(o: PlanOpts) -> str:
    name = PATH_NAMES[o.path]
    if o.path != PATHS["scatter"]:
        return f"{name}{o.counter_bits}"
    return name + ("+hot" if o.aggregation == 1 else "")


def _predictions(best: PlanOpts, entries, count: int) -> tuple[dict, list[dict]]:
    rows = [{"schedule": _schedule_name(e.opts), "opts": _opts_dict(e.opts),
             "predicted_us": float(e.predicted_us), "pass_us": float(e.pass_us),
             "lds_us": float(e.lds_us), "events_us": float(e.events_us),
             "fixed_us": float(e.fixed_us), "status": int(e.status)}
            for e in entries[:count]]
    return _opts_dict(best), rows


def model_calibration() -> ModelCalib:
    c = ModelCalib()
    _check(library().hist_model_calibration(ctypes.byref(c)), "hist_model_calibration")
    return c


def predict(num_bins: int, n: int, sample=None, device: DeviceDesc | None = None,
            calib: ModelCalib | None = None) -> tuple[dict, list[dict]]:
    """The cost model's prediction for every candidate schedule (host only).
    ``sample``: int32 array-like of input elements (or None). Returns the
    fastest predicted schedule's options and every candidate's terms."""
    import numpy as np
    smp = None if sample is None else np.ascontiguousarray(sample, dtype=np.int32)
    best = PlanOpts()
    entries = (Prediction * MODEL_MAX_ENTRIES)()
    count = ctypes.c_uint32(0)
    _check(library().hist_predict(ctypes.byref(device or mi355x()),
                                  ctypes.byref(calib) if calib is not None else None,
                                  int(num_bins), int(n),
                                  smp.ctypes.data if smp is not None and smp.size else None,
                                  0 if smp is None else int(smp.size), ctypes.byref(best), entries,
                                  MODEL_MAX_ENTRIES, ctypes.byref(count)), "hist_predict")
    return _predictions(best, entries, count.value)


def select(input: torch.Tensor, num_bins: int, calib: ModelCalib | None = None,
           workspace: torch.Tensor | None = None) -> tuple[dict, list[dict]]:
    """hist_select: sample the device input, time one stream read of it, and
    predict every schedule (no schedule is run). Blocks until done."""
    if input.dtype != torch.int32 or not input.is_cuda or not input.is_contiguous():
        raise ValueError("input must be a contiguous int32 CUDA tensor")
    with torch.cuda.device(input.device):
        if workspace is None:
            workspace = torch.empty(SELECT_WORKSPACE_BYTES, dtype=torch.uint8, device=input.device)
        best = PlanOpts()
        entries = (Prediction * MODEL_MAX_ENTRIES)()
        count = ctypes.c_uint32(0)
        _check(library().hist_select(int(num_bins), input.data_ptr(), input.numel(),
                                     ctypes.byref(calib) if calib is not None else None,
                                     workspace.data_ptr(), workspace.numel(),
                                     torch.cuda.current_stream().cuda_stream, ctypes.byref(best),
                                     entries, MODEL_MAX_ENTRIES, ctypes.byref(count)),
               "hist_select")
    return _predictions(best, entries, count.value)


_cache: dict = {}


def run(input: torch.Tensor, num_bins: int, out: torch.Tensor | None = None,
        accumulate: bool = False, **opts) -> torch.Tensor:
    """One-call histogram with a cached plan (max_n rounded up to a power of
    two). accumulate=True adds into ``out``. Calls with the same device, bin
    count, size class and options share one plan and its workspace, so they
    must not overlap on different streams (use a Plan per stream for that)."""
    n = max(1, input.numel())
    max_n = 1 << (n - 1).bit_length()
    max_n = min(max_n, 2**32 - 1)
    key = (input.device, int(num_bins), max_n, tuple(sorted(opts.items())))
    plan = _cache.get(key)
    if plan is None:
        plan = _cache[key] = Plan(num_bins, max_n, device=input.device, **opts)
    return plan.run(input, out=out, accumulate=accumulate)


STATIC_SCRATCH_BYTES = 128 << 20


def run_static(input: torch.Tensor, num_bins: int, out: torch.Tensor) -> torch.Tensor:
    """hist_run_static: the histogram with no device allocation (its
    workspace is a device array the library holds), on the current stream.
    ``out`` is required (a contiguous 4-byte tensor of num_bins on the input's
    device), since allocating it here would defeat the point. Calls that
    overlap on one device race on the shared array."""
    if input.dtype != torch.int32 or not input.is_cuda or not input.is_contiguous():
        raise ValueError("input must be a contiguous int32 CUDA tensor")
    if out.device != input.device or out.numel() != num_bins or out.element_size() != 4 or \
            not out.is_contiguous():
        raise ValueError("out must be a contiguous 4-byte tensor of num_bins on the device")
    n = input.numel()
    with torch.cuda.device(input.device):
        _check(library().hist_run_static(out.data_ptr(), input.data_ptr() if n else None, n,
                                         int(num_bins), _stream_handle(input.device)),
               "hist_run_static")
    return out.view(torch.uint32) if out.dtype == torch.int32 else out


# Measurement-only kernels (include/hist_bench.h).

def global_atomic(input: torch.Tensor, num_bins: int) -> torch.Tensor:
    out = torch.empty(num_bins, dtype=torch.int32, device=input.device)
    with torch.cuda.device(input.device):
        _check(library().hist_bench_global_atomic(out.data_ptr(), input.data_ptr(), input.numel(),
                                                  num_bins, _stream_handle(input.device)),
               "hist_bench_global_atomic")
    return out.view(torch.uint32)


def stream_read(src: torch.Tensor, sink: torch.Tensor):
    with torch.cuda.device(src.device):
        _check(library().hist_bench_read(src.data_ptr(), src.numel() * src.element_size(),
                                         sink.data_ptr(), _stream_handle(src.device)),
               "hist_bench_read")


def copy(dst: torch.Tensor, src: torch.Tensor):
    with torch.cuda.device(src.device):
        _check(library().hist_bench_copy(dst.data_ptr(), src.data_ptr(),
                                         src.numel() * src.element_size(),
                                         _stream_handle(src.device)), "hist_bench_copy")


LDS_PATTERNS = {"distinct": 0, "random": 1, "same": 2, "groups8": 3}


def lds_atomic(pattern: str, with_return: bool, iters: int, sink: torch.Tensor):
    """Queue the LDS-atomic calibration kernel (one 1024-thread workgroup per
    CU, 16 waves x iters x 16 atomics each) on the current stream."""
    with torch.cuda.device(sink.device):
        _check(library().hist_bench_lds_atomic(LDS_PATTERNS[pattern], int(with_return), int(iters),
                                               sink.data_ptr(), sink.numel(),
                                               _stream_handle(sink.device)),
               "hist_bench_lds_atomic")


LDS_LATENCY_PATTERNS = {"rtn-one-lane": 0, "rtn-64-words": 1, "rtn-one-word": 2, "read-64-words": 3}


def lds_latency(pattern: str, iters: int, device=None) -> dict:
    """Run the dependent-chain LDS probe (one wave) and return its cycles and
    nanoseconds per operation. Blocks until done."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    out = torch.zeros(4, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        _check(library().hist_bench_lds_latency(LDS_LATENCY_PATTERNS[pattern], int(iters),
                                                out.data_ptr(), _stream_handle(dev)),
               "hist_bench_lds_latency")
    o = out.cpu().tolist()
    return {"cycles_per_op": o[0] / iters, "ns_per_op": o[1] * 10.0 / iters,
            "clock_ghz": o[0] / (o[1] * 10.0) if o[1] else None}


def handoff(partner: int, mode: int, iters: int, device=None) -> dict:
    """Run the two-workgroup ping-pong probe and return the round trip in
    cycles and nanoseconds, the XCDs the two workgroups ran on, and whether
    a wait gave up or a payload word arrived wrong. Blocks until done."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    flags = torch.zeros(80, dtype=torch.int32, device=dev)
    out = torch.zeros(20, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        _check(library().hist_bench_handoff(int(partner), int(mode), int(iters), flags.data_ptr(),
                                            out.data_ptr(), _stream_handle(dev)),
               "hist_bench_handoff")
    o = out.cpu().tolist()
    return {"round_trip_cycles": o[0] / iters, "round_trip_ns": o[1] * 10.0 / iters,
            "timed_out": bool(o[2]), "payload_errors": int(o[3]),
            "xcd_wg0": int(o[4]), "xcd_partner": int(o[4 + partner]),
            "xcds": [int(v) for v in o[4:20]]}
