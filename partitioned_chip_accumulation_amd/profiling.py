"""Summaries of rocprofv3 output for the histogram kernels.

    python -m partitioned_chip_accumulation_amd.profiling trace DIR --cmd "..." --out FILE.md \
        [--sources A B ...] [--entry "KEY|KERNEL-SUBSTRING|WORKGROUPS" ...]
    python -m partitioned_chip_accumulation_amd.profiling counters DIR [DIR...] --cmd "..." --out FILE.md
    python -m partitioned_chip_accumulation_amd.profiling matrix FILE.jsonl --cmd "..." --out FILE.md
    python -m partitioned_chip_accumulation_amd.profiling sweep FILE.jsonl --cmd "..." --out FILE.md
    python -m partitioned_chip_accumulation_amd.profiling calib FILE.jsonl --cmd "..." --out FILE.md
    python -m partitioned_chip_accumulation_amd.profiling model --out FILE.md
    python -m partitioned_chip_accumulation_amd.profiling traffic --fetch DIR --write DIR \
        --kernel k_sweep --calib-kernel k_copy --calib-bytes N --key KEY --sources A B --out FILE.json

DIR is a rocprofv3 output directory written with ``--output-format csv``.
``trace`` tabulates kernel durations per (kernel, workgroups of the
dispatch), so that launches of one kernel on different shapes stay apart,
stamps the hash of the kernel sources into the summary, and with ``--entry``
records a dispatch group's durations under KEY in profiles/kernel_times.json
(for bench.py's cross-check of its live kernel timing).
``traffic`` scales the per-dispatch FETCH_SIZE and WRITE_SIZE of a kernel by
what the same counters read for a plain copy kernel of known size in the same
run (both counters are in KiB per dispatch; on gfx950 FETCH_SIZE reads half
of a copy's source bytes, so the scaling is needed), and records the hash of
the kernel sources so that a later change of the kernels invalidates it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics


def _csvs(d: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def short(name: str) -> str:
    base = name.split("(")[0].strip()
    return base.replace("void ", "")


def _workgroups(r: dict) -> int | None:
    """Workgroups of a dispatch from a kernel-trace row (grid sizes are in
    work-items), or None when the columns are absent."""
    try:
        n = 1
        for ax in "XYZ":
            g, w = int(r[f"Grid_Size_{ax}"]), int(r[f"Workgroup_Size_{ax}"])
            n *= (g + w - 1) // w
        return n
    except (KeyError, ValueError, ZeroDivisionError):
        return None


RUN_GAP_NS = 500_000_000  # dispatches of one group further apart start a new run


def kernel_durations(d: str) -> dict[tuple[str, int | None, int], list[float]]:
    """Durations in microseconds per (kernel, workgroups of the dispatch, run).
    A run is a stretch of a group's dispatches with no gap over half a second
    between them: one program that times several workloads in turn launches
    the same kernel on the same grid for each, seconds apart (their inputs
    are generated in between)."""
    raw = collections.defaultdict(list)
    for f in _csvs(d, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            raw[(short(r["Kernel_Name"]), _workgroups(r))].append((t0, (t1 - t0) / 1e3))
    by = {}
    for (k, wgs), v in raw.items():
        v.sort()
        run, last = 0, None
        for t0, us in v:
            if last is not None and t0 - last > RUN_GAP_NS:
                run += 1
            last = t0
            by.setdefault((k, wgs, run), []).append(us)
    return by


def trace_table(d: str) -> str:
    by = kernel_durations(d)
    lines = ["| kernel | workgroups | run | calls | avg us | median us | min us | total ms |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (k, wgs, run), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {wgs if wgs is not None else '?'} | {run} | {len(v)} | "
                     f"{statistics.mean(v):.2f} | {statistics.median(v):.2f} | {min(v):.2f} | "
                     f"{sum(v) / 1e3:.3f} |")
    return "\n".join(lines)


def trace_entry(d: str, pattern: str, workgroups: int, run: int = 0) -> dict:
    """Duration statistics of run `run` of the dispatches of the kernel
    matching pattern with that many workgroups."""
    hits = {k: v for k, v in kernel_durations(d).items()
            if pattern in k[0] and k[1] == workgroups and k[2] == run}
    if len(hits) != 1:
        raise SystemExit(f"{len(hits)} dispatch groups match {pattern!r} x {workgroups} "
                         f"run {run}: {sorted(hits)}")
    (name, _, _), v = next(iter(hits.items()))
    return {"kernel": name, "workgroups": workgroups, "run": run, "calls": len(v),
            "avg_us": round(statistics.mean(v), 3), "median_us": round(statistics.median(v), 3),
            "min_us": round(min(v), 3)}


def counters_per_dispatch(d: str) -> dict[str, dict[str, float]]:
    """Median over dispatches of each counter (summed over its dimensions)."""
    acc = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for f in _csvs(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            acc[short(r["Kernel_Name"])][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: {c: statistics.median(v.values()) for c, v in cs.items()} for k, cs in acc.items()}


def counters_table(dirs: list[str]) -> str:
    merged = collections.defaultdict(dict)
    for d in dirs:
        for k, cs in counters_per_dispatch(d).items():
            merged[k].update(cs)
    lines = ["| kernel | counter | median per dispatch |", "|---|---|---:|"]
    for k in sorted(merged):
        for c in sorted(merged[k]):
            lines.append(f"| `{k}` | {c} | {merged[k][c]:.6g} |")
    return "\n".join(lines)


def _match(cs: dict, pat: str) -> dict:
    hits = {k: v for k, v in cs.items() if pat in k}
    if not hits:
        raise SystemExit(f"no kernel matching {pat!r} in {sorted(cs)}")
    return next(iter(hits.values()))


def _cells_table(rows: dict, cols: list[str], label) -> list[str]:
    out = ["| " + label + " | " + " | ".join(cols) + " |", "|---:|" + "---:|" * len(cols)]
    for key, cells in rows.items():
        ok = {c: v for c, v in cells.items() if v["parity"] and c != "auto"}
        best = min(ok, key=lambda c: ok[c]["us_per_run"]) if ok else None
        tds = []
        for c in cols:
            v = cells.get(c)
            if v is None:
                tds.append("")
                continue
            t = f"{v['us_per_run']:.1f}" + ("" if v["parity"] else " FAIL")
            tds.append(f"**{t}**" if c == best else t)
        out.append(f"| {key} | " + " | ".join(tds) + " |")
    return out


def _read_cells(jsonl: str, key: str):
    rows, cols, plans = collections.OrderedDict(), [], {}
    for line in open(jsonl):
        line = line.strip()
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        if "us_per_run" not in r:
            continue
        rows.setdefault(r[key], {})[r["cell"]] = r
        if r["cell"] not in cols:
            cols.append(r["cell"])
        if r["cell"] == "auto":
            plans[r[key]] = r["plan"]
    return rows, cols, plans


def calib_markdown(jsonl: str, cmd: str) -> str:
    """Tables from ``bench.py --calibrate``."""
    recs = [json.loads(l) for l in open(jsonl) if l.strip().startswith("{")]
    out = ["# Calibration: the ceilings the histogram kernels meet, one MI355X", "",
           "Command:", "", "```", cmd, "```", "", "## HBM", "",
           "| measurement | GB/s | fraction of 8 TB/s |", "|---|---:|---:|"]
    for r in recs:
        if r["what"] in ("hbm_stream_read", "hbm_copy"):
            out.append(f"| {r['what']} | {r['GBps']:.0f} | {r['GBps'] / 8000:.3f} |")
    out += ["", "## LDS atomics (one 1024-thread workgroup per CU, 16 waves)", "",
            "Time per wave instruction per CU; cycles at the 2.4 GHz peak clock.", "",
            "| address pattern of one wave instruction | form | ns | cycles |",
            "|---|---|---:|---:|"]
    names = {"distinct": "64 consecutive words", "random": "random words of 32,768",
             "same": "all 64 lanes on one word", "groups8": "8 groups of 8 lanes, one word each"}
    for r in recs:
        if r["what"] == "lds_atomic":
            form = "ds_add_rtn_u32" if r["with_return"] else "ds_add_u32"
            out.append(f"| {names[r['pattern']]} | {form} | {r['ns_per_wave_instr_per_cu']:.2f} | "
                       f"{r['cycles_at_2p4GHz']:.1f} |")
    lat = [r for r in recs if r["what"] == "lds_latency"]
    if lat:
        out += ["", "## LDS latency (one wave; each access's address waits for the previous "
                "access's return)", "",
                "| chain | cycles per access | ns per access | shader clock GHz |",
                "|---|---:|---:|---:|"]
        lnames = {"rtn-one-lane": "ds_add_rtn_u32, lane 0 alone",
                  "rtn-64-words": "ds_add_rtn_u32, 64 lanes on 64 consecutive words",
                  "rtn-one-word": "ds_add_rtn_u32, 64 lanes on one word",
                  "read-64-words": "ds_read_b32, 64 lanes on 64 consecutive words"}
        for r in lat:
            out.append(f"| {lnames.get(r['pattern'], r['pattern'])} | {r['cycles_per_op']:.1f} | "
                       f"{r['ns_per_op']:.2f} | {r['clock_ghz']} |")
    ho = [r for r in recs if r["what"] == "handoff"]
    if ho:
        out += ["", "## Handoff between two workgroups through global memory (round trip)", "",
                "| what passes | workgroups | XCDs (wg 0, partner) | cycles | ns | clean |",
                "|---|---|---|---:|---:|---|"]
        for r in ho:
            where = "one XCD" if r["same_xcd"] else "two XCDs"
            clean = "yes" if not r["timed_out"] and not r["payload_errors"] else \
                f"NO (timed out {r['timed_out']}, payload errors {r['payload_errors']})"
            out.append(f"| {r['mode']} | 0 and {r['partner']} ({where}) | "
                       f"{r['xcds'][0]}, {r['xcds'][r['partner']]} | {r['round_trip_cycles']:.0f} | "
                       f"{r['round_trip_ns']:.0f} | {clean} |")
    prim = [r for r in recs if r["what"] == "model_primitive"]
    if prim:
        out += ["", "## Primitives of the schedule cost model (hist_model_calibration)", "",
                "| primitive | value | how |", "|---|---:|---|"]
        for r in prim:
            out.append(f"| {r['name']} | {r['value']} | {r['how']} |")
    out += ["", "## Owners of a chunk sharing an XCD's L2 (RANGE path)", "",
            "| placement | bins | n | us per run | plan |", "|---|---:|---:|---:|---|"]
    for r in recs:
        if r["what"] == "range_owner_placement":
            out.append(f"| {r['placement']} | {r['bins']} | {r['n']} | {r['us_per_run']:.1f} | "
                       f"`{r['plan']}` |")
    return "\n".join(out) + "\n"


def sweep_markdown(jsonl: str, cmd: str) -> str:
    """Bin counts x schedules table from ``bench.py --path-sweep``."""
    rows, cols, plans = _read_cells(jsonl, "bins")
    first = next(iter(next(iter(rows.values())).values()))
    n, kind = first["n"], first.get("input", "uniform")
    kind = "uniform" if kind == "uniform" else f"finite Zipf ({kind}, ranks permuted to bins)"
    rows = collections.OrderedDict((f"2^{b.bit_length() - 1}", v) for b, v in rows.items())
    out = [f"# Path selection: every schedule on {kind} int32 input, n = {n:,}, one MI355X", "",
           "Microseconds per histogram: wall clock over back-to-back runs on four rotated input "
           "copies after 20 warm-up runs. Every cell was checked bit for bit against numpy's "
           "bincount (a failure would be marked FAIL). The fastest cell of a row is in bold. AUTO "
           "is the plan's own choice; it runs last in each row, and every row starts with 0.3 s "
           "of untimed runs so that no cell meets unsettled clocks.",
           "", "Command:", "", "```", cmd, "```", ""]
    out += _cells_table(rows, cols, "bins")
    out += ["", "AUTO's plans:", ""] + \
        [f"- 2^{b.bit_length() - 1}: `{p}`" for b, p in plans.items()]
    return "\n".join(out) + "\n"


def matrix_markdown(jsonl: str, cmd: str) -> str:
    """Workloads x schedules table (microseconds per histogram) from the JSON
    lines of ``bench.py --workload-matrix``."""
    rows, cols, plans = _read_cells(jsonl, "workload")
    out = ["# Every schedule on every workload, one MI355X", "",
           "Microseconds per histogram: wall clock over back-to-back runs on four rotated input "
           "copies after 10 warm-up runs. Every cell was checked bit for bit against numpy's "
           "bincount (a failure would be marked FAIL). The fastest cell of a row is in bold. "
           "\"+hot\" is the wave hot-slot aggregation. An empty cell is a schedule the bin "
           "count does not allow.", "", "Command:", "", "```", cmd, "```", ""]
    out += _cells_table(rows, cols, "workload")
    out += ["", "AUTO's plans:", ""] + [f"- {wl}: `{p}`" for wl, p in plans.items()]
    return "\n".join(out) + "\n"


def measured_rows(profiles_dir: str) -> dict:
    """The committed path-selection sweeps and workload matrix as
    {label: (input kind, bins, n, {schedule: us})} (AUTO's column left out)."""
    import re

    from partitioned_chip_accumulation_amd import inputs
    rows = {}

    def read(name, kind_of):
        hdr = None
        for line in open(os.path.join(profiles_dir, name)):
            line = line.rstrip("\n")
            if line.startswith("| bins") or line.startswith("| workload"):
                hdr = [c.strip() for c in line.strip("|").split("|")]
                continue
            if hdr and line.startswith("| ") and not line.startswith("|---"):
                cells = [c.strip().replace("**", "") for c in line.strip("|").split("|")]
                kind, B, n = kind_of(cells[0])
                rows[f"{name}: {cells[0]}"] = (kind, B, n, {
                    h: float(c) for h, c in zip(hdr[1:], cells[1:])
                    if c and "FAIL" not in c and h != "auto"})
            elif line.startswith("AUTO"):
                hdr = None

    pow2 = lambda l: 1 << int(re.match(r"2\^(\d+)", l).group(1))
    read("path_selection_uniform_n2p26.md", lambda l: ("uniform", pow2(l), 1 << 26))
    read("path_selection_zipf1.1_n2p26.md", lambda l: ("zipf", pow2(l), 1 << 26))
    cfg = {w.name: c for c, w in inputs.WORKLOADS.items()}
    read("path_matrix_workloads.md",
         lambda l: (str(cfg[l]), inputs.WORKLOADS[cfg[l]].num_bins, inputs.WORKLOADS[cfg[l]].n))
    return rows


def model_markdown(profiles_dir: str) -> str:
    """The cost model's predictions (hist_predict, samples of 2^16 elements
    from the same generator and seeds) beside the committed measurements."""
    from partitioned_chip_accumulation_amd import hist, inputs

    def sample(kind, B):
        if kind == "uniform":
            return inputs.uniform(1, 1 << 16, B)
        if kind == "zipf":
            return inputs.zipf(2, 1 << 16, B, 1.1)
        return inputs.generate(int(kind), n=1 << 16)

    c = hist.model_calibration()
    out = ["# The schedule cost model against the measured schedules, one MI355X", "",
           "`hist_predict` with the library's MI355X primitives (HBM read "
           f"{c.read_gbps:.0f} GB/s, copy {c.copy_gbps:.0f} GB/s, LDS atomics {c.lds_cycles} cycles "
           f"a wave instruction + {c.lds_dup_cycles:.3f} per same-word lane, launch "
           f"{c.launch_us} us, sweep fixed {c.sweep_fixed_us} us, carry event {c.event_cycles} "
           f"cycles, two-phase fixed {c.scatter_fixed_us} us; `bench.py --calibrate`) on a "
           "sample of 2^16 elements of each row's input, drawn by the same generator and seed. "
           "The measured times are the committed path-selection sweeps and workload matrix; no "
           "schedule was timed to make a prediction, and nothing was fitted to these tables. A "
           "row is a hit when the schedule predicted fastest (among those the row measured) "
           "took at most 5% longer than the fastest measured one.", "",
           "Command:", "", "```",
           "python -m partitioned_chip_accumulation_amd.profiling model --out "
           "profiles/model_selection.md", "```", "",
           "| row | predicted fastest | its predicted us | its measured us | fastest measured | "
           "us | hit |", "|---|---|---:|---:|---|---:|---|"]
    hits = 0
    rows = measured_rows(profiles_dir)
    for label, (kind, B, n, meas) in rows.items():
        _, preds = hist.predict(B, n, sample(kind, B))
        pred = {p["schedule"]: p["predicted_us"] for p in preds
                if p["status"] == 0 and p["schedule"] in meas}
        pick = min(pred, key=pred.get)
        best = min(meas, key=meas.get)
        hit = meas[pick] <= 1.05 * meas[best]
        hits += hit
        out.append(f"| {label.replace('.md', '')} | {pick} | {pred[pick]:.1f} | {meas[pick]:.1f} | "
                   f"{best} | {meas[best]:.1f} | {'yes' if hit else 'NO'} |")
    out += ["", f"Hits: {hits} of {len(rows)} rows ({100.0 * hits / len(rows):.0f}%)."]
    return "\n".join(out) + "\n"


def sources_sha(paths: list[str]) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--title", default="Kernel trace")
    t.add_argument("--sources", nargs="*", default=[],
                   help="kernel source files whose SHA-256 the summary records")
    t.add_argument("--entry", action="append", default=[],
                   help="KEY|KERNEL-SUBSTRING|WORKGROUPS[|RUN]: record that dispatch group's "
                        "durations (its RUN-th run, default 0) under KEY in --times")
    t.add_argument("--times", default=os.path.join("profiles", "kernel_times.json"))
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--cmd", required=True, action="append")
    c.add_argument("--out", required=True)
    c.add_argument("--title", default="Hardware counters")
    ca = sub.add_parser("calib")
    ca.add_argument("jsonl")
    ca.add_argument("--cmd", required=True)
    ca.add_argument("--out", required=True)
    sw = sub.add_parser("sweep")
    sw.add_argument("jsonl")
    sw.add_argument("--cmd", required=True)
    sw.add_argument("--out", required=True)
    mx = sub.add_parser("matrix")
    mx.add_argument("jsonl")
    mx.add_argument("--cmd", required=True)
    mx.add_argument("--out", required=True)
    mo = sub.add_parser("model")
    mo.add_argument("--out", required=True)
    mo.add_argument("--profiles", default="profiles")
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", required=True)
    tr.add_argument("--write", required=True)
    tr.add_argument("--kernel", required=True)
    tr.add_argument("--calib-kernel", required=True)
    tr.add_argument("--calib-bytes", type=int, required=True)
    tr.add_argument("--key", required=True)
    tr.add_argument("--sources", nargs="+", required=True)
    tr.add_argument("--out", required=True)
    tr.add_argument("--lds", default=None,
                    help="optional pass with SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE")
    tr.add_argument("--occ", default=None, help="optional pass with MeanOccupancyPerActiveCU")
    a = ap.parse_args()

    if a.cmd_ == "calib":
        open(a.out, "w").write(calib_markdown(a.jsonl, a.cmd))
        return
    if a.cmd_ == "sweep":
        open(a.out, "w").write(sweep_markdown(a.jsonl, a.cmd))
        return
    if a.cmd_ == "matrix":
        open(a.out, "w").write(matrix_markdown(a.jsonl, a.cmd))
        return
    if a.cmd_ == "model":
        open(a.out, "w").write(model_markdown(a.profiles))
        return
    if a.cmd_ == "trace":
        sha = sources_sha(a.sources) if a.sources else None
        stamp = "" if not sha else \
            f"Kernel sources (SHA-256 of {' '.join(a.sources)}): `{sha}`\n\n"
        text = f"# {a.title}\n\nCommand (rocprofv3 kernel trace):\n\n```\n{a.cmd}\n```\n\n" \
               f"{stamp}{trace_table(a.dir)}\n"
        open(a.out, "w").write(text)
        if a.entry:
            if not sha:
                raise SystemExit("--entry needs --sources")
            data = json.load(open(a.times)) if os.path.exists(a.times) else {}
            for spec in a.entry:
                key, pat, wgs, *run = spec.split("|")
                e = trace_entry(a.dir, pat, int(wgs), int(run[0]) if run else 0)
                e.update({"profile": a.out, "cmd": a.cmd, "kernel_source_sha": sha,
                          "sources": a.sources})
                data[key] = e
                print(json.dumps({key: e}))
            with open(a.times, "w") as f:
                json.dump(data, f, indent=1, sort_keys=True)
                f.write("\n")
    elif a.cmd_ == "counters":
        cmds = "\n".join(a.cmd)
        text = f"# {a.title}\n\nCommands (one rocprofv3 --pmc pass each):\n\n```\n{cmds}\n```\n\n" \
               f"{counters_table(a.dirs)}\n"
        open(a.out, "w").write(text)
    else:
        fetch = counters_per_dispatch(a.fetch)
        write = counters_per_dispatch(a.write)
        f_k = _match(fetch, a.kernel)["FETCH_SIZE"]
        w_k = _match(write, a.kernel)["WRITE_SIZE"]
        f_c = _match(fetch, a.calib_kernel)["FETCH_SIZE"]
        w_c = _match(write, a.calib_kernel)["WRITE_SIZE"]
        f_scale = a.calib_bytes / (f_c * 1024.0)
        w_scale = a.calib_bytes / (w_c * 1024.0)
        entry = {"fetch_bytes": round(f_k * 1024 * f_scale), "write_bytes": round(w_k * 1024 * w_scale),
                 "fetch_kib_raw": f_k, "write_kib_raw": w_k, "fetch_scale": f_scale,
                 "write_scale": w_scale, "calib_kernel": a.calib_kernel,
                 "calib_bytes": a.calib_bytes, "kernel_source_sha": sources_sha(a.sources),
                 "sources": a.sources}
        entry["bytes_per_launch"] = entry["fetch_bytes"] + entry["write_bytes"]
        lds = {}
        if a.lds:
            c = _match(counters_per_dispatch(a.lds), a.kernel)
            if c.get("SQ_LDS_IDX_ACTIVE"):
                # cycles the LDS stalled on bank conflicts, per cycle it was active
                lds["lds_bank_conflict_per_active_cycle"] = round(
                    c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"], 4)
            for name in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAVES"):
                if name in c:
                    lds[name] = c[name]
        if a.occ:
            c = _match(counters_per_dispatch(a.occ), a.kernel)
            if "MeanOccupancyPerActiveCU" in c:
                lds["MeanOccupancyPerActiveCU"] = round(c["MeanOccupancyPerActiveCU"], 4)
        if lds:
            entry["lds_counters"] = lds
        data = {}
        if os.path.exists(a.out):
            data = json.load(open(a.out))
        data[a.key] = entry
        with open(a.out, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(entry))


if __name__ == "__main__":
    main()
