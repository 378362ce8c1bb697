"""Host-side checks of the rocprofv3/bench summarisers (no GPU): the tables in
profiles/ are generated from JSON lines and CSV files by these functions."""
from __future__ import annotations

import json
import os

from partitioned_chip_accumulation_amd import profiling


def write_lines(path, recs):
    with open(path, "w") as f:
        f.write("# a comment line the renderers skip\n")
        for r in recs:
            f.write(json.dumps(r) + "\n")


def cell(key, keyval, name, us, ok=True, plan="p"):
    return {key: keyval, "n": 1024, "cell": name, "us_per_run": us, "parity": ok, "plan": plan}


def test_matrix_bolds_the_fastest_exact_cell_and_marks_failures(tmp_path):
    f = tmp_path / "m.jsonl"
    write_lines(f, [cell("workload", "w1", "auto", 10.0, plan="auto-plan"),
                    cell("workload", "w1", "a", 9.0),
                    cell("workload", "w1", "b", 8.0, ok=False),
                    cell("workload", "w2", "auto", 5.0),
                    cell("workload", "w2", "b", 6.0),
                    {"workload": "w2", "cell": "c", "error": "unsupported"}])
    md = profiling.matrix_markdown(str(f), "cmd")
    rows = {l.split("|")[1].strip(): l for l in md.splitlines() if l.startswith("| w")}
    assert "**9.0**" in rows["w1"] and "8.0 FAIL" in rows["w1"] and "**8.0" not in rows["w1"]
    assert "**6.0**" in rows["w2"]  # auto is never the bold cell
    assert "`auto-plan`" in md and "cmd" in md


def test_sweep_rows_are_powers_of_two(tmp_path):
    f = tmp_path / "s.jsonl"
    write_lines(f, [cell("bins", 1024, "auto", 3.0), cell("bins", 1024, "full", 2.0),
                    cell("bins", 4096, "auto", 4.0), cell("bins", 4096, "scatter", 5.0)])
    md = profiling.sweep_markdown(str(f), "cmd")
    assert "| 2^10 |" in md and "| 2^12 |" in md and "**2.0**" in md and "**5.0**" in md
    assert "n = 1,024" in md


def test_calibration_tables(tmp_path):
    f = tmp_path / "c.jsonl"
    write_lines(f, [{"what": "hbm_stream_read", "GBps": 6000.0, "bytes": 1},
                    {"what": "lds_atomic", "pattern": "groups8", "with_return": True,
                     "ns_per_wave_instr_per_cu": 12.5, "cycles_at_2p4GHz": 30.0},
                    {"what": "range_owner_placement", "placement": "plain order", "bins": 8,
                     "n": 16, "us_per_run": 1.5, "plan": "p"}])
    md = profiling.calib_markdown(str(f), "cmd")
    assert "| hbm_stream_read | 6000 | 0.750 |" in md
    assert "| 8 groups of 8 lanes, one word each | ds_add_rtn_u32 | 12.50 | 30.0 |" in md
    assert "| plain order | 8 | 16 | 1.5 | `p` |" in md


def test_counters_take_the_median_over_dispatches(tmp_path):
    d = tmp_path / "pmc" / "host"
    os.makedirs(d)
    with open(d / "x_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        # two dimensions of one dispatch are summed; the median is over dispatches
        for disp, vals in [(1, (1, 2)), (2, (5, 5)), (3, (100, 0))]:
            for v in vals:
                f.write(f'{disp},"void pca::k_sweep<1024>(int)",FETCH_SIZE,{v}\n')
    cs = profiling.counters_per_dispatch(str(tmp_path / "pmc"))
    assert cs == {"pca::k_sweep<1024>": {"FETCH_SIZE": 10.0}}


def test_trace_table(tmp_path):
    d = tmp_path / "tr"
    os.makedirs(d)
    with open(d / "t_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        f.write('"void pca::k_merge<4>(x)",1000,3000\n')
        f.write('"void pca::k_merge<4>(x)",5000,9000\n')
    table = profiling.trace_table(str(d))
    assert "| `pca::k_merge<4>` | ? | 0 | 2 | 3.00 | 3.00 | 2.00 | 0.006 |" in table  # no shapes


def test_sweep_title_names_the_input(tmp_path):
    f = tmp_path / "z.jsonl"
    recs = [dict(cell("bins", 1 << 14, "full16", 2.0), input="zipf s=1.1"),
            dict(cell("bins", 1 << 14, "auto", 2.1), input="zipf s=1.1")]
    write_lines(f, recs)
    md = profiling.sweep_markdown(str(f), "cmd")
    assert "finite Zipf (zipf s=1.1" in md.splitlines()[0]
    g = tmp_path / "u.jsonl"
    write_lines(g, [cell("bins", 1 << 14, "full16", 2.0)])  # records without the field
    assert "uniform int32 input" in profiling.sweep_markdown(str(g), "cmd").splitlines()[0]


def test_trace_groups_dispatches_by_shape_and_records_entries(tmp_path):
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
            "Grid_Size_Z", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"]
    rows = [("void pca::k_sweep<1024, 2, 0, 16>(args)", 0, 44000, 262144),
            ("void pca::k_sweep<1024, 2, 0, 16>(args)", 100000, 146000, 262144),
            ("void pca::k_sweep<1024, 2, 0, 16>(args)", 0, 5000, 131072),
            ("void pca::k_merge<4, false>(args)", 0, 5000, 65536),
            # the same kernel and grid seconds later: a second run
            ("void pca::k_sweep<1024, 2, 0, 16>(args)", 9 * 10**9, 9 * 10**9 + 90000, 262144)]
    with open(d / "run_kernel_trace.csv", "w") as f:
        f.write(",".join(cols) + "\n")
        for name, t0, t1, grid in rows:
            wg = 1024 if "sweep" in name else 256
            f.write(f'"{name}",{t0},{t1},{grid},1,1,{wg},1,1\n')
    table = profiling.trace_table(str(tmp_path / "trace"))
    assert "| `pca::k_sweep<1024, 2, 0, 16>` | 256 | 0 | 2 | 45.00 |" in table
    assert "| `pca::k_sweep<1024, 2, 0, 16>` | 256 | 1 | 1 | 90.00 |" in table
    assert "| `pca::k_sweep<1024, 2, 0, 16>` | 128 | 0 | 1 | 5.00 |" in table
    e = profiling.trace_entry(str(tmp_path / "trace"), "k_sweep", 256)
    assert e["calls"] == 2 and e["avg_us"] == 45.0 and e["kernel"] == "pca::k_sweep<1024, 2, 0, 16>"
    assert profiling.trace_entry(str(tmp_path / "trace"), "k_sweep", 256, 1)["avg_us"] == 90.0
