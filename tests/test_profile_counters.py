"""Host logic of the counter and trace summaries (CPU only): comment-insensitive source
digests, the copy calibration of FETCH_SIZE / WRITE_SIZE, the matrix-core counter file,
the stale-digest rule, and the kernel-trace summary with its per-workload split. The
inputs are small synthetic rocprofv3-shaped CSV files and a SQLite table."""
import csv
import io
import os
import sqlite3
from contextlib import redirect_stdout

import pytest

from learned_context_ranking_amd import profile_counters as pc

HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
DKV = "void sas::dkv_kernel<128, false>(sas::AttnArgs)"
DQ = "void sas::dq_kernel<128, false>(sas::AttnArgs, int)"
FWD = "void sas::fwd_kernel<128, 1, 4, false>(sas::AttnArgs, int, int)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::copy_>(...)"


def _csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(HEADER)
        for i, (name, counter, value, start, end) in enumerate(rows):
            w.writerow([i, i, "Agent 1", 1, 1, 1, 256, 7, name, 256, 0, 0, 128, 0, 16, counter, value, start, end])


def _read_kv(path, section=None):
    kv, sec = {}, None
    for line in open(path):
        line = line.strip()
        if line.startswith("[") and "]" in line:
            sec = line[1:line.index("]")]
        elif "=" in line and not line.startswith("#") and (section is None or sec == section):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_code_lines_drop_comments_but_not_strings():
    src = 'int a = 1;  // note\n\n   // whole line\nconst char* s = "a // b";  // tail\n'
    assert pc._code_lines(src) == ["int a = 1;", 'const char* s = "a // b";']


def test_traffic_scaled_by_the_copy(tmp_path):
    kib = pc.CALIB_BYTES / 1024
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1)
    _csv(tmp_path / "f", [(COPY, "FETCH_SIZE", kib / 2, 0, 1), (DKV, "FETCH_SIZE", 1000.0, 0, 1),
                          (DKV, "FETCH_SIZE", 3000.0, 0, 1)])
    _csv(tmp_path / "w", [(COPY, "WRITE_SIZE", kib, 0, 1), (DKV, "WRITE_SIZE", 10.0, 0, 1),
                          (DKV, "WRITE_SIZE", 30.0, 0, 1)])
    with redirect_stdout(io.StringIO()):
        pc.main(["x", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path), "cmd"])
    kv = _read_kv(tmp_path / "traffic_dkv.txt")
    assert float(kv["read_bytes_per_launch"]) == pytest.approx(2000.0 * 1024 * 2)
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(20.0 * 1024)
    assert kv["source_sha256"] == pc.source_digest("dkv")
    assert pc.profiled_traffic("dkv", str(tmp_path)) == int(2000 * 1024 * 2 + 20 * 1024)
    # a digest that no longer matches the sources voids the figure
    text = open(tmp_path / "traffic_dkv.txt").read().replace(kv["source_sha256"], "0" * 16)
    open(tmp_path / "traffic_dkv.txt", "w").write(text)
    assert pc.profiled_traffic("dkv", str(tmp_path)) is None


def test_traffic_needs_the_calibration_copy(tmp_path):
    _csv(tmp_path / "f", [(DKV, "FETCH_SIZE", 1000.0, 0, 1)])
    _csv(tmp_path / "w", [(DKV, "WRITE_SIZE", 10.0, 0, 1)])
    with pytest.raises(SystemExit):
        pc.main(["x", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path), "cmd"])


def test_mfma_counter_file(tmp_path):
    rows = []
    for name, flops, util, dur in ((FWD, 1.0e12, 40.0, 1_000_000), (DQ, 1.5e12, 45.0, 1_500_000),
                                   (DKV, 2.0e12, 30.0, 2_000_000)):
        for r in range(2):   # two dispatches each, the second 10 % slower
            d = int(dur * (1.1 if r else 1.0))
            rows.append((name, "MfmaFlopsBF16", flops, 100, 100 + d))
            rows.append((name, "MfmaUtil", util + r, 100, 100 + d))
    _csv(tmp_path / "m", rows)
    with redirect_stdout(io.StringIO()):
        pc.main(["x", "--mfma", str(tmp_path / "m"), str(tmp_path), "cmd"])
    path = tmp_path / "mfma_train_step.txt"
    dkv = _read_kv(path, "dkv")
    assert float(dkv["mfma_bf16_flops_per_launch"]) == pytest.approx(2.0e12)
    assert float(dkv["duration_us_mean"]) == pytest.approx(2100.0)
    assert float(dkv["executed_tflops_at_mean"]) == pytest.approx(2.0e12 / 2.1e-3 / 1e12, rel=1e-3)
    assert float(dkv["mfma_util_pct"]) == pytest.approx(30.5)
    assert float(dkv["attended_pairs_x_d_implied"]) == pytest.approx(2.0e12 / 8)
    assert float(_read_kv(path, "dq")["attended_pairs_x_d_implied"]) == pytest.approx(1.5e12 / 6)
    got = pc.profiled_mfma("dkv", str(tmp_path))
    assert got == {"executed_flop_per_launch": 2.0e12, "mfma_util_pct": 30.5}
    assert pc.profiled_mfma("decode", str(tmp_path)) is None


def test_trace_summary_and_workload_split(tmp_path):
    db = tmp_path / "run_results.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, duration integer, grid_x integer)")
    rand = "void at::native::(anonymous namespace)::distribution_elementwise_grid_stride_kernel<...>"
    seq = [(rand, 10), ("void sas::fwd_kernel<128, 1, 4, false>(sas::AttnArgs, int, int)", 1000),   # main step
           (rand, 10), (rand, 10), ("void sas::fwd_kernel<128, 1, 4, false>(sas::AttnArgs, int, int)", 2000),
           (rand, 10), ("void sas::fwd_kernel<128, 1, 4, false>(sas::AttnArgs, int, int)", 3000),
           ("void sas::dkv_kernel<128, false>(sas::AttnArgs)", 4000)]
    t = 0
    for name, dur in seq:
        con.execute("insert into kernels values (?, ?, ?, ?)", (name, t, dur, 4096 if dur > 1500 else 1024))
        t += dur + 5
    con.commit()
    con.close()
    buf = io.StringIO()
    with redirect_stdout(buf):
        pc.main(["x", "--trace", str(db), "title", "cmd", "--by-workload", "first", "second"])
    out = buf.getvalue()
    assert out.startswith("# title")
    assert "| `void sas::fwd_kernel<128, 1, 4, false>(sas::AttnArgs, int, int)` | 3 | 2.0 | 1.0 | 3.0 | 0.006 |" in out
    first = out[out.index("## first"):out.index("## second")]
    second = out[out.index("## second"):]
    assert "fwd_kernel" in first and "| 4096 | 1 | 2.0 | 2.0 |" in first and "dkv" not in first
    assert "| 4096 | 1 | 3.0 | 3.0 |" in second and "dkv_kernel" in second
