"""HBM traffic and matrix-core use of the library's kernels from rocprofv3 counter runs.

Two counter passes over the same command (``bench.py --calib-copy``), one collecting
FETCH_SIZE and one WRITE_SIZE (KiB per dispatch), are reduced to bytes per launch for each
kernel, each counter scaled by what it reads for a plain copy of known size (the 256 MiB
``copy_`` that ``--calib-copy`` runs first). The result is written as
``profiles/traffic_<kernel>.txt`` together with a digest of the kernel's sources, so that a
later run can tell whether the counters still describe the code:

    python3 -m learned_context_ranking_amd.profile_counters FETCH_DIR WRITE_DIR OUT_DIR "COMMAND"

A third run collecting the derived counters MfmaFlopsBF16 (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)
and MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) is reduced to the bf16
matrix FLOPs each attention kernel executes per launch, its duration under the counters
and the matrix-core busy fraction, written as ``profiles/mfma_train_step.txt``:

    python3 -m learned_context_ranking_amd.profile_counters --mfma MFMA_DIR OUT_DIR "COMMAND"

A kernel trace (``rocprofv3 --kernel-trace --stats``, its ``*_results.db``) is summarised as a
markdown table per kernel; with ``--by-workload`` the dispatches are also split into the
bench's workloads (each begins with its input generation, torch's random-number kernels)
and the library's kernels listed per workload:

    python3 -m learned_context_ranking_amd.profile_counters --trace DB TITLE "COMMAND" [--by-workload NAME ...]

SQ counters (waits, instruction activity, matrix/vector co-execution) collected in several
runs are summarised per attention kernel with:

    python3 -m learned_context_ranking_amd.profile_counters --sq OUT_FILE "COMMAND" DIR [DIR ...]
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# kernel short name -> (substring of the device symbol, the sources its code comes from)
KERNELS = {
    "dkv": ("dkv_kernel<128, false>", ["attn_bwd.hip", "sas_common.h"]),
    "dq": ("dq_kernel<128, false>", ["attn_bwd.hip", "sas_common.h"]),
    "fwd": ("fwd3_kernel<128, false>", ["attn_fwd.hip", "sas_common.h"]),
    "decode": ("decode_split_kernel<128, false, false, 0>", ["decode.hip", "sas_common.h"]),
    "select": ("select_kernel<8, 0>", ["select.hip", "sas_common.h"]),
}
CALIB_BYTES = 256 << 20


def _code_lines(text: str):
    """The source's code without // comments, whitespace-trimmed, blank lines dropped: a
    comment edit does not change what the counters describe."""
    out = []
    for line in text.splitlines():
        cut = len(line)
        pos = line.find("//")
        while pos != -1:
            if line[:pos].count('"') % 2 == 0:   # not inside a string literal
                cut = pos
                break
            pos = line.find("//", pos + 2)
        code = line[:cut].strip()
        if code:
            out.append(code)
    return out


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNELS[kernel][1]:
        with open(os.path.join(ROOT, "learned_context_ranking_amd", "csrc", f), encoding="utf-8") as fh:
            h.update("\n".join(_code_lines(fh.read())).encode())
            h.update(b"\0")
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str, profiles_dir: str | None = None):
    """HBM bytes per launch recorded in profiles/traffic_<kernel>.txt, or None when the file
    is missing or the kernel's sources changed since the counters were taken."""
    if kernel not in KERNELS:
        return None
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), f"traffic_{kernel}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def profiled_mfma(kernel: str, profiles_dir: str | None = None):
    """{executed bf16 matrix FLOPs per launch, matrix-core busy %} recorded for an attention
    kernel in profiles/mfma_train_step.txt, or None when missing or the sources changed."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), "mfma_train_step.txt")
    if kernel not in MFMA_PER_PAIR_D or not os.path.exists(path):
        return None
    kv, sec = {}, None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("[") and "]" in line:
                sec = line[1:line.index("]")]
            elif sec == kernel and "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return {"executed_flop_per_launch": float(kv["mfma_bf16_flops_per_launch"]),
                "mfma_util_pct": float(kv["mfma_util_pct"])}
    except (KeyError, ValueError):
        return None


def _per_dispatch(d: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter from a rocprofv3 csv directory."""
    rows = defaultdict(float)
    names = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (f, r["Dispatch_Id"])
                rows[key] += float(r["Counter_Value"])   # summed over dimensions, if any
                names[key] = r["Kernel_Name"]
    out = defaultdict(list)
    for key, v in rows.items():
        out[names[key]].append(v)
    return out


def _calibration(per: dict) -> float:
    """Counter value (KiB) of the 256 MiB calibration copy."""
    cands = [vals[0] for name, vals in per.items() if "copy" in name.lower() and vals]
    cands = [v for v in cands if 0.25 * CALIB_BYTES / 1024 < v < 4 * CALIB_BYTES / 1024]
    if not cands:
        raise SystemExit("no calibration copy dispatch found (run bench.py with --calib-copy)")
    return cands[0]


def _per_dispatch_timed(d: str, counter: str):
    """{kernel name: [(value, duration ns)]} for one counter from a rocprofv3 csv directory."""
    rows = defaultdict(float)
    meta = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (f, r["Dispatch_Id"])
                rows[key] += float(r["Counter_Value"])
                meta[key] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = defaultdict(list)
    for key, v in rows.items():
        name, dur = meta[key]
        out[name].append((v, dur))
    return out


# executed bf16 matrix FLOPs per (query, key) pair of each attention kernel, by its design
MFMA_PER_PAIR_D = {"fwd": 4, "dq": 6, "dkv": 8}


def main_mfma(argv):
    mfma_dir, out_dir, command = argv[0], argv[1], argv[2]
    flops = _per_dispatch_timed(mfma_dir, "MfmaFlopsBF16")
    util = _per_dispatch_timed(mfma_dir, "MfmaUtil")
    path = os.path.join(out_dir, "mfma_train_step.txt")
    with open(path, "w") as fh:
        fh.write("# bf16 matrix-core use of the attention kernels per launch, from one rocprofv3 counter run of:\n")
        fh.write(f"#   {command}\n")
        fh.write("# MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (FLOPs the matrix cores executed);\n")
        fh.write("# MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) in %; durations are the\n")
        fh.write("# dispatches' own timestamps under counter collection (kernels serialised). Executed\n")
        fh.write("# TFLOP/s = MfmaFlopsBF16 / duration, against the 2500 TFLOP/s dense bf16 peak. The\n")
        fh.write("# design executes 4 d (fwd), 6 d (dq) and 8 d (dkv) FLOPs per attended (query, key) pair.\n")
        for short in ("fwd", "dq", "dkv"):
            sym = KERNELS[short][0]
            fv = [x for n, vals in flops.items() if sym in n for x in vals]
            uv = [x for n, vals in util.items() if sym in n for x in vals]
            if not fv:
                continue
            f_mean = sum(v for v, _ in fv) / len(fv)
            d_min = min(t for _, t in fv)
            d_mean = sum(t for _, t in fv) / len(fv)
            u_mean = sum(v for v, _ in uv) / len(uv) if uv else float("nan")
            fh.write(f"[{short}] {sym}\n")
            fh.write(f"dispatches = {len(fv)}\n")
            fh.write(f"mfma_bf16_flops_per_launch = {f_mean:.6g}\n")
            fh.write(f"attended_pairs_x_d_implied = {f_mean / MFMA_PER_PAIR_D[short]:.6g}\n")
            fh.write(f"duration_us_mean = {d_mean / 1e3:.1f}\n")
            fh.write(f"duration_us_min = {d_min / 1e3:.1f}\n")
            fh.write(f"executed_tflops_at_mean = {f_mean / d_mean / 1e3:.1f}\n")
            fh.write(f"executed_frac_of_bf16_peak = {f_mean / d_mean / 1e3 / 2500.0:.3f}\n")
            fh.write(f"mfma_util_pct = {u_mean:.1f}\n")
            fh.write(f"source_sha256 = {source_digest(short)}\n")
            print(f"{short}: {f_mean:.4g} bf16 MFMA FLOPs/launch, {d_mean / 1e3:.0f} us, "
                  f"{f_mean / d_mean / 1e3:.0f} TFLOP/s executed, MfmaUtil {u_mean:.1f} %")
    print("->", path)


def _short(name: str) -> str:
    if name.startswith("void at::") or "rocclr" in name:
        return "(torch) " + name[:60]
    return name[:90]


def main_trace(argv):
    import sqlite3
    db, title, command = argv[0], argv[1], argv[2]
    names = argv[4:] if len(argv) > 3 and argv[3] == "--by-workload" else []
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, duration, grid_x from kernels order by start").fetchall()
    print(f"# {title}\n\nCommand (run from /tmp on the MI355X box, repository at $R):\n\n    {command}\n")
    agg = defaultdict(list)
    for n, _, d, _ in rows:
        agg[n].append(d)
    print("| kernel | calls | avg us | min us | max us | total ms |\n|---|---:|---:|---:|---:|---:|")
    for n, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{_short(n)}` | {len(ds)} | {sum(ds) / len(ds) / 1e3:.1f} | {min(ds) / 1e3:.1f} | "
              f"{max(ds) / 1e3:.1f} | {sum(ds) / 1e6:.3f} |")
    if not names:
        return
    # workloads: runs of dispatches that start with torch's random-number kernels; the last
    # len(names) runs that launch library kernels are the named workloads, in order
    runs, cur, prev_rand = [], [], False
    for n, st, d, g in rows:
        rand = "distribution_elementwise" in n or "normal_kernel" in n
        if rand and not prev_rand and cur:
            runs.append(cur)
            cur = []
        cur.append((n, d, g))
        prev_rand = rand
    runs.append(cur)
    runs = [r for r in runs if any("sas::" in n for n, _, _ in r)][-len(names):]
    for wname, run in zip(names, runs):
        print(f"\n## {wname}\n\n| kernel | grid | calls | avg us | min us |\n|---|---:|---:|---:|---:|")
        per = defaultdict(list)
        for n, d, g in run:
            if "sas::" in n:
                per[(n, g)].append(d)
        for (n, g), ds in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            print(f"| `{_short(n)}` | {g} | {len(ds)} | {sum(ds) / len(ds) / 1e3:.1f} | {min(ds) / 1e3:.1f} |")


SQ_RATIOS = ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
             "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS")


def main_sq(argv):
    """Per-launch means of SQ counters of the attention kernels over several counter runs
    (one directory each), with each wait / activity counter as a fraction of the waves'
    resident cycles (SQ_WAVE_CYCLES) and the matrix cores' co-execution fraction
    (SQ_VALU_MFMA_COEXEC_CYCLES over SQ_VALU_MFMA_BUSY_CYCLES)."""
    out_path, command, dirs = argv[0], argv[1], argv[2:]
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as fh:
                for row in csv.DictReader(fh):
                    for short in ("fwd", "dq", "dkv"):
                        if KERNELS[short][0] in row["Kernel_Name"]:
                            vals[short][row["Counter_Name"]].append(float(row["Counter_Value"]))
    with open(out_path, "w") as fh:
        fh.write("# SQ counters of the attention kernels per launch (mean over dispatches), from rocprofv3\n")
        fh.write("# counter runs of (one run per group of counters):\n")
        fh.write(f"#   {command}\n")
        fh.write("# *_frac = counter / SQ_WAVE_CYCLES (share of the waves' resident cycles);\n")
        fh.write("# coexec_frac = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (share of the\n")
        fh.write("# matrix cores' busy cycles with vector instructions executing beside them).\n")
        for short in ("fwd", "dq", "dkv"):
            cs = vals.get(short)
            if not cs:
                continue
            avg = {c: sum(v) / len(v) for c, v in cs.items()}
            fh.write(f"[{short}] {KERNELS[short][0]}\n")
            for c in sorted(avg):
                fh.write(f"{c} = {avg[c]:.6g}\n")
            if avg.get("SQ_WAVE_CYCLES"):
                for c in SQ_RATIOS:
                    if c in avg:
                        fh.write(f"{c}_frac = {avg[c] / avg['SQ_WAVE_CYCLES']:.3f}\n")
            if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
                fh.write(f"coexec_frac = {avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}\n")
            fh.write(f"source_sha256 = {source_digest(short)}\n")
    print("->", out_path)


def main(argv):
    if argv[1] == "--mfma":
        return main_mfma(argv[2:])
    if argv[1] == "--sq":
        return main_sq(argv[2:])
    if argv[1] == "--trace":
        return main_trace(argv[2:])
    fetch_dir, write_dir, out_dir, command = argv[1], argv[2], argv[3], argv[4]
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(write_dir, "WRITE_SIZE")
    f_cal, w_cal = _calibration(fetch), _calibration(write)
    f_scale = CALIB_BYTES / (f_cal * 1024.0)
    w_scale = CALIB_BYTES / (w_cal * 1024.0)
    for short, (sym, _) in KERNELS.items():
        fv = [v for n, vals in fetch.items() if sym in n for v in vals]
        wv = [v for n, vals in write.items() if sym in n for v in vals]
        if not fv or not wv:
            continue
        f_kib = sum(fv) / len(fv)
        w_kib = sum(wv) / len(wv)
        rd = f_kib * 1024.0 * f_scale
        wr = w_kib * 1024.0 * w_scale
        path = os.path.join(out_dir, f"traffic_{short}.txt")
        with open(path, "w") as fh:
            fh.write(f"# HBM traffic of the {sym} kernel per launch, from two rocprofv3 counter runs of:\n")
            fh.write(f"#   {command}\n")
            fh.write(f"# (one with --pmc FETCH_SIZE, one with --pmc WRITE_SIZE; values are KiB per dispatch,\n")
            fh.write(f"#  averaged over {len(fv)} / {len(wv)} dispatches). Each counter is scaled by what it reads\n")
            fh.write(f"# for a plain copy of {CALIB_BYTES} bytes in the same run:\n")
            fh.write(f"#   copy FETCH_SIZE = {f_cal:.1f} KiB -> scale {f_scale:.4f}; "
                     f"copy WRITE_SIZE = {w_cal:.1f} KiB -> scale {w_scale:.4f}\n")
            fh.write(f"fetch_kib_per_dispatch = {f_kib:.1f}\n")
            fh.write(f"write_kib_per_dispatch = {w_kib:.1f}\n")
            fh.write(f"read_bytes_per_launch = {rd:.0f}\n")
            fh.write(f"write_bytes_per_launch = {wr:.0f}\n")
            fh.write(f"hbm_bytes_per_launch = {rd + wr:.0f}\n")
            fh.write(f"source_sha256 = {source_digest(short)}\n")
        print(f"{short}: read {rd / 1e9:.3f} GB + write {wr / 1e9:.3f} GB per launch -> {path}")


if __name__ == "__main__":
    main(sys.argv)
