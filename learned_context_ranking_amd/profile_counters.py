"""HBM traffic of the library's kernels from rocprofv3 counter runs.

Two counter passes over the same command (``bench.py --calib-copy``), one collecting
FETCH_SIZE and one WRITE_SIZE (KiB per dispatch), are reduced to bytes per launch for each
kernel, each counter scaled by what it reads for a plain copy of known size (the 256 MiB
``copy_`` that ``--calib-copy`` runs first). The result is written as
``profiles/traffic_<kernel>.txt`` together with a digest of the kernel's sources, so that a
later run can tell whether the counters still describe the code:

    python3 -m learned_context_ranking_amd.profile_counters FETCH_DIR WRITE_DIR OUT_DIR "COMMAND"
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
    "fwd": ("fwd_kernel<128, 1, 4, false>", ["attn_fwd.hip", "sas_common.h"]),
    "decode": ("decode_split_kernel<128, false, false>", ["decode.hip", "sas_common.h"]),
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


def main(argv):
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
