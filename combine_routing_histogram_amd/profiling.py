"""Summaries of rocprofv3 output for this library's kernels.

`traffic`: HBM-side bytes per launch of one kernel from two counter runs
(rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE; both in KiB per
dispatch), each scaled by the ratio known bytes / counted bytes of a plain
device copy of known size recorded in the same run.  The result is written as
JSON with the hash of the kernel source it was measured on, so a reader can
tell when the figure has gone stale.

    python -m combine_routing_histogram_amd.profiling traffic \\
        --fetch-dir prof/pmc_fetch --write-dir prof/pmc_write \\
        --kernel k_combine --workload deepseek_v3_bf16 --calib-bytes 536870912 \\
        --out profiles/traffic_k_combine_deepseek_v3_bf16.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(PKG, "csrc", "epdc_kernels.hpp")
CALIB_PATTERNS = ("copyBuffer", "elementwise")


def _code_only(text: str) -> str:
    """The kernel source without comments and blank space, so that a comment
    edit does not mark counter figures as stale (string literals hold no
    comment markers in this file)."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(text: str = None) -> str:
    """Hash of the kernel code (comments and spacing ignored)."""
    if text is None:
        text = open(KERNEL_SRC).read()
    return hashlib.sha256(_code_only(text).encode()).hexdigest()[:16]


def read_counters(run_dir: str, counter: str) -> Dict[str, List[float]]:
    """{kernel name: [counter value per dispatch]} from a rocprofv3 csv run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {run_dir}")
    per: Dict[str, Dict[str, float]] = {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                key = row.get("Dispatch_Id") or row.get("Correlation_Id")
                # a counter may be reported per dimension/instance: sum them per dispatch
                per.setdefault(name, {})
                per[name][key] = per[name].get(key, 0.0) + float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def _pick(values: Dict[str, List[float]], needle: str) -> List[float]:
    hits = [k for k in values if needle in k]
    if not hits:
        raise KeyError(f"no kernel matching {needle!r} in {sorted(values)}")
    out: List[float] = []
    for k in hits:
        out += values[k]
    return out


def traffic(fetch_dir: str, write_dir: str, kernel: str, calib_bytes: int) -> dict:
    f = read_counters(fetch_dir, "FETCH_SIZE")
    w = read_counters(write_dir, "WRITE_SIZE")
    calib = next(p for p in CALIB_PATTERNS if any(p in k for k in f))
    # the calibration copy is the largest launch of the copy kernel (the run
    # also uploads its inputs with small copies)
    cf = max(_pick(f, calib)) * 1024.0   # KiB -> bytes
    cw = max(_pick(w, calib)) * 1024.0
    kf = statistics.median(_pick(f, kernel)) * 1024.0
    kw = statistics.median(_pick(w, kernel)) * 1024.0
    sf, sw = calib_bytes / cf, calib_bytes / cw
    return {
        "kernel": kernel,
        "launches_matched": sorted(k for k in f if kernel in k),
        "fetch_bytes_raw": kf, "write_bytes_raw": kw,
        "calibration_kernel": calib, "calibration_bytes": calib_bytes,
        "calibration_fetch_raw": cf, "calibration_write_raw": cw,
        "fetch_scale": sf, "write_scale": sw,
        "hbm_bytes_per_launch": kf * sf + kw * sw,
        "kernel_source_sha256_16": kernel_source_hash(),
    }


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch-dir", required=True)
    t.add_argument("--write-dir", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--command", default="")
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    d = traffic(a.fetch_dir, a.write_dir, a.kernel, a.calib_bytes)
    d["workload"] = a.workload
    d["command"] = a.command
    with open(a.out, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d, indent=1))


if __name__ == "__main__":
    main()
