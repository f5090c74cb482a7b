"""Turn two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE) over a bench run into the
HBM-traffic record that bench.py reports for the dominant kernel.

    python -m sparse_mixture_experts_29_amd.traffic_summary FETCH_DIR WRITE_DIR \
        --workload NAME --copy-mib 1024 [--kernel-regex "grouped_gemm_bf16<0, 256>"]

Both passes must come from `bench.py ... --copy-mib M`, which also runs one device copy of M
MiB: its counters, against the bytes it is known to move, give the scale of each counter on
this GPU. The record (per-launch bytes of the kernel, scales, and the hash of the kernel's
source) is merged into profiles/traffic_counters.json; bench.py uses it only while the
kernel source still has that hash.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def source_hash(path: str) -> str:
    """Hash of a source file's code: comments and blank lines do not count, so a record
    stays valid across comment edits and goes stale on any change to the code."""
    code = []
    for line in open(path, encoding="utf-8"):
        line = re.sub(r"//.*", "", line).rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def _rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    for f in files:
        out.extend(csv.DictReader(open(f)))
    return out


def _per_dispatch_kib(rows, counter, regex):
    """Counter value (KiB) of each matching dispatch."""
    vals = {}
    for r in rows:
        if r.get("Counter_Name") != counter or not re.search(regex, r.get("Kernel_Name", "")):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(vals))
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def summarize(fetch_dir, write_dir, copy_mib, kernel_regex, copy_regex="copyBuffer"):
    copy_bytes = copy_mib * (1 << 20)
    fr, wr = _rows(fetch_dir), _rows(write_dir)
    f_copy = max(_per_dispatch_kib(fr, "FETCH_SIZE", copy_regex)) * 1024
    w_copy = max(_per_dispatch_kib(wr, "WRITE_SIZE", copy_regex)) * 1024
    f_k = statistics.median(_per_dispatch_kib(fr, "FETCH_SIZE", kernel_regex)) * 1024
    w_k = statistics.median(_per_dispatch_kib(wr, "WRITE_SIZE", kernel_regex)) * 1024
    fs, ws = copy_bytes / f_copy, copy_bytes / w_copy
    return dict(fetch_scale=fs, write_scale=ws, fetch_bytes_per_launch=f_k * fs,
                write_bytes_per_launch=w_k * ws, hbm_bytes_per_launch=f_k * fs + w_k * ws)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--kernel-regex", default=r"grouped_gemm_bf16<0, 256>")
    ap.add_argument("--kernel-name", default="grouped_gemm_bf16<kGemmGated, 256> (gate/up + SiLU*mul)")
    ap.add_argument("--source", default="grouped_mlp.hip")
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    rec = summarize(a.fetch_dir, a.write_dir, a.copy_mib, a.kernel_regex)
    src = os.path.join(ROOT, "sparse_mixture_experts_29_amd", "csrc", a.source)
    rec["kernel"] = a.kernel_name
    rec["source_sha256_16"] = source_hash(src)
    rec["command"] = a.command
    out = os.path.join(ROOT, "profiles", "traffic_counters.json")
    d = json.load(open(out)) if os.path.exists(out) else {}
    d[a.workload] = rec
    with open(out, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
