"""Average kernel durations from a rocprofv3 kernel-trace statistics file.

Reads the ``*_kernel_stats.csv`` that ``rocprofv3 --kernel-trace --stats``
writes for a bench run and records, for the batch-1 (GEMV) and batch-32
(matrix-core) megakernel instances, the average duration per launch, tagged
with the hash of the sources the kernels were built from.  bench.py reports
these durations next to its own HIP-event timings while the sources are
unchanged.

    python -m persistent_megakernel_latency_amd.kernel_stats \\
        --stats prof/bench_kernel_stats.csv --source-hash HASH \\
        --out profiles/megakernel_kernel_durations.json
"""
from __future__ import annotations

import argparse
import csv
import json

INSTANCES = {
    "batch1": "void wpk::megakernel<unsigned short, 256, 1024, false, false>",
    "batch32": "void wpk::megakernel<unsigned short, 256, 1024, false, true>",
    "baseline_phase_batch1": "void wpk::phase_kernel<unsigned short, 256, 1024, false>",
    "baseline_phase_batch32": "void wpk::phase_kernel<unsigned short, 256, 1024, true>",
}


def read_stats(path: str):
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
            avg = r.get("AverageNs") or r.get("Average(ns)") or r.get("AverageDurationNs")
            calls = r.get("Calls") or r.get("Count")
            if name and avg:
                rows[name.strip()] = (float(avg), int(float(calls)) if calls else None)
    return rows


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--source-hash", required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    rows = read_stats(a.stats)
    out = {"source_hash": a.source_hash, "stats_file": a.stats}
    for key, prefix in INSTANCES.items():
        hit = [(n, v) for n, v in rows.items() if n.startswith(prefix)]
        if hit:
            name, (avg_ns, calls) = hit[0]
            out[key] = {"kernel": name, "average_us": round(avg_ns / 1000.0, 2), "calls": calls}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
