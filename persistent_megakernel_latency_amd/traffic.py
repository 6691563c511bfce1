"""HBM traffic of the megakernel from rocprofv3 hardware counters.

Two counter passes over a short bench run (FETCH_SIZE, then WRITE_SIZE, in
KiB per dispatch) and the same two passes over the microbenchmark's plain
copy kernel, which reads and writes exactly 1 GiB per dispatch.  The copy
gives the factor from each counter's reading to bytes; the megakernel's
average reading times that factor is its measured HBM traffic per launch.
The result is tagged with the hash of the kernel sources it was measured on:
bench.py only reports it while the sources are unchanged.

    python -m persistent_megakernel_latency_amd.traffic \\
        --fetch pmc_FETCH_SIZE/bench_counter_collection.csv \\
        --write pmc_WRITE_SIZE/bench_counter_collection.csv \\
        --copy-fetch pmc_copy_FETCH_SIZE/copy_counter_collection.csv \\
        --copy-write pmc_copy_WRITE_SIZE/copy_counter_collection.csv \\
        --source-hash HASH --out profiles/megakernel_llama1b_b1_traffic.json

The batch-1 instance is the default --kernel; the batch-32 (matrix-core)
instance is "void wpk::megakernel<unsigned short, 256, 1024, false, true>".
"""
from __future__ import annotations

import argparse
import csv
import json

COPY_BYTES = 1 << 30  # bytes the copy kernel reads, and writes, per dispatch


def mean_counter(path: str, kernel_prefix: str, counter: str) -> float:
    vals = []
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and row["Kernel_Name"].startswith(kernel_prefix):
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_prefix!r} in {path}")
    return sum(vals) / len(vals)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--kernel", default="void wpk::megakernel<unsigned short, 256, 1024, false, false>")
    ap.add_argument("--source-hash", required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    fetch_kib = mean_counter(a.fetch, a.kernel, "FETCH_SIZE")
    write_kib = mean_counter(a.write, a.kernel, "WRITE_SIZE")
    copy_fetch_kib = mean_counter(a.copy_fetch, "k_copy", "FETCH_SIZE")
    copy_write_kib = mean_counter(a.copy_write, "k_copy", "WRITE_SIZE")
    fetch_factor = COPY_BYTES / (copy_fetch_kib * 1024.0)
    write_factor = COPY_BYTES / (copy_write_kib * 1024.0)
    read_bytes = fetch_kib * 1024.0 * fetch_factor
    write_bytes = write_kib * 1024.0 * write_factor
    out = {
        "kernel": a.kernel,
        "source_hash": a.source_hash,
        "fetch_size_kib_per_launch": fetch_kib,
        "write_size_kib_per_launch": write_kib,
        "copy_fetch_size_kib": copy_fetch_kib,
        "copy_write_size_kib": copy_write_kib,
        "fetch_bytes_per_kib_reading": fetch_factor * 1024.0,
        "write_bytes_per_kib_reading": write_factor * 1024.0,
        "hbm_read_bytes_per_launch": read_bytes,
        "hbm_write_bytes_per_launch": write_bytes,
        "hbm_bytes_per_launch": read_bytes + write_bytes,
    }
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
