"""Summaries of rocprofv3 output for the map GEMM (HBM traffic from counter runs).

    python -m cross_model_kv_amd.profiling traffic FETCH_CSV WRITE_CSV WORKLOAD OUT_JSON

FETCH_CSV / WRITE_CSV are the `*_counter_collection.csv` files of two single-counter passes
(`rocprofv3 --pmc FETCH_SIZE ...` and `--pmc WRITE_SIZE ...`) of
`bench.py --copy-calibration`.  That bench option first runs one plain device copy of 1 GiB,
whose counter reading gives the bytes-per-KiB factor of each counter; the map GEMM dispatches'
readings are scaled by it.  The output records the source hash of the kernel it was taken
on, so bench.py can drop the figure once the kernel changes.
"""

from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(HERE, "csrc", "gemm_bf16.hip")
COPY_BYTES = 1 << 30


def _per_dispatch(path, counter):
    vals = collections.defaultdict(float)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            vals[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    return [(d, names[d], vals[d]) for d in sorted(vals)]


def _scale(rows):
    copies = [v for _, n, v in rows if "copyBuffer" in n]
    if not copies:
        raise SystemExit("no copy-calibration dispatch found (run bench.py --copy-calibration)")
    return COPY_BYTES / (max(copies) * 1024.0)


def traffic(fetch_csv, write_csv, workload, out_json):
    f_rows = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w_rows = _per_dispatch(write_csv, "WRITE_SIZE")
    fs, ws = _scale(f_rows), _scale(w_rows)
    fk = [v for _, n, v in f_rows if "map_bf16_kernel" in n]
    wk = [v for _, n, v in w_rows if "map_bf16_kernel" in n]
    if not fk or not wk:
        raise SystemExit("no map_bf16_kernel dispatches in the counter files")
    fetch = sum(fk) / len(fk) * 1024.0 * fs
    write = sum(wk) / len(wk) * 1024.0 * ws
    with open(GEMM_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    out = {"kernel": "map_bf16_kernel", "workload": workload, "kernel_source_sha": sha,
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "hbm_bytes_per_launch": fetch + write, "fetch_scale_bytes_per_KiB": fs * 1024.0,
           "write_scale_bytes_per_KiB": ws * 1024.0, "dispatches": len(fk)}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    if len(sys.argv) != 6 or sys.argv[1] != "traffic":
        print(__doc__)
        sys.exit(2)
    traffic(*sys.argv[2:])
