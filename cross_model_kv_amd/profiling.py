"""Summaries of rocprofv3 output for the map GEMM (HBM traffic from counter runs).

    python -m cross_model_kv_amd.profiling traffic FETCH_CSV WRITE_CSV WORKLOAD OUT_JSON

FETCH_CSV / WRITE_CSV are the `*_counter_collection.csv` files of two single-counter passes
(`rocprofv3 --pmc FETCH_SIZE ...` and `--pmc WRITE_SIZE ...`) of
`bench.py --copy-calibration`.  That bench option first runs one plain device copy of 1 GiB,
whose counter reading gives the bytes-per-KiB factor of each counter; the map GEMM dispatches'
readings are scaled by it.  The output records a fingerprint of the kernel's code (its
sources with comments and layout removed) so that bench.py can drop the figure once the
kernel's code changes.
"""

from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = [os.path.join(HERE, "csrc", n) for n in ("gemm_bf16.hip", "lds_dma.h", "common.h")]
COPY_BYTES = 1 << 30


_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/|\s+', re.S)


def kernel_fingerprint(paths=GEMM_SOURCES):
    """Hash of the map GEMM's code: string literals kept, comments dropped, whitespace runs
    collapsed, so that edits to comments or layout keep counter summaries valid."""
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        norm = _TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
        h.update(" ".join(norm.split()).encode())
    return h.hexdigest()[:16]


def _per_dispatch(path, counter):
    vals = collections.defaultdict(float)
    names, grids = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            vals[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
            grids[d] = int(r.get("Grid_Size") or 0)
    return [(d, names[d], vals[d], grids[d]) for d in sorted(vals)]


def _workload_launches(rows):
    """The map GEMM's readings on the workload itself: its largest grid (the run also times
    short caches, whose launches of the same kernel are smaller)."""
    mine = [(v, g) for _, n, v, g in rows if "map_bf16_kernel" in n]
    if not mine:
        return []
    top = max(g for _, g in mine)
    return [v for v, g in mine if g == top]


def _scale(rows):
    copies = [v for _, n, v, _ in rows if "copyBuffer" in n]
    if not copies:
        raise SystemExit("no copy-calibration dispatch found (run bench.py --copy-calibration)")
    return COPY_BYTES / (max(copies) * 1024.0)


def traffic(fetch_csv, write_csv, workload, out_json):
    f_rows = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w_rows = _per_dispatch(write_csv, "WRITE_SIZE")
    fs, ws = _scale(f_rows), _scale(w_rows)
    fk = _workload_launches(f_rows)
    wk = _workload_launches(w_rows)
    if not fk or not wk:
        raise SystemExit("no map_bf16_kernel dispatches in the counter files")
    fetch = sum(fk) / len(fk) * 1024.0 * fs
    write = sum(wk) / len(wk) * 1024.0 * ws
    out = {"kernel": "map_bf16_kernel", "workload": workload, "kernel_code_fingerprint": kernel_fingerprint(),
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
