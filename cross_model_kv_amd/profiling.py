"""Summaries of rocprofv3 counter runs: HBM traffic per launch and matrix-core busy cycles.

    python -m cross_model_kv_amd.profiling traffic FETCH_CSV WRITE_CSV WORKLOAD OUT_JSON [KERNEL]
    python -m cross_model_kv_amd.profiling mfma COUNTER_CSV WORKLOAD OUT_JSON KERNEL
    python -m cross_model_kv_amd.profiling counters COUNTER_CSV KERNEL

traffic: FETCH_CSV / WRITE_CSV are the `*_counter_collection.csv` files of two single-counter
passes (`rocprofv3 --pmc FETCH_SIZE ...` and `--pmc WRITE_SIZE ...`) of `bench.py
--copy-calibration`.  That bench option first runs one plain device copy of 1 GiB, whose
counter reading gives the bytes-per-KiB factor of each counter; the kernel's dispatches at the
workload's grid (its largest) are scaled by it.  KERNEL defaults to the map GEMM.

mfma: one pass with SQ_INSTS_MFMA, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: the clock the
chip ran (GRBM_GUI_ACTIVE per XCD over the dispatch's duration) and the matrix pipes' busy
cycles as a share of the SIMD cycles at that clock.

Every summary records a fingerprint of the kernel's code (its sources with comments and
layout removed), so that a reader (bench.py) can drop the figure once the code changes.
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
_CSRC = lambda *names: [os.path.join(HERE, "csrc", n) for n in names]
# The source files whose code decides each kernel's memory traffic and instruction mix.
KERNEL_SOURCES = {
    "map_bf16_kernel": _CSRC("gemm_bf16.hip", "lds_dma.h", "common.h"),
    "derope_kernel": _CSRC("rope.hip", "common.h"),
    "colsum_kernel": _CSRC("gram.hip", "common.h"),
    "gram_split_kernel": _CSRC("gram_x3.hip", "common.h"),
    "gram_x3_kernel": _CSRC("gram_x3.hip", "lds_dma.h", "common.h"),
}
GEMM_SOURCES = KERNEL_SOURCES["map_bf16_kernel"]
COPY_BYTES = 1 << 30
XCDS = 8          # MI355X: 8 XCDs, each with its own GRBM_GUI_ACTIVE instance
SIMDS = 1024      # 256 compute units x 4 SIMDs


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


def _per_dispatch(path, counter, with_time=False):
    vals = collections.defaultdict(float)
    names, grids, dur = {}, {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            vals[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
            grids[d] = int(r.get("Grid_Size") or 0)
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if with_time:
        return [(d, names[d], vals[d], grids[d], dur.get(d)) for d in sorted(vals)]
    return [(d, names[d], vals[d], grids[d]) for d in sorted(vals)]


def _is_kernel(name, kernel):
    """Kernel_Name is the demangled signature, e.g. 'void kvmap::derope_kernel<true, 128>(...)'."""
    return ("::" + kernel + "<") in name or ("::" + kernel + "(") in name


def _workload_launches(rows, kernel="map_bf16_kernel"):
    """The kernel's readings on the workload itself: its largest grid (the same run also times
    smaller launches of some kernels: short caches, the Y half of the fit batches)."""
    mine = [(v, g) for _, n, v, g in rows if _is_kernel(n, kernel)]
    if not mine:
        return []
    top = max(g for _, g in mine)
    return [v for v, g in mine if g == top]


def _scale(rows):
    copies = [v for _, n, v, _ in rows if "copyBuffer" in n]
    if not copies:
        raise SystemExit("no copy-calibration dispatch found (run bench.py --copy-calibration)")
    return COPY_BYTES / (max(copies) * 1024.0)


def traffic(fetch_csv, write_csv, workload, out_json, kernel="map_bf16_kernel"):
    f_rows = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w_rows = _per_dispatch(write_csv, "WRITE_SIZE")
    fs, ws = _scale(f_rows), _scale(w_rows)
    fk = _workload_launches(f_rows, kernel)
    wk = _workload_launches(w_rows, kernel)
    if not fk or not wk:
        raise SystemExit(f"no {kernel} dispatches in the counter files")
    fetch = sum(fk) / len(fk) * 1024.0 * fs
    write = sum(wk) / len(wk) * 1024.0 * ws
    out = {"kernel": kernel, "workload": workload,
           "kernel_code_fingerprint": kernel_fingerprint(KERNEL_SOURCES[kernel]),
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "hbm_bytes_per_launch": fetch + write, "fetch_scale_bytes_per_KiB": fs * 1024.0,
           "write_scale_bytes_per_KiB": ws * 1024.0, "dispatches": len(fk)}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def mfma(counter_csv, workload, out_json, kernel):
    """Clock and matrix-pipe busy share of the kernel's dispatches at the workload's grid."""
    rows = {c: _per_dispatch(counter_csv, c, with_time=True)
            for c in ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")}
    mine = {c: [r for r in v if _is_kernel(r[1], kernel)] for c, v in rows.items()}
    if not all(mine.values()):
        raise SystemExit(f"no {kernel} dispatches with all three counters in {counter_csv}")
    top = max(r[3] for r in mine["GRBM_GUI_ACTIVE"])
    pick = {c: {r[0]: r for r in v if r[3] == top} for c, v in mine.items()}
    ids = sorted(set.intersection(*(set(v) for v in pick.values())))
    per = []
    for d in ids:
        grbm = pick["GRBM_GUI_ACTIVE"][d][2] / XCDS
        secs = pick["GRBM_GUI_ACTIVE"][d][4]
        busy = pick["SQ_VALU_MFMA_BUSY_CYCLES"][d][2]
        per.append({"dispatch": d, "seconds": secs, "clock_GHz": grbm / secs / 1e9 if secs else None,
                    "mfma_insts": pick["SQ_INSTS_MFMA"][d][2], "mfma_busy_cycles": busy,
                    "mfma_busy_share": busy / (grbm * SIMDS)})
    avg = lambda key: sum(p[key] for p in per) / len(per)
    out = {"kernel": kernel, "workload": workload,
           "kernel_code_fingerprint": kernel_fingerprint(KERNEL_SOURCES[kernel]), "dispatches": len(per),
           "seconds": avg("seconds"), "clock_GHz": avg("clock_GHz"), "mfma_insts": avg("mfma_insts"),
           "mfma_busy_share": avg("mfma_busy_share")}
    if len(per) <= 8:
        out["per_dispatch"] = per
    else:  # a short summary: the spread over the dispatches and the first three of them
        out["range"] = {key: [min(p[key] for p in per), max(p[key] for p in per)]
                        for key in ("seconds", "clock_GHz", "mfma_busy_share")}
        out["first_dispatches"] = per[:3]
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v for k, v in out.items() if k not in ("per_dispatch", "first_dispatches")}, indent=1))


def counters(counter_csv, kernel):
    """Average of every counter in the file over the kernel's dispatches at its largest grid."""
    names = set()
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            names.add(r["Counter_Name"])
    out = {}
    for c in sorted(names):
        vals = _workload_launches(_per_dispatch(counter_csv, c), kernel)
        if vals:
            out[c] = sum(vals) / len(vals)
    out["dispatches"] = len(_workload_launches(_per_dispatch(counter_csv, sorted(names)[0]), kernel))
    print(json.dumps({"kernel": kernel, "kernel_code_fingerprint": kernel_fingerprint(KERNEL_SOURCES[kernel]),
                      "averages": out}, indent=1))
    return out


if __name__ == "__main__":
    if len(sys.argv) in (6, 7) and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:])
    elif len(sys.argv) == 6 and sys.argv[1] == "mfma":
        mfma(*sys.argv[2:])
    elif len(sys.argv) == 4 and sys.argv[1] == "counters":
        counters(*sys.argv[2:])
    else:
        print(__doc__)
        sys.exit(2)
