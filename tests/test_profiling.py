"""Host tests of the counter summary behind bench.py's `roofline.traffic` (no GPU)."""

import csv
import json

import pytest

from cross_model_kv_amd import profiling


def _write(path, text):
    path.write_text(text)
    return str(path)


def test_fingerprint_ignores_comments_and_layout(tmp_path):
    a = _write(tmp_path / "a.hip", 'int f(int x) {\n  // scale\n  return x * 2; /* twice */\n}\nconst char* s = "a // b";\n')
    b = _write(tmp_path / "b.hip", 'int f(int x) { return x * 2; }\n\n\nconst char* s = "a // b";')
    c = _write(tmp_path / "c.hip", 'int f(int x) { return x * 3; }\nconst char* s = "a // b";')
    d = _write(tmp_path / "d.hip", 'int f(int x) { return x * 2; }\nconst char* s = "a // c";')
    fa, fb, fc, fd = (profiling.kernel_fingerprint([p]) for p in (a, b, c, d))
    assert fa == fb          # comments and whitespace runs do not count
    assert fa != fc          # code does
    assert fa != fd          # and so does text inside a string literal, even after a "//"


def _counter_csv(path, counter, dispatches):
    """dispatches: (id, kernel name, grid size, [per-agent readings in KiB])"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, grid, vals in dispatches:
            for v in vals:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                            "Counter_Value": v})
    return str(path)


def test_traffic_scales_by_the_copy_and_keeps_the_workload_launches(tmp_path):
    gemm = "void kvmap::map_bf16_kernel<128>(kvmap::MapArgs, int, int, int, long, int, int)"
    small = "void kvmap::map_bf16_kernel<128>(kvmap::MapArgs, int, int, int, long, int, int)"
    copy = "__amd_rocclr_copyBuffer"
    # the 1 GiB copy reads as 1.25 GiB on FETCH_SIZE (factor 0.8) and as 0.5 GiB on WRITE_SIZE (factor 2)
    fetch = _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [
        (1, copy, 1 << 20, [(1 << 20) * 1.25 / 2, (1 << 20) * 1.25 / 2]),
        (2, small, 4096, [1000.0, 1000.0]),                       # a short-cache launch: smaller grid
        (3, gemm, 524288, [60000.0, 40000.0]),                    # per-agent rows are summed
        (4, gemm, 524288, [70000.0, 50000.0]),
    ])
    write = _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [
        (1, copy, 1 << 20, [(1 << 20) * 0.5]),
        (2, gemm, 524288, [8000.0]),
        (3, gemm, 524288, [12000.0]),
    ])
    out = tmp_path / "t.json"
    profiling.traffic(fetch, write, "test workload", str(out))
    r = json.loads(out.read_text())
    assert r["dispatches"] == 2
    assert r["fetch_bytes_per_launch"] == pytest.approx((100000.0 + 120000.0) / 2 * 1024 * 0.8)
    assert r["write_bytes_per_launch"] == pytest.approx((8000.0 + 12000.0) / 2 * 1024 * 2.0)
    assert r["hbm_bytes_per_launch"] == pytest.approx(r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"])
    assert r["kernel_code_fingerprint"] == profiling.kernel_fingerprint()


def test_traffic_needs_the_copy_calibration(tmp_path):
    gemm = "void kvmap::map_bf16_kernel<128>(kvmap::MapArgs, int, int, int, long, int, int)"
    fetch = _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(3, gemm, 524288, [1.0])])
    write = _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(3, gemm, 524288, [1.0])])
    with pytest.raises(SystemExit):
        profiling.traffic(fetch, write, "w", str(tmp_path / "t.json"))
