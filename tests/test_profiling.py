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


def test_traffic_of_another_kernel_by_exact_name(tmp_path):
    """A kernel is picked by its own name (not one that merely contains it), at its largest grid,
    and its fingerprint covers its own sources."""
    copy = "__amd_rocclr_copyBuffer"
    der = "void kvmap::derope_kernel<true, 128>(void const*, void*, int const*, int, int, long, float2 const*)"
    other = "void kvmap::derope_kernel_probe<true>(void const*)"
    fetch = _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [
        (1, copy, 1 << 20, [(1 << 20) / 2]),
        (2, der, 81920, [3000.0]),
        (3, der, 2048, [5.0]),          # a short cache: smaller grid
        (4, other, 81920, [99999.0]),   # another kernel whose name starts the same
    ])
    write = _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [
        (1, copy, 1 << 20, [1 << 20]),
        (2, der, 81920, [2500.0]),
    ])
    out = tmp_path / "d.json"
    profiling.traffic(fetch, write, "wl", str(out), "derope_kernel")
    r = json.loads(out.read_text())
    assert r["kernel"] == "derope_kernel" and r["dispatches"] == 1
    assert r["fetch_bytes_per_launch"] == pytest.approx(3000.0 * 1024 * 2.0)
    assert r["write_bytes_per_launch"] == pytest.approx(2500.0 * 1024)
    assert r["kernel_code_fingerprint"] == profiling.kernel_fingerprint(profiling.KERNEL_SOURCES["derope_kernel"])
    assert r["kernel_code_fingerprint"] != profiling.kernel_fingerprint()


def test_mfma_summary_clock_and_busy_share(tmp_path):
    """Clock = GRBM_GUI_ACTIVE per XCD over the dispatch's duration; busy share = matrix-pipe busy
    cycles over (cycles per XCD x 1024 SIMDs); the workload's largest grid only."""
    k = "void kvmap::gram_x3_kernel(unsigned short const*)"
    path = tmp_path / "m.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
                               "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d, grid, grbm, busy in ((5, 4096, 8 * 2.0e6, 0.5 * 2.0e6 * 1024), (6, 512, 8 * 10.0, 1.0)):
            # 1 ms at 2.0 GHz; the small-grid dispatch is left out
            for name, v in (("GRBM_GUI_ACTIVE", grbm), ("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("SQ_INSTS_MFMA", 77.0)):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Grid_Size": grid, "Counter_Name": name,
                            "Counter_Value": v, "Start_Timestamp": 1_000_000, "End_Timestamp": 2_000_000})
    out = tmp_path / "m.json"
    profiling.mfma(str(path), "wl", str(out), "gram_x3_kernel")
    r = json.loads(out.read_text())
    assert r["dispatches"] == 1
    assert r["clock_GHz"] == pytest.approx(2.0)
    assert r["mfma_busy_share"] == pytest.approx(0.5)
