"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds tests/sanitize/host_checks.cpp against the C-ABI layer (api.hip, its host code
instrumented) and the host ridge solver (ridge.cpp, instrumented), with the other kernel files'
objects as they are, and runs it: validation of every kind of refused argument, the host ridge
solve on ragged shapes and thread counts (checked by its residual) and its refusals.  The
sanitizers stop the run at the first out-of-bounds access, use after free, overflow or other
undefined behaviour they detect."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cross_model_kv_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="no ROCm toolchain")
def test_host_code_under_asan_and_ubsan(tmp_path):
    from cross_model_kv_amd import build
    objs = [os.path.join(build.BUILD, s + ".o") for s in build.HIP_SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    api = str(tmp_path / "api_san.o")
    # host pass instrumented only: each sanitizer flag goes to the host compiler
    host_san = [a for f in SAN for a in ("-Xarch_host", f)]
    _run([HIPCC, *build.HIP_FLAGS, "-O1", "-g", *host_san, "-c", os.path.join(CSRC, "api.hip"), "-o", api])
    ridge = str(tmp_path / "ridge_san.o")
    _run(["g++", "-O1", "-g", "-std=c++17", "-mavx2", "-mfma", "-pthread", *SAN, "-c",
          os.path.join(CSRC, "ridge.cpp"), "-o", ridge])
    drv = str(tmp_path / "host_checks.o")
    _run(["g++", "-O1", "-g", "-std=c++17", *SAN, "-I/opt/rocm/include", "-c",
          os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", drv])
    exe = str(tmp_path / "host_checks")
    _run(["g++", *SAN, "-pthread", "-o", exe, drv, api, ridge, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks: 0 failure(s)" in out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
