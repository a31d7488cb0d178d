"""The host half of the library (argument validation, planning, the planner
override's parser, error messages: csrc/api.cpp) built with AddressSanitizer
and UndefinedBehaviorSanitizer and driven through every entry point and the
planning queries over a grid of shapes, CU caps and override strings
(tests/host/abi_driver.c).  Runs on the CPU: without a device every launch
stops at the device check, after all host-side arithmetic has run.  The
kernels' objects come from the regular build and are linked unchanged."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "moe_grouped_matmul_amd")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _objects():
    from moe_grouped_matmul_amd import build

    objs = [os.path.join(build.BUILD, os.path.splitext(s)[0] + ".o") for s in build.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    return objs


@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    import torch

    if torch.cuda.is_available():
        pytest.skip("host-only check; on a GPU host the calls would launch kernels")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-I", "/opt/rocm/include"]
    api_o = str(tmp_path / "api_san.o")
    drv_o = str(tmp_path / "driver.o")
    exe = str(tmp_path / "abi_driver")
    steps = [
        ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN, *inc, "-c", os.path.join(PKG, "csrc", "api.cpp"),
         "-o", api_o],
        ["gcc", "-std=c11", *SAN, *inc, "-c", os.path.join(ROOT, "tests", "host", "abi_driver.c"), "-o", drv_o],
        ["g++", *SAN, drv_o, api_o, *_objects(), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
         "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd[:2])} failed:\n{r.stderr[-4000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("DG_FORCE_CONFIG", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=500)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "0 failures" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
