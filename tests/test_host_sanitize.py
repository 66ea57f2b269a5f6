"""The host code of the C-ABI library (nc.cpp) built with AddressSanitizer
and UndefinedBehaviorSanitizer, driven through every entry point's host-side
paths (validation, sizing, layout) on the CPU by tests/abi_sanitize_driver.c.
The device code and the other translation units are the normal build's
objects; no GPU work is launched.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "sanitize")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _objects():
    from bwd_step_amd import build as B
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "nc.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    return objs


@pytest.mark.timeout(600)
def test_host_runtime_under_address_and_ub_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    nc_o = os.path.join(OUT, "nc_san.o")
    drv_o = os.path.join(OUT, "driver.o")
    exe = os.path.join(OUT, "abi_sanitize")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-I", os.path.join(ROOT, "include"),
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    subprocess.run([HIPCC, *common, "-std=c++17", *san, "-x", "hip", "-c",
                    os.path.join(ROOT, "bwd_step_amd", "csrc", "nc.cpp"), "-o", nc_o],
                   check=True, capture_output=True, text=True)
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "abi_sanitize_driver.c"), "-o", drv_o],
                   check=True, capture_output=True, text=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", *san, "-o", exe, drv_o, nc_o, *_objects()],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert r.returncode == 0 and "ok" in r.stdout, report[-4000:]
