"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer builds (no GPU).

  * the CPU oracle (oracle/txl_oracle.c) with tests/sanitize/oracle_driver.c,
    which calls every oracle function on small and edge-case shapes;
  * the host half of the C ABI (relative_position_memory_amd/csrc/txl_api.cpp,
    sanitizers on the host side only) linked with the library's other objects
    and tests/sanitize/abi_driver.c, which walks the size queries and every
    argument check that returns before a launch.
Each program must exit 0 with no sanitizer report (leak detection on).
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
REPORT = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    text = p.stdout + p.stderr
    assert p.returncode == 0, text[-4000:]
    assert not any(r in text for r in REPORT), text[-4000:]
    return text


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    subprocess.run(["gcc", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-g", "-O1", "-std=c11", "-fopenmp",
                    "-o", exe, os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "txl_oracle.c"), "-lm"], check=True)
    assert "oracle driver done" in _run(exe)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc missing")
def test_abi_host_side_under_asan_ubsan():
    from relative_position_memory_amd import build as B
    os.makedirs(OUT, exist_ok=True)
    objs = [o for o in glob.glob(os.path.join(B.OBJ, "*.o")) if "txl_api" not in o]
    if len(objs) < len(glob.glob(os.path.join(B.CSRC, "*.hip"))):
        B.build()
        objs = [o for o in glob.glob(os.path.join(B.OBJ, "*.o")) if "txl_api" not in o]
    api = os.path.join(OUT, "txl_api_san.o")
    # sanitizers on the host side only; the device code is the library's own
    subprocess.run(["hipcc", "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
                    "-I", os.path.join(ROOT, "include"),
                    "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer",
                    "-c", os.path.join(B.CSRC, "txl_api.cpp"), "-o", api],
                   check=True, capture_output=True)
    drv = os.path.join(OUT, "abi_driver.o")
    subprocess.run(["gcc", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1",
                    "-std=c11", "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv], check=True)
    exe = os.path.join(OUT, "abi_driver")
    subprocess.run(["hipcc", f"--offload-arch={B.ARCH}",
                    "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined",
                    "-o", exe, drv, api, *objs], check=True, capture_output=True)
    assert "0 failed expectations" in _run(exe)
