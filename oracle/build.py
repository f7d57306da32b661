"""Builds the CPU oracle (test infrastructure) with gcc.

Plain C, fp64, OpenMP, -O3 without fast-math and without contraction: gcc then
keeps every sum in source order (no reassociation) and forms no fused
multiply-adds, so the flags change speed, not results.

  build()             oracle/liboracle.so, generic x86-64 code: what the tests,
                      the smoke check and any host load.
  build(native=True)  liboracle_native.so with -march=native, compiled on the
                      host that runs it (into a temporary directory unless
                      out_dir is given): the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "txl_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
FLAGS = ["-O3", "-ffp-contract=off", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
         "-Wextra"]


def native_lib_path(out_dir=None) -> str:
    return os.path.join(out_dir or tempfile.gettempdir(), f"txl_liboracle_native_{os.getuid()}.so")


def build(verbose: bool = False, native: bool = False, out_dir=None) -> str:
    lib = native_lib_path(out_dir) if native else LIB
    cmd = ["gcc", *FLAGS, *(["-march=native"] if native else []),
           "-o", lib + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def flags(native: bool = False) -> str:
    return " ".join(FLAGS + (["-march=native"] if native else []))


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
