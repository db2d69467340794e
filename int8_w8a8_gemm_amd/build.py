"""Build libw8a8.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m int8_w8a8_gemm_amd.build

Each source compiles to its own object under ``_build/``; the shared library
is linked into this package directory.  The GELU lookup table is generated
first, by a host program (csrc/gen_gelu_table.c, gcc + libquadmath).  Flags: gfx950 only, -O3, no floating
point contraction (the epilogue spells out its one fma), and packed-fp32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw8a8.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["quantize_rows.hip", "compact_rows.hip", "gemm_tiled.hip", "gemm_bf16.hip", "w8a8_api.hip"]
ABI_CHECK_SRC = os.path.join(os.path.dirname(HERE), "tests", "c", "abi_check.cpp")
ABI_CHECK = os.path.join(BUILD, "abi_check")
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{BUILD}"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    return err


def _gelu_table():
    """Generates _build/gelu_table.inc (the bf16 GELU table) with the host
    compiler; the generator fails if any entry's rounding is not certain."""
    gen = os.path.join(BUILD, "gen_gelu_table")
    _run(["gcc", "-O2", "-std=c11", "-Wall", os.path.join(CSRC, "gen_gelu_table.c"), "-o", gen,
          "-lquadmath", "-lm"])
    _run([gen, os.path.join(BUILD, "gelu_table.inc")])


def build(verbose: bool = False, jobs: int = 5) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    _gelu_table()

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        out = _run([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    # the C-ABI check program of the tests (uses the library with no PyTorch)
    _run([hipcc, "-O2", "-std=c++17", f"-I{INCLUDE}", ABI_CHECK_SRC, f"-L{HERE}", "-lw8a8",
          "-Wl,-rpath,$ORIGIN/..", "-o", ABI_CHECK])
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
