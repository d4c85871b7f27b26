"""Build libkvshare.so in-tree: host C++ with g++, HIP kernels with hipcc for
gfx950, linked against the HIP runtime.

    python -m attention_cross_layer_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvshare.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CXXFLAGS = ["-O2", "-fPIC", "-fvisibility=hidden", "-std=c++17", "-Wall", "-I", INCLUDE, "-I", CSRC]
HIPFLAGS = ["-O3", "-fPIC", "-fvisibility=hidden", "-std=c++17", f"--offload-arch={ARCH}",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]
# Per-file additions.  The factorized decode rescales and reads its MFMA
# accumulators with VALU instructions, which cannot take AGPR operands: in
# the AGPR form the compiler copied all 48 value accumulators into AGPRs and
# back on every page (about 165 v_accvgpr moves per page); in the VGPR form
# none (32.5 vs 33.4 us per 64K-context layer call, one box).
FILE_FLAGS = {"k_factorized.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    return cpp, hip


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


# The plain streaming-read kernel bench.py sets the decode kernels against
# (a measurement aid beside bench.py, not part of the library).
READ_SRC = os.path.join(ROOT, "bench_read.hip")
READ_LIB = os.path.join(ROOT, "bench_read.so")


def build_read_probe(verbose: bool = False) -> str:
    tmp = READ_LIB + ".tmp"
    _run([HIPCC] + HIPFLAGS + ["-shared", READ_SRC, "-o", tmp], verbose)
    os.replace(tmp, READ_LIB)
    return READ_LIB


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cpp, hip = sources()
    cmds = []
    objs = []
    for f in cpp:
        o = os.path.join(BUILD, f + ".o")
        cmds.append(["g++"] + CXXFLAGS + ["-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    for f in hip:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([HIPCC] + HIPFLAGS + FILE_FLAGS.get(f, []) + ["-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fvisibility=hidden", "-o", tmp] + objs
         + ["-Wl,--no-undefined"], verbose)
    os.replace(tmp, LIB)
    build_read_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
