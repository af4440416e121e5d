"""Build ``liboctopus_dag.so`` in-tree for gfx950.

HIP sources are compiled with ``hipcc --offload-arch=gfx950`` (packed-fp32 ops
disabled), host C++ with ``g++`` against the HIP runtime headers, and everything is
linked into one shared library next to this file.  Objects go to ``_build/`` at the
repository root.  Always recompiles (the caller decides when to build).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liboctopus_dag.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["fwd.hip", "bwd.hip", "dq.hip", "decode.hip", "extend.hip", "rope.hip",
               "scan_chunk.hip", "noalloc.hip"]
CXX_SOURCES = ["plan.cpp", "api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source code-generation options.  The kernels never produce NaN on purpose, so
# fmaxf need not quiet NaN operands (that costs one extra instruction per maximum).
# VGPR-form MFMAs keep the accumulators in the architectural registers: in the default
# form the compiler puts them in AGPRs wherever a kernel needs more than 256 registers or
# runs one head per workgroup, and copies them back and forth around every VALU operation
# on them (the two-head attention kernels compile to the same code either way).  Measured
# per file: the forward, extend, decode and scan kernels are faster in VGPR form; the dK/dV
# pass (bwd.hip, more than 256 registers) and the one-head dQ pass (dq.hip) are faster in
# the default form.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
HIP_FILE_FLAGS: dict = {"fwd.hip": ["-fno-honor-nans", *_VGPR_FORM],
                        "decode.hip": ["-fno-honor-nans", *_VGPR_FORM],
                        "extend.hip": ["-fno-honor-nans", *_VGPR_FORM],
                        "scan_chunk.hip": _VGPR_FORM}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
             "-D__HIP_PLATFORM_AMD__"]


def _hipcc():
    return shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False, extra_cxx=(), out=LIB, extra_hip=(), csrc=CSRC,
          build_dir=BUILD) -> str:
    os.makedirs(build_dir, exist_ok=True)
    inc = ["-I" + INCLUDE, "-I" + csrc]
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        jobs.append([_hipcc(), *HIPCC_FLAGS, *HIP_FILE_FLAGS.get(src, ()), *extra_hip, *inc,
                     "-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(build_dir, src.replace(".cpp", ".o"))
        jobs.append(["g++", *CXX_FLAGS, *extra_cxx, *inc, "-I" + os.path.join(ROCM, "include"),
                     "-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        logs = list(ex.map(_run, jobs))
    if verbose:
        for cmd, log in zip(jobs, logs):
            print(" ".join(cmd))
            if log.strip():
                print(log)
    tmp = out + ".tmp"
    _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *extra_cxx,
          "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
