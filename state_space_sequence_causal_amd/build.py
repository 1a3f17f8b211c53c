"""Build libmamba2.so in-tree with hipcc for gfx950.

    python state_space_sequence_causal_amd/build.py

Every HIP source is compiled with packed-FP32 instructions disabled (the code
never relies on them), objects in parallel, then linked into one shared
library exporting only the C ABI of include/mamba2.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmamba2.so")
SOURCES = ["conv1d.hip", "ssd_prefill.hip", "state_update.hip", "rmsnorm.hip", "gemm.cpp", "mamba2_api.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include")]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # NEEDED libamdhip64.so.7 and libhipblaslt.so.1 bind to whichever libraries of those
    # sonames the process already holds (PyTorch's, when the binding imports torch first).
    cmd = ["/opt/rocm/llvm/bin/clang++", "-shared", "-fPIC", "-o", tmp, *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
