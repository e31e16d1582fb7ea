"""Compile the HIP kernels and the C ABI into ``lib/libsgemm.so`` (gfx950).

Every HIP source is built with hipcc for gfx950 only, with packed FP32
instructions turned off (-Xclang -target-feature -Xclang -packed-fp32-ops);
the pure C++ argument checks are built with g++. Objects go to ``_build/`` at
the repository root; the shared library lands next to this file.
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
OBJDIR = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIBDIR, "libsgemm.so")

ARCH = "gfx950"
HIP_SOURCES = ["api.hip", "naive.hip", "tiled.hip", "regblock.hip", "scale.hip",
               "mfma_nn.hip", "mfma_nt.hip", "mfma_tn.hip", "mfma_tt.hip", "lowp_bf16.hip", "lowp_f16.hip", "noalloc.hip"]
CXX_SOURCES = ["args.cpp", "select.cpp"]
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror"]


def _hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        jobs.append([_hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, f"-I{INCLUDE}", "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for f in [ex.submit(_run, j) for j in jobs]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
