"""Build libmnb.so for gfx950 in-tree.

hipcc compiles the kernels (mnb_gemv.hip, mnb_gemv_mfma4.hip,
mnb_gemm_mfma.hip, mnb_layout.hip); the host front end
(mnb_api.cpp) is plain C++ built with g++; hipcc links both into one shared
library next to this file.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmnb.so")
PROBE_LIB = os.path.join(HERE, "libmnb_probe.so")
ARCH = "gfx950"

HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE,
             "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile and link libmnb.so (always recompiles). Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-save-temps=obj"] if save_temps else []
    objs = []
    jobs = []
    for name in ("mnb_gemv", "mnb_gemv_mfma4", "mnb_gemm_mfma", "mnb_layout"):
        obj = os.path.join(BUILD, name + ".o")
        objs.append(obj)
        jobs.append(["hipcc", "-c", os.path.join(CSRC, name + ".hip"), "-o", obj]
                    + HIP_FLAGS + extra)
    api_o = os.path.join(BUILD, "mnb_api.o")
    objs.append(api_o)
    jobs.append(["g++", "-c", os.path.join(CSRC, "mnb_api.cpp"), "-o", api_o] + CXX_FLAGS)
    # The translation units are independent: compile them side by side.
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    # measurement support: read-only HBM streaming probe (bench only)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", "-shared", os.path.join(CSRC, "mnb_probe.hip"), "-o", tmp] + HIP_FLAGS,
         verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
