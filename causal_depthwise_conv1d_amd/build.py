"""Build libccv.so (and the measurement helper libccv_calib.so) in-tree for gfx950.

    python -m causal_depthwise_conv1d_amd.build

Each HIP translation unit is compiled by hipcc for --offload-arch=gfx950 (in
parallel), the host-only ABI layer by g++, and hipcc links the shared objects.
Packed-FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libccv.so")
CALIB_LIB = os.path.join(HERE, "libccv_calib.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", CSRC, "-I", INCLUDE]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", CSRC, "-I", INCLUDE]

KERNEL_SOURCES = ["ccv_cf.hip", "ccv_cl.hip", "ccv_update.hip", "ccv_bwd.hip", "ccv_bwd_static.hip",
                  "ccv_device_info.hip"]
HOST_SOURCES = ["ccv_api.cpp", "ccv_update_api.cpp", "ccv_bwd_api.cpp"]
CALIB_SOURCES = ["ccv_calib.hip"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"compile failed: {cmd[-1] if cmd else ''}")
    # hipcc's host pass does not know the device feature flag; drop that note.
    for line in (r.stdout + r.stderr).splitlines():
        if "packed-fp32-ops" in line or not line.strip():
            continue
        sys.stderr.write(line + "\n")


def _obj(src):
    return os.path.join(OBJ, os.path.splitext(src)[0] + ".o")


def build(verbose: bool = True) -> str:
    """Compile every source (always; no up-to-date check) and link both libraries."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in KERNEL_SOURCES + CALIB_SOURCES:
        jobs.append([HIPCC] + HIP_FLAGS + ["-c", "-o", _obj(s), os.path.join(CSRC, s)])
    for s in HOST_SOURCES:
        jobs.append(["g++"] + HOST_FLAGS + ["-c", "-o", _obj(s), os.path.join(CSRC, s)])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(_run, jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp]
         + [_obj(s) for s in KERNEL_SOURCES + HOST_SOURCES])
    os.replace(tmp, LIB)
    tmp = CALIB_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp]
         + [_obj(s) for s in CALIB_SOURCES])
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


def clean():
    shutil.rmtree(OBJ, ignore_errors=True)


if __name__ == "__main__":
    build()
