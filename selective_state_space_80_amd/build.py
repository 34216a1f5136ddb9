"""Build libmamba_amd.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage:  python -m selective_state_space_80_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libmamba_amd.so")
# VALU issue-rate probe (measurement aid for the roofline; not part of the C ABI)
PROBE_SOURCE = "valu_probe.hip"
PROBE_LIBRARY = os.path.join(HERE, "libmamba_probe.so")
SOURCES = ["api.cpp", "scan_fwd.hip", "scan_bwd.hip", "ssd_fwd.hip", "conv1d_silu.hip", "state_update.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled on purpose: the kernels are written for
# scalar fp32 issue and must not be rewritten into v_pk_* by the compiler.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [hipcc()] + HIPCC_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    probe_obj = _compile(PROBE_SOURCE)
    tmp = PROBE_LIBRARY + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, probe_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIBRARY)
    if verbose:
        print("built", LIBRARY, "and", PROBE_LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
