"""Build libsvgemm.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python speculative_verify_gemm_amd/build.py      # (by path: the package itself loads the library)

Every source is compiled with IEEE-exact fp32 settings (no FMA contraction,
correctly rounded division, denormals kept) because the transform and the
quantizers must reproduce integer codes bit for bit, and with packed-fp32
instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsvgemm.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["rht_quant.hip", "linear_w4.hip", "linear_w8.hip", "tree_accept.hip", "tree_deltanet.hip",
           "pass.hip", "layout.hip", "svgemm.hip"]

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def source_digest() -> str:
    """Digest of everything that decides the built kernels: the sources, the
    public header and the compile flags.  Profile summaries record it, so a
    counter reading can be matched to the code it was taken on."""
    import hashlib
    h = hashlib.sha256()
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "svgemm.h"), "rb") as f:
        h.update(f.read())
    h.update(" ".join(CFLAGS[:-4]).encode())  # flags, without the include paths
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: a ROCm toolchain is required to build libsvgemm.so")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libsvgemm.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


CALIB = os.path.join(HERE, "calib")
CALIB_PROGRAMS = ("mfma_peak", "hbm_read")


def build_calibration(verbose: bool = False) -> list:
    """The calibration programs (not part of the library): the int8 MFMA pipe
    and HBM streaming, measured on the GPU they run on."""
    out = []
    for name in CALIB_PROGRAMS:
        exe = os.path.join(CALIB, name)
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", os.path.join(CALIB, name + ".hip"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(f"built {exe}")
        out.append(exe)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_calibration(verbose=True)
    sys.exit(0)
