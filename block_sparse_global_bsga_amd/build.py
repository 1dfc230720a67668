"""Build libbsga.so (HIP, gfx950) in-tree with hipcc.

    python -m block_sparse_global_bsga_amd.build

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off (ordinary float code only), then linked into
``block_sparse_global_bsga_amd/libbsga.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsga.so")
SOURCES = ["bsga_api.cpp", "budget.cpp", "predict.hip", "select.hip", "probe.hip",
           "metrics.hip", "attention.hip", "backward.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsga)")


# Per-source extras.  The attention kernels never depend on NaN propagation
# (masked scores are -inf, not NaN), so they run with the IEEE mode bit off,
# which lets float max chains fold into v_max3 without canonicalising every
# MFMA result first.
EXTRA = {"attention.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
         "backward.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    for line in (r.stdout + r.stderr).splitlines():
        if line.strip() and noise not in line:
            print(line, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_layer.c")
C_CALLER = os.path.join(BUILD, "c_layer")


def build_c_caller(out: str = C_CALLER, verbose: bool = False) -> str:
    """Compile tests/c_layer.c, a plain C99 caller of bsga_layer that its GPU
    test runs, against the in-tree libbsga.so (found through a run path
    relative to the executable) and the HIP runtime."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    out_dir = os.path.dirname(os.path.abspath(out))
    os.makedirs(out_dir, exist_ok=True)
    rel = os.path.relpath(PKG, out_dir)
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), C_CALLER_SRC,
           "-L", PKG, "-lbsga", f"-Wl,-rpath,$ORIGIN/{rel}",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {C_CALLER_SRC}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_c_caller(verbose=True)
