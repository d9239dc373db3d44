"""Build libbgb.so in-tree with hipcc for gfx950 (run: python -m bit_gemm_binarize_amd.build)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbgb.so")
CEIL_SRC = os.path.join(HERE, "ceilings", "ceilings.hip")
CEIL_LIB = os.path.join(HERE, "ceilings", "libbgb_ceilings.so")
OBJ = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    errs = [ln for ln in r.stderr.splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build_ceilings(verbose: bool = True) -> str:
    """The ceiling microbenchmarks (measurement only; not linked into libbgb.so)."""
    tmp = CEIL_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, "-shared", CEIL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEIL_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CEIL_LIB)
    if verbose:
        print(f"built {CEIL_LIB}")
    return CEIL_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        ceil = ex.submit(build_ceilings, verbose)
        objs = list(ex.map(_compile, srcs))
        ceil.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
