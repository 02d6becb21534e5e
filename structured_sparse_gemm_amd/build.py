"""Builds libhinm.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhinm.so")
SOURCES = ("hinm_plan.cpp", "hinm_pack.hip", "hinm_spmm.hip", "hinm_gyro.hip")
ARCH = "gfx950"
# Packed-fp32 VALU forms are kept off for every kernel of this library.  MFMA
# accumulators stay in ordinary VGPRs: with one wave per SIMD the compiler
# would otherwise park them in AGPRs and copy them at every loop back edge.
DEVICE_FLAGS = ("-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1")
# The product kernels: leading scalar kernel arguments (up to ten) are
# preloaded into SGPRs at wave launch, so the first loads of a decode launch
# do not wait for the argument buffer.
FILE_FLAGS = {"hinm_spmm.hip": ("-mllvm", "-amdgpu-kernarg-preload-count=10")}


def _hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def build(verbose: bool = False) -> str:
    """Compiles every source and links ``libhinm.so`` next to this file; returns its path."""
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        cmd = [hipcc, "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Wno-unused-function", *DEVICE_FLAGS, *FILE_FLAGS.get(src, ()), "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l
                        and "not a recognized feature" not in l and l.strip())
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
        if verbose and msg:
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
