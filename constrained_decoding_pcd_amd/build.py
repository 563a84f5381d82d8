"""Builds libpcd.so in-tree for gfx950 (hipcc for the device code, g++ for
the host-only plan builder)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpcd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 instructions stay off; the compiler would otherwise form them from float2 code.
# Matrix-core accumulators live in ordinary VGPRs: with the accumulation
# registers the allocator moved partial sums between them around every
# matrix instruction of the unrolled loops, serialising them.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wall", "-Wno-unused-variable"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "pcd_kernels.hip"), "-o", os.path.join(BUILD, "pcd_kernels.o")],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "pcd_api.hip"), "-o", os.path.join(BUILD, "pcd_api.o")],
        ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, "pcd_plan.cpp"),
         "-o", os.path.join(BUILD, "pcd_plan.o")],
    ]
    with ThreadPoolExecutor(3) as ex:
        for r in ex.map(_run, jobs):
            if verbose and r.stderr:
                sys.stderr.write(r.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, os.path.join(BUILD, "pcd_kernels.o"),
          os.path.join(BUILD, "pcd_api.o"), os.path.join(BUILD, "pcd_plan.o")])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
