"""Build libgi.so (HIP, gfx950) in-tree with hipcc.

Flags:
  -ffp-contract=off      every fused multiply-add is written out (fmaf); the cutoff
                         rule's fp32 op sequence is part of the ABI contract.
  -munsafe-fp-atomics    fp32 atomicAdd lowers to the hardware global atomic add
                         (device memory from hipMalloc / torch is coarse-grained).
  -Xclang -target-feature -Xclang -packed-fp32-ops
                         no packed-FP32 instructions are generated.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgi.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["gi_api.hip", "k_preprocess.hip", "k_binning.hip", "k_raster_sum.hip", "k_raster_alpha.hip",
           "k_optim.hip", "k_params.hip", "k_ssim.hip", "k_adapt.hip"]
ARCH = os.environ.get("GI_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libgi.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
