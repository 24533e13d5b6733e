"""Build the HIP library libnystrom.so in-tree for gfx950.

Usage: python -m efficient_transformer_attention_mean_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnystrom.so")

SOURCES = ["nys_landmarks.hip", "nys_apply.hip", "nys_backward.hip", "nys_layer.hip", "nys_error.hip", "nys_launch.hip",
           "nys_abi.hip", "nys_timing.hip"]
ROCM_LIB = "/opt/rocm/lib"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # Packed fp32 ops (v_pk_fma_f32 and friends) are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core accumulators in ordinary VGPRs: no copies to and from AGPRs.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libnystrom.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    # The layer's two projections are plain GEMMs on rocBLAS.
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, f"-L{ROCM_LIB}",
          f"-Wl,-rpath,{ROCM_LIB}", "-lrocblas", "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
