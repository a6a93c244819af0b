"""Build libgdn.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m gated_deltanet_causal_amd.build

compiles every ``csrc/*.hip`` with hipcc (one object per source, in parallel)
under ``_build/`` and links ``gated_deltanet_causal_amd/libgdn.so``.  hipcc
cross-compiles the device code, so this runs on a host without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libgdn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # no packed fp32 (v_pk_*_f32) instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: on gfx950 independent MFMAs whose
    # accumulators live in AGPRs issue at ~46 cycles each when eight chains
    # alternate, against ~17 in VGPRs (measured on MI355X)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIBRARY + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY} from {len(sources)} sources")
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
