"""Build the gfx950 HIP library libfp8moe.so in-tree with hipcc.

The library is the whole compute path of the layer; the Python package only
marshals arguments to its C ABI (include/fp8moe.h).
"""
from __future__ import annotations

import os
import pathlib
import subprocess
import sys

HERE = pathlib.Path(__file__).resolve().parent
CSRC = HERE / "csrc"
LIB = HERE / "libfp8moe.so"
SOURCES = ["kernels_route.hip", "kernels_permute.hip", "kernels_expert.hip", "kernels_persistent.hip",
           "abi.hip", "batching.hip"]
ARCH = os.environ.get("FP8MOE_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off: hipcc only uses them when allowed to
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = pathlib.Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def build(verbose: bool = False, resource_usage: bool = False) -> pathlib.Path:
    """Compile every HIP source into libfp8moe.so (always recompiles)."""
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [_hipcc(), *HIPCC_FLAGS, "-o", str(tmp)] + [str(CSRC / s) for s in SOURCES]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and (verbose or resource_usage):
        print(err, file=sys.stderr)
    tmp.replace(LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, resource_usage="--usage" in sys.argv))
