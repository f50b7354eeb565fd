"""Build the gfx950 HIP library libfp8moe.so in-tree with hipcc.

The library is the whole compute path of the layer; the Python package only
marshals arguments to its C ABI (include/fp8moe.h).  `debug=True` builds the
same sources with FP8MOE_DEBUG into libfp8moe_debug.so: device-side checks of
the preconditions and index invariants, reported by every entry point.
"""
from __future__ import annotations

import os
import pathlib
import subprocess
import sys

HERE = pathlib.Path(__file__).resolve().parent
CSRC = HERE / "csrc"
LIB = HERE / "libfp8moe.so"
LIB_DEBUG = HERE / "libfp8moe_debug.so"
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    return res.returncode, err


def build(verbose: bool = False, resource_usage: bool = False, debug: bool = False) -> pathlib.Path:
    """Compile every HIP source into libfp8moe.so, or with `debug` into
    libfp8moe_debug.so (always recompiles; the sources compile in parallel,
    then link)."""
    from concurrent.futures import ThreadPoolExecutor

    lib = LIB_DEBUG if debug else LIB
    objdir = HERE / ("_build_debug" if debug else "_build")
    objdir.mkdir(exist_ok=True)
    tmp = lib.with_name(lib.name + ".tmp")
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    if debug:
        flags = ["-DFP8MOE_DEBUG=1"] + flags
    if resource_usage:
        flags = ["-Rpass-analysis=kernel-resource-usage"] + flags
    jobs = []
    for s in SOURCES:
        obj = objdir / (pathlib.Path(s).stem + ".o")
        jobs.append((obj, [_hipcc(), *flags, "-c", "-o", str(obj), str(CSRC / s)]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(lambda j: _run(j[1], verbose), jobs))
    for (obj, _), (rc, err) in zip(jobs, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {obj.stem} ({rc}):\n{err}")
        if err.strip() and (verbose or resource_usage):
            print(err, file=sys.stderr)
    rc, err = _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp)] +
                   [str(o) for o, _ in jobs], verbose)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    tmp.replace(lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, resource_usage="--usage" in sys.argv, debug="--debug" in sys.argv))
