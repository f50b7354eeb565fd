"""Host code under AddressSanitizer and UndefinedBehaviourSanitizer (CPU only).

- The CPU oracle (oracle/moe_oracle.c) built with gcc and both sanitizers,
  driven through every entry point on small seeded layers
  (tests/sanitize/oracle_driver.c).
- The HIP library's host code: abi.hip (validation, workspace layout, tile
  planning) and batching.hip (moe_group_tokens, moe_k_tiers) compiled with
  both sanitizers on the host side only (the device code is built as usual),
  linked with the release objects of the kernel files, and driven through
  their GPU-free paths (tests/sanitize/abi_host_driver.c).  The kernel files'
  launchers are not instrumented; nothing here touches a GPU.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), which
fails the test.  Leak checking is off for the library driver: the HIP
runtime that the library loads keeps allocations until exit."""
import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SAN = ROOT / "tests" / "sanitize"
ROCM = pathlib.Path(os.environ.get("ROCM_PATH", "/opt/rocm"))
HIPCC = ROCM / "bin" / "hipcc"
CLANG = ROCM / "llvm" / "bin" / "clang"
RELEASE_OBJ = ROOT / "fp8_moe_layer_amd" / "_build"
KERNEL_FILES = ("kernels_route", "kernels_permute", "kernels_expert", "kernels_persistent")


def _run(cmd, **kw):
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True, timeout=600, **kw)
    assert res.returncode == 0, f"{' '.join(map(str, cmd))}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off", "-pthread",
          "-o", exe, SAN / "oracle_driver.c", ROOT / "oracle" / "moe_oracle.c", "-lm"])
    res = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle driver ok" in res.stdout


@pytest.mark.skipif(not HIPCC.exists() or not CLANG.exists(), reason="ROCm toolchain not found")
def test_library_host_code_under_address_and_ub_sanitizers(tmp_path):
    objs = [RELEASE_OBJ / f"{k}.o" for k in KERNEL_FILES]
    if not all(o.exists() for o in objs):
        pytest.skip("release objects not built (fp8_moe_layer_amd/build.py)")
    csrc = ROOT / "fp8_moe_layer_amd" / "csrc"
    san_objs = []
    for src in ("abi", "batching"):
        o = tmp_path / f"{src}.o"
        # host-side sanitizers only: each -fsanitize= applies to the host pass
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-c", "-o", o, csrc / f"{src}.hip"])
        san_objs.append(o)
    lib = tmp_path / "libfp8moe_hostsan.so"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *san_objs, *objs])
    exe = tmp_path / "abi_host_driver"
    _run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
          SAN / "abi_host_driver.c", f"-L{tmp_path}", "-lfp8moe_hostsan",
          f"-Wl,-rpath,{tmp_path}"])
    res = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
                               UBSAN_OPTIONS="print_stacktrace=1"))
    assert "abi host driver ok" in res.stdout
