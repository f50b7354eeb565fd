"""Build the CPU oracle (test infrastructure only) into oracle/libmoe_oracle.so.

Plain C11, IEEE fp32 with no contraction and no fast-math, so every step is
the sequence of operations written in moe_oracle.c.
"""
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
LIB = HERE / "libmoe_oracle.so"
SRC = HERE / "moe_oracle.c"

CFLAGS = [
    "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing",
    "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> pathlib.Path:
    """Compile the oracle library (always recompiles)."""
    tmp = LIB.with_suffix(".so.tmp")
    cmd = ["gcc", *CFLAGS, "-o", str(tmp), str(SRC), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    tmp.replace(LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
