"""Compile the CPU oracle (test infrastructure only) into oracle/_build/.

Plain gcc, -O2, no FMA contraction, no fast-math, SSE scalar binary32 (the
x86-64 default), so that every float operation in fp4_oracle.c is one IEEE
binary32 operation in the order written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "liboracle.so")

CFLAGS = [
    "-std=c11", "-O2", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> str:
    """Compile fp4_oracle.c every time it is called; return the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, os.path.join(HERE, "fp4_oracle.c"), "-lm", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
