"""Build the CPU oracle (test infrastructure) into oracle/liboracle_tbik.so.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
the result.  Flags keep every float operation a single IEEE binary32
operation: no contraction into fma, no fast-math, SSE arithmetic on x86-64.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tbik_oracle.c")
LIB = os.path.join(HERE, "liboracle_tbik.so")

CFLAGS = [
    "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
