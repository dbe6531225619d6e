"""Build libtbik.so (HIP, gfx950) in-tree with hipcc.

Numerics flags: no fp contraction, no fast-math, IEEE fp32 denormals,
correctly rounded fp32 divide and sqrt, and packed-fp32 instructions
disabled.  Every kernel source under csrc/ is compiled into one shared
library exporting the C ABI declared in include/tbik.h.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtbik.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["gemm.hip", "rowops.hip", "attention.hip", "training.hip", "microbench.hip",
           "tbik_abi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source (in parallel) and link libtbik.so."""
    objdir = os.path.join(ROOT, "_build", "tbik")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd)))
        if len(procs) >= jobs:
            s, p = procs.pop(0)
            if p.wait() != 0:
                raise RuntimeError("hipcc failed on " + s)
    for s, p in procs:
        if p.wait() != 0:
            raise RuntimeError("hipcc failed on " + s)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # every kernel launched from host code must have its stub in the library
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "_ZN4tbik" in ln]
    if missing:
        os.unlink(tmp)
        raise RuntimeError("libtbik.so has undefined kernel symbols: %s" % missing[:4])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
