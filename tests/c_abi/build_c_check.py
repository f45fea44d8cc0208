"""Build tests/c_abi/rmsq_c_check, a C program that calls librmsq through
include/rmsq.h (host C, gcc; links the in-tree librmsq.so and the HIP
runtime).  Test infrastructure: nothing in the library uses it."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBDIR = os.path.join(ROOT, "fp4_activation_quantization_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(HERE, "rmsq_c_check.c")
EXE = os.path.join(HERE, "rmsq_c_check")


def build(out: str = EXE, verbose: bool = False) -> str:
    # hip_runtime_api.h selects its AMD declarations by this macro (hipcc
    # defines it; a plain C compiler needs it spelled out)
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", out + ".tmp",
           "-L", LIBDIR, "-lrmsq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
