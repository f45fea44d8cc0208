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
    # RMSQ_SANITIZE=1 (tests/sanitize/run_sanitized.py): the program under
    # ASan / UBSan, over the sanitized host layer built there
    san = os.environ.get("RMSQ_SANITIZE") == "1"
    libdir = os.path.join(ROOT, "tests", "sanitize") if san else LIBDIR
    flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"] if san \
        else []
    # hip_runtime_api.h selects its AMD declarations by this macro (hipcc
    # defines it; a plain C compiler needs it spelled out)
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", *flags, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", out + ".tmp",
           "-L", libdir, "-lrmsq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
