"""Build the host code under AddressSanitizer and UndefinedBehaviorSanitizer
(test infrastructure, CPU only):

* tests/sanitize/liboracle.so -- oracle/rmsq_oracle.c with the oracle's own
  flags plus the sanitizers;
* tests/sanitize/librmsq.so -- the library's host layer
  (csrc/rmsq_api.cpp: argument validation, shape choice, aliasing checks)
  built by the host C++ compiler, linked with tests/sanitize/launch_stubs.cpp
  in place of the kernels (a call that passes every check fails as a launch);
* the C program over the boundary (tests/c_abi) is built with the same
  flags against that library when RMSQ_SANITIZE=1 (build_c_check.py).

run_sanitized.py builds these and runs the CPU test suite against them."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "fp4_activation_quantization_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ORACLE_LIB = os.path.join(HERE, "liboracle.so")
HOST_LIB = os.path.join(HERE, "librmsq.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> None:
    _run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", *SAN, "-shared",
          "-fPIC", os.path.join(ROOT, "oracle", "rmsq_oracle.c"), "-o", ORACLE_LIB + ".tmp", "-lm"], verbose)
    os.replace(ORACLE_LIB + ".tmp", ORACLE_LIB)
    _run(["g++", "-std=c++17", "-O1", "-Wall", *SAN, "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          os.path.join(CSRC, "rmsq_api.cpp"), os.path.join(HERE, "launch_stubs.cpp"), "-o", HOST_LIB + ".tmp",
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")], verbose)
    os.replace(HOST_LIB + ".tmp", HOST_LIB)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
