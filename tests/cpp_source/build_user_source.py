"""Build tests/cpp_source/libuser_source.so: a caller's translation unit that
instantiates the public template of include/rmsq_fused.hpp with a producer
of its own (hipcc, gfx950; links the in-tree librmsq.so).  Test
infrastructure: nothing in the library uses it."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "fp4_activation_quantization_amd")
SRC = os.path.join(HERE, "user_source.hip")
LIB = os.path.join(HERE, "libuser_source.so")


def build(out: str = LIB, verbose: bool = False) -> str:
    sys.path.insert(0, ROOT)
    from fp4_activation_quantization_amd import build as lib_build

    cmd = [lib_build.HIPCC, f"--offload-arch={lib_build.ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-x", "hip", SRC,
           "-o", out + ".tmp", "-L", PKG, "-lrmsq", "-Wl,-rpath," + PKG]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {SRC}:\n{err}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
