"""Build librmsq.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled on each call (no staleness checks), in parallel,
then linked into fp4_activation_quantization_amd/librmsq.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librmsq.so")
SOURCES = ["rmsq_api.cpp", "rmsq_fp8.hip", "rmsq_fp8_f16.hip", "rmsq_fp8_f32.hip", "rmsq_fp8_ragged.hip",
           "rmsq_fp8_sum.hip", "rmsq_fp8_sum_f16.hip", "rmsq_fp8_sum_f32.hip",
           "rmsq_fp8_ragged_f16.hip", "rmsq_fp8_ragged_f32.hip", "rmsq_fp4.hip", "rmsq_fp4_wave.hip", "rmsq_fp4_wave_f16.hip",
           "rmsq_fp4_f16.hip", "rmsq_fp4_f32.hip", "rmsq_wide.hip", "rmsq_wide_f16.hip", "rmsq_wide_f32.hip",
           "rmsq_convert.hip", "rmsq_stream.hip"]
ARCH = os.environ.get("RMSQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep hipcc from forming packed fp32 instructions (v_pk_fma_f32 & co.)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, obj: str, verbose: bool) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="rmsq_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(SOURCES, objs)))
        out = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
