"""Build librmsq.so (HIP, gfx950) in-tree with hipcc, and the measurement
library librmsq_probe.so (the streaming reference kernels bench.py times).

Every source is compiled on each call (no staleness checks), in parallel,
then linked into fp4_activation_quantization_amd/librmsq.so and
fp4_activation_quantization_amd/probe/librmsq_probe.so.
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
PROBE = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(PROBE, "librmsq_probe.so")
SOURCES = ["rmsq_api.cpp", "rmsq_fp8.hip", "rmsq_fp8_f16.hip", "rmsq_fp8_f32.hip", "rmsq_fp8_ragged.hip",
           "rmsq_fp8_sum.hip", "rmsq_fp8_sum_f16.hip", "rmsq_fp8_sum_f32.hip",
           "rmsq_fp8_ragged_f16.hip", "rmsq_fp8_ragged_f32.hip", "rmsq_fp4.hip", "rmsq_fp4_wave.hip", "rmsq_fp4_wave_f16.hip",
           "rmsq_fp4_f16.hip", "rmsq_fp4_f32.hip", "rmsq_wide.hip", "rmsq_wide_f16.hip", "rmsq_wide_f32.hip",
           "rmsq_convert.hip", "rmsq_fp8_gated.hip"]
ARCH = os.environ.get("RMSQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep hipcc from forming packed fp32 instructions (v_pk_fma_f32 & co.)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    # include/rmsq_fused.hpp pulls in the kernel templates
    "-I", CSRC,
]


def _compile(src: str, obj: str, verbose: bool) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)


def _link(objs: list[str], lib: str, verbose: bool) -> None:
    out = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out, lib)


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(PROBE, "rmsq_probe.hip")]
    with tempfile.TemporaryDirectory(prefix="rmsq_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1)) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
        _link(objs[:-1], LIB, verbose)
        _link(objs[-1:], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
