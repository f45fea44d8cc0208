"""The boundary from C: tests/c_abi/rmsq_c_check.c includes include/rmsq.h
alone, links librmsq.so and the HIP runtime with a plain C compiler, and
calls the entry points with raw device pointers and a stream of its own.

* CPU: the program builds (the header is valid C99) and its argument-error
  calls return the documented status codes (no GPU work).
* GPU: its residual_rmsnorm_fp8, rmsnorm_fp8 (e4m3fnuz, bf16 scales, offset
  1.0) and rmsnorm_fp4 outputs match the oracle on seeded rows.  It runs the
  copy __graft_entry__.build() made next to its source."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import compare_fp4, compare_fp8

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c_abi"))
import build_c_check as c_build  # noqa: E402


def test_c_program_builds_and_argument_errors(tmp_path):
    exe = c_build.build(out=str(tmp_path / "rmsq_c_check"))
    r = subprocess.run([exe, "errors"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "errors ok"


@pytest.mark.gpu
@pytest.mark.parametrize("shape", ["headline", "wide"])
def test_c_program_outputs_match_the_oracle(tmp_path, shape):
    """headline: 37 rows of the headline workload; wide: 9 x 65536 bf16 rows
    (the residual call stages them in LDS, the other two hold them in
    registers), from a process that uses the HIP runtime alone."""
    import torch
    from gpu_common import say

    assert os.path.exists(c_build.EXE), "tests/c_abi/rmsq_c_check is missing: run __graft_entry__.build()"
    gs = 40.0
    if shape == "headline":
        w = workloads.WORKLOADS[workloads.HEADLINE]
        rows, hidden = 37, w.hidden
        inp = workloads.make(w, rows=rows)
    else:
        rows, hidden = 9, 65536
        rng = np.random.default_rng(65536)
        inp = {"x": torch.from_numpy(rng.standard_normal((rows, hidden))).to(torch.bfloat16),
               "residual": torch.from_numpy(rng.standard_normal((rows, hidden))).to(torch.bfloat16),
               "gamma": torch.from_numpy(rng.uniform(0.5, 1.5, hidden)).to(torch.bfloat16)}
    x, r, g = (workloads.bits(inp[k]) for k in ("x", "residual", "gamma"))
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(np.array([rows, hidden], "<i8").tobytes())
        for a in (x, r, g):
            f.write(np.ascontiguousarray(a, "<u2").tobytes())
        f.write(np.array([gs], "<f4").tobytes())
    say(f"[c program] run {rows}x{hidden}")
    p = subprocess.run([c_build.EXE, "run", str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    n = rows * hidden
    buf = open(fout, "rb").read()
    sizes = [("codes", n, "u1"), ("scales", rows, "<f4"), ("ro", n, "<u2"), ("codes2", n, "u1"),
             ("scales2", rows, "<u2"), ("fp4", n // 2, "u1"), ("fp4s", n // 16, "u1")]
    out, off = {}, 0
    for name, cnt, dt in sizes:
        nb = cnt * np.dtype(dt).itemsize
        out[name] = np.frombuffer(buf[off:off + nb], dt)
        off += nb
    assert off == len(buf)
    kw = dict(in_dtype="bf16")
    ref = oracle.rmsnorm_fp8(x, g, residual=r, eps=1e-5, weight_offset=0.0, scale_ub=1200.0, out_fmt="e4m3fn",
                             scales_dtype="f32", **kw)
    y = oracle.rmsnorm_y(x, g, residual=r, eps=1e-5, weight_offset=0.0, **kw)["y"]
    say("  residual FP8:", compare_fp8(out["codes"].reshape(rows, hidden), out["scales"], ref, y, out_fmt="e4m3fn",
                                       scales_dtype="f32", gpu_residual_out=out["ro"].reshape(rows, hidden)))
    ref2 = oracle.rmsnorm_fp8(x, g, eps=1e-6, weight_offset=1.0, scale_ub=1e4, out_fmt="e4m3fnuz",
                              scales_dtype="bf16", **kw)
    y2 = oracle.rmsnorm_y(x, g, eps=1e-6, weight_offset=1.0, **kw)["y"]
    say("  FP8 fnuz:", compare_fp8(out["codes2"].reshape(rows, hidden), out["scales2"], ref2, y2, out_fmt="e4m3fnuz",
                                   scales_dtype="bf16"))
    ref4 = oracle.rmsnorm_fp4(x, g, global_scale=gs, eps=1e-6, weight_offset=0.0, **kw)
    y4 = oracle.rmsnorm_y(x, g, eps=1e-6, weight_offset=0.0, **kw)["y"]
    say("  FP4:", compare_fp4(out["fp4"].reshape(rows, hidden // 2), out["fp4s"].reshape(rows, hidden // 16), ref4, y4,
                              global_scale=gs))
