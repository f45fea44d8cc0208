"""gated_rmsnorm_fp8: the FP8 kernel fed by the GatedProduct source (x = a * b
rounded once to the input type, produced as the kernel loads a and b)
against the oracle's gated_product followed by its rmsnorm_fp8, every element
compared; and bit-identical to rmsnorm_fp8 on the materialized product."""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import oracle
import workloads
from gpu_common import DEV, say
from parity import compare_fp8

pytestmark = pytest.mark.gpu

SC_T = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _inputs(rows, hidden, dt, seed):
    rng = np.random.default_rng(seed)
    td = workloads.TORCH_DTYPES[dt]
    a = torch.from_numpy(rng.standard_normal((rows, hidden)) * 2.0).to(td)
    b = torch.from_numpy(rng.standard_normal((rows, hidden))).to(td)
    g = torch.from_numpy(rng.uniform(0.5, 1.5, hidden)).to(td)
    return a, b, g


def _check(a, b, g, dt, *, eps=1e-6, off=0.0, ub=float("inf"), fmt="e4m3fn", sdt="f32", label=""):
    rows, hidden = a.shape
    da, db, dg = a.to(DEV), b.to(DEV), g.to(DEV)
    codes, scales = rq.gated_rmsnorm_fp8(da, db, dg, eps=eps, weight_offset=off, scale_ub=ub, out_fp8=fmt,
                                         scales_dtype=SC_T[sdt])
    torch.cuda.synchronize()
    x = oracle.gated_product(workloads.bits(a), workloads.bits(b), in_dtype=dt)
    gb = workloads.bits(g)
    kw = dict(in_dtype=dt, eps=eps, weight_offset=off)
    ref = oracle.rmsnorm_fp8(x, gb, scale_ub=ub, out_fmt=fmt, scales_dtype=sdt, **kw)
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref,
                      lambda: oracle.rmsnorm_y(x, gb, **kw)["y"], out_fmt=fmt, scales_dtype=sdt)
    say(f"  parity gated {label}: {rep}")
    # the same kernel on the product written out: the same bytes
    td = workloads.TORCH_DTYPES[dt]
    xd = torch.from_numpy(x.view(np.float32) if dt == "f32" else x.view(np.int16)).view(td).to(DEV)
    c2, s2 = rq.rmsnorm_fp8(xd, dg, eps=eps, weight_offset=off, scale_ub=ub, out_fp8=fmt, scales_dtype=SC_T[sdt])
    torch.cuda.synchronize()
    assert torch.equal(codes, c2) and torch.equal(scales.view(torch.uint8), s2.view(torch.uint8)), label


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,hidden", [(1, 8), (7, 4096), (300, 4096), (260, 1024), (33, 16384), (261, 2056)])
def test_gated_matches_oracle(dt, rows, hidden):
    if hidden % (4 if dt == "f32" else 8):
        pytest.skip("hidden is not whole vectors")
    say(f"[gated] {dt} {rows}x{hidden}")
    a, b, g = _inputs(rows, hidden, dt, seed=rows * 31 + hidden)
    _check(a, b, g, dt, label=f"{dt} {rows}x{hidden}")


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_gated_numerics_variants(dt):
    """A weight offset (fp64 products), a binding scale bound, fnuz codes,
    16-bit scales, a == b (shared memory) and ragged batch sizes."""
    a, b, g = _inputs(97, 2048, dt, seed=5)
    _check(a, b, g, dt, off=1.0, label=f"{dt} offset 1")
    _check(a, b, g, dt, ub=1e-3, fmt="e4m3fnuz", sdt="bf16", label=f"{dt} ub fnuz bf16 scales")
    _check(a, a, g, dt, sdt="f16", label=f"{dt} a == b")
    a2, b2, g2 = _inputs(513, 2048, dt, seed=6)
    _check(a2, b2, g2, dt, eps=0.25, label=f"{dt} 513 rows eps 0.25")


def test_gated_argument_checks():
    a = torch.zeros(4, 64, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):  # b of another type
        rq.gated_rmsnorm_fp8(a, torch.zeros(4, 64, dtype=torch.float16, device=DEV), g)
    over = a.view(torch.uint8).reshape(-1)[:256].view(4, 64)  # the codes written over an operand
    with pytest.raises(rq.RmsqError, match="ALIAS|alias|overlap"):
        rq.gated_rmsnorm_fp8(a, torch.ones_like(a), g, out=over)
    x = torch.zeros(4, 36, dtype=torch.bfloat16, device=DEV)  # 36 is not whole vectors
    with pytest.raises(rq.RmsqError):
        rq.gated_rmsnorm_fp8(x, x, torch.ones(36, dtype=torch.bfloat16, device=DEV))


def _user_lib():
    import ctypes
    import os

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cpp_source", "libuser_source.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: __graft_entry__.build() builds it")
    L = ctypes.CDLL(path)
    P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.user_abs_rmsnorm_fp8.argtypes = [I64, I64, I, P, P, F, F, F, I, P, I, P, P]
    L.user_abs_rmsnorm_fp8.restype = I
    return L


@pytest.mark.parametrize("dt,rows,hidden", [("bf16", 300, 4096), ("f16", 5, 1032), ("f32", 260, 2048)])
def test_public_template_with_a_callers_producer(dt, rows, hidden):
    """A caller's translation unit (tests/cpp_source/user_source.hip)
    instantiates rmsq_fused.hpp's template with a producer of its own,
    x = |a|: the oracle's rmsnorm_fp8 of |a|, and the library's rmsnorm_fp8
    on |a| written out, byte for byte."""
    import ctypes

    say(f"[user source] {dt} {rows}x{hidden}")
    a, _, g = _inputs(rows, hidden, dt, seed=hidden + rows)
    da, dg = a.to(DEV), g.to(DEV)
    out = torch.empty(rows, hidden, dtype=torch.uint8, device=DEV)
    sc = torch.empty(rows, dtype=torch.float32, device=DEV)
    code = {"f32": rq.F32, "f16": rq.F16, "bf16": rq.BF16}[dt]
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = _user_lib().user_abs_rmsnorm_fp8(rows, hidden, code, P(da), P(dg), 1e-6, 0.0, float("inf"), rq.E4M3FN,
                                          P(out), rq.F32, P(sc), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    xabs = oracle.round_to(dt, np.abs(oracle.value_of(dt, workloads.bits(a))))
    gb = workloads.bits(g)
    kw = dict(in_dtype=dt, eps=1e-6, weight_offset=0.0)
    ref = oracle.rmsnorm_fp8(xabs, gb, scale_ub=float("inf"), out_fmt="e4m3fn", scales_dtype="f32", **kw)
    rep = compare_fp8(out.cpu().numpy(), workloads.bits(sc.cpu()), ref, lambda: oracle.rmsnorm_y(xabs, gb, **kw)["y"],
                      out_fmt="e4m3fn", scales_dtype="f32")
    say(f"  parity user |a| {dt}: {rep}")
    c2, s2 = rq.rmsnorm_fp8(da.abs(), dg)
    torch.cuda.synchronize()
    assert torch.equal(out, c2) and torch.equal(sc, s2)
