"""GPU: the FP8 entry points on rows that are not whole, 16-byte aligned
vectors (any hidden, element-aligned pointers and strides), which run the
element-wise kernel, checked against the oracle; plus the FP8 hand rows
byte-exact on both kernels.

The Mojo pages' fused RMSNorm + FP8 functions take any shape (their input_fn
is generic in its SIMD width), so these rows are in the operation's domain."""
import json
import os

import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import workloads
from gpu_common import DEV, check_fp8, say

pytestmark = pytest.mark.gpu
TD = workloads.TORCH_DTYPES
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")))


def _inputs(rows, hidden, dt, seed, resid=False):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((rows, hidden))).to(TD[dt])
    r = torch.from_numpy(rng.standard_normal((rows, hidden))).to(TD[dt]) if resid else None
    g = torch.from_numpy(rng.uniform(0.5, 1.5, hidden)).to(TD[dt])
    return {"x": x, "residual": r, "gamma": g}


def _wl(op, rows, hidden, dt, **kw):
    return workloads.Workload("elementwise", op, rows, hidden, dt, 97, eps=1e-6, **kw)


@pytest.fixture(autouse=True)
def automatic_shapes():
    rq.set_tuning(0, 0, 0)
    yield
    rq.set_tuning(0, 0, 0)


@pytest.mark.parametrize("dt,hiddens", [("bf16", [1, 3, 7, 13, 100, 515, 4100, 8191, 16383]),
                                        ("f16", [2, 9, 1001, 6150]),
                                        ("f32", [1, 5, 127, 4097, 16382])])
@pytest.mark.parametrize("rows", [1, 3, 67, 300])
def test_any_width(dt, hiddens, rows):
    for h in hiddens:
        for resid in (False, True):
            op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
            w = _wl(op, rows, h, dt)
            say(f"[elementwise] {op} {dt} rows={rows} hidden={h} shape={rq.query_shape(rows, h, TD[dt], elementwise=True)}")
            check_fp8(w, _inputs(rows, h, dt, seed=h * 7 + rows, resid=resid), label=f"{op} {dt} {rows}x{h}")


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_formats_and_scale_types(fmt, sdt):
    for dt in ("bf16", "f32"):
        w = _wl("residual_rmsnorm_fp8", 70, 1003, dt, out_fmt=fmt, scales_dtype=sdt, weight_offset=0.5)
        say(f"[elementwise matrix] {dt} {fmt} {sdt}")
        check_fp8(w, _inputs(70, 1003, dt, seed=17, resid=True), label=f"{dt} {fmt} {sdt}")


@pytest.mark.parametrize("where", ["x", "residual"])
def test_in_place_residual_odd_width(where):
    w = _wl("residual_rmsnorm_fp8", 131, 2049, "bf16")
    say(f"[elementwise in place] over {where}")
    check_fp8(w, _inputs(131, 2049, "bf16", seed=23, resid=True), in_place=where, label=f"in place over {where}")


@pytest.mark.parametrize("waves,blocks", [(1, 0), (2, 0), (3, 0), (5, 0), (16, 0), (4, 7), (1, 3)])
def test_forced_shapes_and_row_strided_grid(waves, blocks):
    h = 1003  # needs 16 elements per lane at one wave
    w = _wl("residual_rmsnorm_fp8", 201, h, "f16")
    inp = _inputs(201, h, "f16", seed=29, resid=True)
    rq.set_tuning(waves, 0, blocks)
    s = rq.query_shape(201, h, torch.float16, elementwise=True)
    assert s["waves_per_row"] == waves
    say(f"[elementwise shape] waves={waves} blocks={blocks} {s}")
    check_fp8(w, inp, label=f"shape {waves} waves, {blocks} blocks")


def _offset_view(t: torch.Tensor, k: int) -> torch.Tensor:
    """A contiguous copy of t on the GPU whose first element sits k elements
    past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 16, dtype=t.dtype, device=DEV)
    v = flat[k:k + t.numel()].view(t.shape)
    v.copy_(t.to(DEV))
    return v


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_element_aligned_pointers(dt):
    """hidden a whole number of vectors, but x, gamma, residual and the
    codes start off 16-byte boundaries: the element-wise kernel runs and
    matches the oracle; the outputs around the views are left alone."""
    rows, h = 45, 2048
    inp = _inputs(rows, h, dt, seed=31, resid=True)
    x, r, g = _offset_view(inp["x"], 1), _offset_view(inp["residual"], 3), _offset_view(inp["gamma"], 1)
    ro_buf = torch.full((rows * h + 16,), 7, dtype=TD[dt], device=DEV)
    ro = ro_buf[2:2 + rows * h].view(rows, h)
    out_buf = torch.full((rows * h + 16,), 0xA5, dtype=torch.uint8, device=DEV)
    out = out_buf[5:5 + rows * h].view(rows, h)
    say(f"[elementwise pointers] {dt}")
    codes, scales, rout = rq.residual_rmsnorm_fp8(x, r, g, eps=1e-6, scale_ub=1200.0, out=out, residual_out=ro)
    torch.cuda.synchronize()
    assert torch.all(out_buf[:5] == 0xA5) and torch.all(out_buf[5 + rows * h:] == 0xA5)
    assert torch.all(ro_buf[:2] == 7) and torch.all(ro_buf[2 + rows * h:] == 7)
    # the same values through contiguous, aligned tensors (vector kernel) and
    # the oracle: both paths must agree with the oracle
    w = _wl("residual_rmsnorm_fp8", rows, h, dt, scale_ub=1200.0)
    check_fp8(w, inp, label=f"aligned {dt}")
    from gpu_common import oracle_fp8
    from parity import compare_fp8
    ref, y = oracle_fp8(w, inp)
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref, y, out_fmt=w.out_fmt,
                      scales_dtype=w.scales_dtype, gpu_residual_out=workloads.bits(rout.cpu()))
    say(f"  parity element-aligned {dt}: {rep}")


@pytest.mark.parametrize("resid", [False, True])
def test_element_strides(resid):
    """Row strides that keep rows off 16-byte boundaries (strided entry point)."""
    rows, h, dt = 67, 1000, "bf16"
    inp = _inputs(rows, h, dt, seed=37, resid=resid)
    xs, rs, ros, os_ = h + 3, h + 5, h + 1, h + 9
    xb = torch.zeros((rows, xs), dtype=TD[dt], device=DEV)
    xb[:, :h] = inp["x"].to(DEV)
    r = ro = None
    if resid:
        rb = torch.zeros((rows, rs), dtype=TD[dt], device=DEV)
        rb[:, :h] = inp["residual"].to(DEV)
        r = rb[:, :h]
        rob = torch.full((rows, ros), 7, dtype=TD[dt], device=DEV)
        ro = rob[:, :h]
    ob = torch.full((rows, os_), 0xA5, dtype=torch.uint8, device=DEV)
    say(f"[elementwise strides] resid={resid}")
    codes, scales, rout = rq.rmsnorm_fp8_strided(xb[:, :h], inp["gamma"].to(DEV), residual=r, residual_out=ro,
                                                eps=1e-6, scale_ub=1200.0, out=ob[:, :h])
    torch.cuda.synchronize()
    assert torch.all(ob[:, h:] == 0xA5)
    if resid:
        assert torch.all(rob[:, h:] == 7)
    from gpu_common import oracle_fp8
    from parity import compare_fp8
    op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
    w = _wl(op, rows, h, dt, scale_ub=1200.0)
    ref, y = oracle_fp8(w, inp)
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref, y, out_fmt=w.out_fmt,
                      scales_dtype=w.scales_dtype,
                      gpu_residual_out=workloads.bits(rout.contiguous().cpu()) if resid else None)
    say(f"  parity strided elementwise: {rep}")


@pytest.mark.parametrize("row", GOLDEN["fp8_rows"], ids=lambda r: r["id"])
@pytest.mark.parametrize("kernel", ["vector", "elementwise"])
def test_fp8_hand_rows_byte_exact(row, kernel):
    dt = row["in_dtype"]
    n = len(row["x"])
    epv = 4 if dt == "f32" else 8
    if kernel == "vector" and n % epv:
        pytest.skip("a row that is not whole vectors always takes the element-wise kernel")
    x = torch.tensor([row["x"]], dtype=torch.float64).to(TD[dt])
    g = torch.tensor(row["gamma"], dtype=torch.float64).to(TD[dt])
    # one element off a 16-byte boundary forces the element-wise kernel
    k = 1 if kernel == "elementwise" else 0
    x, g = _offset_view(x, k), _offset_view(g, k)
    sdt = TD[row["scales_dtype"]]
    say(f"[hand row] {row['id']} {kernel}")
    codes, scales = rq.rmsnorm_fp8(x, g, eps=row["eps"], weight_offset=row["weight_offset"],
                                   scale_ub=row["scale_ub"], out_fp8=row["out_fmt"], scales_dtype=sdt)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()[0]
    want = np.array([int(c, 16) for c in row["expect_codes"]])
    if row["id"] == "tie_row":
        # an exact tie in exact arithmetic: the fp32 quantization factor may
        # land on either side of it, so the neighbouring code is correct too
        assert np.all(np.abs(got.astype(int) - want) <= 1), (got, want)
    else:
        assert [f"0x{v:02X}" for v in got] == row["expect_codes"]
    if "expect_scale_bits" in row:
        assert f"0x{int(workloads.bits(scales.cpu())[0]):04X}" == row["expect_scale_bits"]
