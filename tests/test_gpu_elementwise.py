"""GPU: the FP8 entry points on rows that are not whole, 16-byte aligned
vectors, checked against the oracle.  Two kernels serve them: the phased
kernel (every tensor at the same offset from the 16-byte grid, e.g. any
hidden in contiguous tensors) and the element-wise kernel (anything else
that is element-aligned).  Each test places its tensors so that the kernel
it names is the one the library takes (the placement rules are those of
include/rmsq.h); outputs around the tensors must keep their fill.  The FP8
hand rows run byte-exact on all three kernels.

The Mojo pages' fused RMSNorm + FP8 functions take any shape (their input_fn
is generic in its SIMD width), so these rows are in the operation's domain."""
import json
import os

import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import workloads
from gpu_common import DEV, check_fp8, oracle_fp8, say
from parity import compare_fp8

pytestmark = pytest.mark.gpu
TD = workloads.TORCH_DTYPES
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")))
FILL_CODES, FILL_RESID = 0xA5, 7


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


def _offset_view(t: torch.Tensor, k: int, fill=None) -> torch.Tensor:
    """A contiguous GPU tensor of t's shape whose first element sits k
    elements past a 16-byte boundary, holding t (or `fill`), inside a buffer
    16 elements longer.  Returns (view, buffer)."""
    flat = torch.empty(t.numel() + 16, dtype=t.dtype, device=DEV)
    assert flat.data_ptr() % 16 == 0
    if fill is not None:
        flat.fill_(fill)
    v = flat[k:k + t.numel()].view(t.shape)
    if fill is None:
        v.copy_(t.to(DEV))
    return v, flat


# element offsets from the 16-byte grid (codes: bytes) that select each kernel
PLACEMENTS = {
    # every tensor 3 elements past the grid (16-bit; fp32 wraps to 3 of 4),
    # codes 3 bytes past it: the phased kernel
    "phased": {"x": 3, "residual": 3, "residual_out": 3, "gamma": 0, "out": 3},
    # residual off x's phase: the element-wise kernel
    "element": {"x": 1, "residual": 2, "residual_out": 1, "gamma": 1, "out": 0},
}


def run_placed(w, inp, place, label, in_place=None):
    """Run w's FP8 op on copies of inp placed per `place`; check the fills
    around every output and compare with the oracle."""
    dt, rows, h = w.in_dtype, w.rows, w.hidden
    x, _ = _offset_view(inp["x"], place["x"])
    g, _ = _offset_view(inp["gamma"], place["gamma"])
    out, out_buf = _offset_view(torch.empty((rows, h), dtype=torch.uint8), place["out"], fill=FILL_CODES)
    sc_t = TD[w.scales_dtype]
    kw = dict(eps=w.eps, weight_offset=w.weight_offset, scale_ub=w.scale_ub, out_fp8=w.out_fmt, out=out,
              scales_dtype=sc_t)
    ro = None
    if w.residual:
        r, _ = _offset_view(inp["residual"], place["residual"])
        if in_place == "x":
            ro = x
        elif in_place == "residual":
            ro = r
        else:
            ro, ro_buf = _offset_view(inp["x"], place["residual_out"], fill=FILL_RESID)
        codes, scales, rout = rq.residual_rmsnorm_fp8(x, r, g, residual_out=ro, **kw)
    else:
        codes, scales = rq.rmsnorm_fp8(x, g, **kw)
        rout = None
    torch.cuda.synchronize()
    n, o = rows * h, place["out"]
    assert torch.all(out_buf[:o] == FILL_CODES) and torch.all(out_buf[o + n:] == FILL_CODES)
    if w.residual and in_place is None:
        k = place["residual_out"]
        assert torch.all(ro_buf[:k] == FILL_RESID) and torch.all(ro_buf[k + n:] == FILL_RESID)
    ref, y = oracle_fp8(w, inp)
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref, y, out_fmt=w.out_fmt,
                      scales_dtype=w.scales_dtype,
                      gpu_residual_out=workloads.bits(rout.cpu()) if rout is not None else None)
    say(f"  parity {label}: {rep}")
    return rep


@pytest.mark.parametrize("kernel", ["contiguous", "element"])
@pytest.mark.parametrize("dt,hiddens", [("bf16", [1, 3, 7, 13, 100, 515, 4100, 8191, 16383]),
                                        ("f16", [2, 9, 1001, 6150]),
                                        ("f32", [1, 5, 127, 4097, 16382])])
@pytest.mark.parametrize("rows", [1, 3, 67, 300])
def test_any_width(dt, hiddens, rows, kernel):
    """Contiguous tensors of any width take the phased kernel (every row at
    its own offset from the grid, rows sharing boundary vectors)."""
    for h in hiddens:
        for resid in (False, True):
            op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
            w = _wl(op, rows, h, dt)
            inp = _inputs(rows, h, dt, seed=h * 7 + rows, resid=resid)
            say(f"[any width] {kernel} {op} {dt} rows={rows} hidden={h}")
            if kernel == "contiguous":
                check_fp8(w, inp, label=f"{op} {dt} {rows}x{h}")
            else:
                run_placed(w, inp, PLACEMENTS["element"], f"element {op} {dt} {rows}x{h}")


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_every_phase(dt):
    """Tensors all k elements past the grid, for every k, on widths that are
    and are not whole vectors: the phased kernel."""
    epv = 4 if dt == "f32" else 8
    for h in (8 * epv, 8 * epv + 1, 1000 + epv - 1):
        for k in range(epv):
            place = {"x": k, "residual": k, "residual_out": k, "gamma": 0, "out": k}
            w = _wl("residual_rmsnorm_fp8", 37, h, dt)
            say(f"[phase] {dt} hidden={h} k={k}")
            run_placed(w, _inputs(37, h, dt, seed=h + k, resid=True), place, f"phase {k} {dt} {h}")


@pytest.mark.parametrize("kernel", ["phased", "element"])
@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_formats_and_scale_types(fmt, sdt, kernel):
    for dt in ("bf16", "f32"):
        for resid in (False, True):
            op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
            w = _wl(op, 70, 1003, dt, out_fmt=fmt, scales_dtype=sdt, weight_offset=0.5)
            say(f"[matrix] {kernel} {op} {dt} {fmt} {sdt}")
            run_placed(w, _inputs(70, 1003, dt, seed=17, resid=resid), PLACEMENTS[kernel],
                       f"{kernel} {op} {dt} {fmt} {sdt}")


@pytest.mark.parametrize("kernel", ["phased", "element"])
@pytest.mark.parametrize("where", ["x", "residual"])
def test_in_place_residual(where, kernel):
    w = _wl("residual_rmsnorm_fp8", 131, 2049, "bf16")
    place = dict(PLACEMENTS[kernel], residual_out=PLACEMENTS[kernel][where])
    say(f"[in place] {kernel} over {where}")
    run_placed(w, _inputs(131, 2049, "bf16", seed=23, resid=True), place, f"{kernel} in place over {where}",
               in_place=where)


@pytest.mark.parametrize("waves,vpt,blocks", [(1, 0, 0), (2, 0, 0), (3, 0, 0), (5, 0, 0), (16, 0, 0), (4, 0, 7),
                                              (1, 0, 3), (1, 4, 0), (2, 4, 5), (8, 1, 0)])
def test_forced_shapes_and_row_strided_grid(waves, vpt, blocks):
    h = 1003  # up to 127 vectors on the grid; 16 elements per lane at one wave
    w = _wl("residual_rmsnorm_fp8", 201, h, "f16")
    inp = _inputs(201, h, "f16", seed=29, resid=True)
    rq.set_tuning(waves, vpt, blocks)
    say(f"[shape] waves={waves} vpt={vpt} blocks={blocks}")
    s = rq.query_shape(201, h, torch.float16, residual=True)
    assert s["waves_per_row"] == waves and (vpt == 0 or s["vectors_per_lane"] == vpt)
    check_fp8(w, inp, label=f"phased {waves}x{vpt} / {blocks} blocks")
    s = rq.query_shape(201, h, torch.float16, elementwise=True)
    assert s["waves_per_row"] == waves
    run_placed(w, inp, PLACEMENTS["element"], f"element {waves} waves / {blocks} blocks")


@pytest.mark.parametrize("kernel", ["phased", "element"])
@pytest.mark.parametrize("resid", [False, True])
def test_strides(resid, kernel):
    """Row strides that keep rows off 16-byte boundaries (strided entry
    point): all congruent modulo the vector (phased) or not (element)."""
    rows, h, dt = 67, 1000, "bf16"
    inp = _inputs(rows, h, dt, seed=37, resid=resid)
    if kernel == "phased":
        xs, rs, ros, os_ = h + 3, h + 11, h + 19, h + 3
    else:
        xs, rs, ros, os_ = h + 3, h + 5, h + 1, h + 9
    xb = torch.zeros((rows, xs), dtype=TD[dt], device=DEV)
    xb[:, :h] = inp["x"].to(DEV)
    r = ro = None
    if resid:
        rb = torch.zeros((rows, rs), dtype=TD[dt], device=DEV)
        rb[:, :h] = inp["residual"].to(DEV)
        r = rb[:, :h]
        rob = torch.full((rows, ros), FILL_RESID, dtype=TD[dt], device=DEV)
        ro = rob[:, :h]
    ob = torch.full((rows, os_), FILL_CODES, dtype=torch.uint8, device=DEV)
    say(f"[strides] {kernel} resid={resid}")
    codes, scales, rout = rq.rmsnorm_fp8_strided(xb[:, :h], inp["gamma"].to(DEV), residual=r, residual_out=ro,
                                                eps=1e-6, scale_ub=1200.0, out=ob[:, :h])
    torch.cuda.synchronize()
    assert torch.all(ob[:, h:] == FILL_CODES)
    if resid:
        assert torch.all(rob[:, h:] == FILL_RESID)
    op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
    w = _wl(op, rows, h, dt, scale_ub=1200.0)
    ref, y = oracle_fp8(w, inp)
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref, y, out_fmt=w.out_fmt,
                      scales_dtype=w.scales_dtype,
                      gpu_residual_out=workloads.bits(rout.contiguous().cpu()) if resid else None)
    say(f"  parity strided {kernel}: {rep}")


@pytest.mark.parametrize("row", GOLDEN["fp8_rows"], ids=lambda r: r["id"])
@pytest.mark.parametrize("kernel", ["vector", "phased", "element"])
def test_fp8_hand_rows_byte_exact(row, kernel):
    dt = row["in_dtype"]
    n = len(row["x"])
    epv = 4 if dt == "f32" else 8
    if kernel == "vector" and n % epv:
        pytest.skip("a row that is not whole vectors never takes the vector kernel")
    x = torch.tensor([row["x"]], dtype=torch.float64).to(TD[dt])
    g = torch.tensor(row["gamma"], dtype=torch.float64).to(TD[dt])
    k = {"vector": 0, "phased": 3 % epv, "element": 1}[kernel]
    x, _ = _offset_view(x, k)
    g, _ = _offset_view(g, 1 if kernel == "element" else 0)
    out, _ = _offset_view(torch.empty((1, n), dtype=torch.uint8), 0 if kernel == "element" else k, fill=0)
    say(f"[hand row] {row['id']} {kernel}")
    codes, scales = rq.rmsnorm_fp8(x, g, eps=row["eps"], weight_offset=row["weight_offset"],
                                   scale_ub=row["scale_ub"], out_fp8=row["out_fmt"], out=out,
                                   scales_dtype=TD[row["scales_dtype"]])
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
