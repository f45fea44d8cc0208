"""GPU: rows wider than the register-resident kernels hold (more than 4096
16-byte vectors: 32768 16-bit or 16384 fp32 elements) run the wide-row
kernels, up to 10112 vectors (80896 16-bit or 40448 fp32 elements): rows
with a residual above 7 (16-bit FP8) or 6 (FP4, fp32) vectors per lane, and
any row whose LDS form fits two blocks on a CU, stage the row in LDS; the
others hold it in registers (5 to 10 vectors per lane, gamma in LDS).
Against the oracle: FP8 (both formats, every scale type, with and without
the residual, in place), FP4 (every block size, scale format and layout,
with and without the residual), row strides, each register width with a
partly filled last vector slot, and forced grids smaller than the row count
(blocks loop over rows)."""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import oracle
import workloads
from gpu_common import DEV, check_fp4, check_fp8, say
from parity import compare_fp8

pytestmark = pytest.mark.gpu
TD = workloads.TORCH_DTYPES
MAX16, MAX32 = 8 * 10112, 4 * 10112


@pytest.fixture(autouse=True)
def automatic_shapes():
    rq.set_tuning(0, 0, 0)
    yield
    rq.set_tuning(0, 0, 0)


def _inputs(rows, hidden, dt, seed, resid):
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.integers(-6, 6, (rows, 1)))
    x = torch.from_numpy(rng.standard_normal((rows, hidden)) * mag).to(TD[dt])
    r = torch.from_numpy(rng.standard_normal((rows, hidden)) * mag).to(TD[dt]) if resid else None
    return {"x": x, "residual": r, "gamma": torch.from_numpy(rng.uniform(0.5, 1.5, hidden)).to(TD[dt])}


def _gs(inp, w):
    amax = oracle.absmax(workloads.bits(inp["x"]), workloads.bits(inp["gamma"]), in_dtype=w.in_dtype, eps=w.eps,
                         weight_offset=w.weight_offset)
    return float(np.float32(448 * 6 / amax))


@pytest.mark.parametrize("dt,hidden", [("bf16", 32776), ("bf16", 65536), ("bf16", MAX16), ("f16", 40000),
                                       ("f32", 16388), ("f32", MAX32)])
@pytest.mark.parametrize("resid", [False, True])
def test_fp8_wide_rows(dt, hidden, resid):
    rows = 37
    assert rq.query_shape(rows, hidden, TD[dt], residual=resid)["waves_per_row"] == 16
    for fmt, sdt, off in (("e4m3fn", "f32", 0.0), ("e4m3fnuz", "bf16", 1.0)):
        op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
        w = workloads.Workload("wide", op, rows, hidden, dt, 95, eps=1e-6, weight_offset=off, out_fmt=fmt,
                               scales_dtype=sdt)
        inp = _inputs(rows, hidden, dt, seed=hidden + rows, resid=resid)
        say(f"[wide fp8] {op} {dt} {rows}x{hidden} {fmt} {sdt}")
        check_fp8(w, inp, label=f"wide {op} {dt} {rows}x{hidden} {fmt}")


def test_fp8_wide_in_place_and_forced_grid():
    rows, hidden = 37, 49152
    w = workloads.Workload("wide", "residual_rmsnorm_fp8", rows, hidden, "bf16", 95, eps=1e-6)
    inp = _inputs(rows, hidden, "bf16", seed=5, resid=True)
    say("[wide fp8] residual_out over x, then over residual")
    check_fp8(w, inp, in_place="x", label="wide in place over x")
    check_fp8(w, inp, in_place="residual", label="wide in place over residual")
    rq.set_tuning(0, 0, 3)  # 3 blocks: each loops over its rows
    say("[wide fp8] 3 blocks for 37 rows")
    check_fp8(w, inp, label="wide 3 blocks")


@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "ue8m0"), (32, "e4m3"), (16, "ue8m0")])
@pytest.mark.parametrize("swz", [False, True], ids=["rowmajor", "swizzled"])
@pytest.mark.parametrize("resid", [False, True])
def test_fp4_wide_rows(block, fmt, swz, resid):
    for dt, rows, hidden in (("bf16", 37, 65536), ("f32", 5, 20480), ("f16", 3, MAX16)):
        op = "residual_rmsnorm_fp4" if resid else "rmsnorm_fp4"
        w = workloads.Workload("wide", op, rows, hidden, dt, 95, eps=1e-6, fp4_block=block, fp4_scale=fmt,
                               fp4_swizzled=swz)
        inp = _inputs(rows, hidden, dt, seed=hidden + block, resid=resid)
        say(f"[wide fp4] {op} {dt} {rows}x{hidden} block={block} {fmt} swizzled={swz}")
        check_fp4(w, inp, _gs(inp, w), label=f"wide {op} {dt} {rows}x{hidden} {block} {fmt} swz={swz}")


# rows without a residual past one LDS block per CU: held in registers, the
# last of NV vector slots partly filled (NV = 6, 6, 7, 8, 9; NV = 5 and 10
# are the fp32 20480 and 16-bit 80896 rows above)
REG_ROWS = [("f32", 20484, 5121), ("bf16", 45056, 5632), ("bf16", 56000, 7000), ("bf16", 60000, 7500),
            ("f16", 72000, 9000)]


@pytest.mark.parametrize("dt,hidden,nvec", REG_ROWS, ids=[f"{d}-{h}" for d, h, _ in REG_ROWS])
def test_fp8_rows_held_in_registers(dt, hidden, nvec):
    assert hidden * {"bf16": 2, "f16": 2, "f32": 4}[dt] == nvec * 16
    for rows, grid in ((37, 0), (600, 0), (37, 3)):
        rq.set_tuning(0, 0, grid)  # 600 rows or 3 blocks: blocks loop over rows
        for fmt, sdt in (("e4m3fn", "f32"), ("e4m3fnuz", "f16")):
            w = workloads.Workload("wide", "rmsnorm_fp8", rows, hidden, dt, 95, eps=1e-6, out_fmt=fmt,
                                   scales_dtype=sdt)
            inp = _inputs(rows, hidden, dt, seed=hidden + rows + grid, resid=False)
            say(f"[wide fp8 registers] {dt} {rows}x{hidden} {fmt} grid={grid or 'auto'}")
            check_fp8(w, inp, label=f"wide registers {dt} {rows}x{hidden} {fmt} grid={grid}")


@pytest.mark.parametrize("block,fmt,swz", [(16, "e4m3", False), (32, "ue8m0", True), (16, "ue8m0", True),
                                           (32, "e4m3", False)])
def test_fp4_rows_held_in_registers(block, fmt, swz):
    for dt, rows, hidden, grid in (("bf16", 300, 45056, 0), ("bf16", 37, 60000, 3), ("f32", 37, 28672, 0),
                                   ("f16", 260, 72000, 0)):
        rq.set_tuning(0, 0, grid)
        w = workloads.Workload("wide", "rmsnorm_fp4", rows, hidden, dt, 95, eps=1e-6, fp4_block=block,
                               fp4_scale=fmt, fp4_swizzled=swz)
        inp = _inputs(rows, hidden, dt, seed=hidden + block + rows, resid=False)
        say(f"[wide fp4 registers] {dt} {rows}x{hidden} block={block} {fmt} swizzled={swz} grid={grid or 'auto'}")
        check_fp4(w, inp, _gs(inp, w), label=f"wide registers {dt} {rows}x{hidden} {block} {fmt} swz={swz}")


@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "ue8m0")])
def test_fp4_wide_round_product_and_offset(block, fmt):
    """The FlashInfer page's 16-bit x * w product (round_product) and a
    weight offset on wide rows: registers (no residual: 65536, f16 36000),
    LDS (with a residual at 65536: 8 vectors per lane)."""
    for dt, rows, hidden, resid, off in (("bf16", 37, 65536, False, 0.0), ("bf16", 37, 65536, True, 1.0),
                                         ("f16", 21, 36000, False, 1.0)):
        op = "residual_rmsnorm_fp4" if resid else "rmsnorm_fp4"
        w = workloads.Workload("wide", op, rows, hidden, dt, 95, eps=1e-6, weight_offset=off, fp4_block=block,
                               fp4_scale=fmt, fp4_round_product=True)
        inp = _inputs(rows, hidden, dt, seed=hidden + block + 7, resid=resid)
        if off:
            inp["gamma"] = (inp["gamma"].double() - 1.0).to(TD[dt])  # g' = gamma + 1 stays near 1
        say(f"[wide fp4 round_product] {op} {dt} {rows}x{hidden} block={block} {fmt} offset={off}")
        check_fp4(w, inp, _gs(inp, w), label=f"wide round_product {op} {dt} {rows}x{hidden} {block} {fmt}")


# rows with a residual held in registers: 16-bit FP8 up to 7 vectors per
# lane, FP4 and fp32 up to 6 (7125, 5632 and 6000 vectors)
RESID_REG_ROWS = [("bf16", 57000, 7125), ("f16", 45056, 5632), ("f32", 24000, 6000)]


@pytest.mark.parametrize("dt,hidden,nvec", RESID_REG_ROWS, ids=[f"{d}-{h}" for d, h, _ in RESID_REG_ROWS])
def test_fp8_residual_rows_held_in_registers(dt, hidden, nvec):
    assert hidden * {"bf16": 2, "f16": 2, "f32": 4}[dt] == nvec * 16
    for rows, grid in ((37, 0), (300, 0), (37, 3)):
        rq.set_tuning(0, 0, grid)  # 300 rows or 3 blocks: blocks loop over rows
        w = workloads.Workload("wide", "residual_rmsnorm_fp8", rows, hidden, dt, 95, eps=1e-6)
        inp = _inputs(rows, hidden, dt, seed=hidden + rows + grid, resid=True)
        say(f"[wide fp8 registers, residual] {dt} {rows}x{hidden} grid={grid or 'auto'}")
        check_fp8(w, inp, label=f"wide registers residual {dt} {rows}x{hidden} grid={grid}")
    rq.set_tuning(0, 0, 0)
    say(f"[wide fp8 registers, residual] {dt} residual_out over x, then over residual")
    check_fp8(w, inp, in_place="x", label="wide registers in place over x")
    check_fp8(w, inp, in_place="residual", label="wide registers in place over residual")


@pytest.mark.parametrize("block,fmt,swz,rp", [(16, "e4m3", False, False), (32, "ue8m0", True, False),
                                              (16, "e4m3", True, True)])
def test_fp4_residual_rows_held_in_registers(block, fmt, swz, rp):
    """rp: the FlashInfer page's 16-bit x * w product (round_product)."""
    for dt, rows, hidden, grid in (("bf16", 300, 45056, 0), ("bf16", 37, 49152, 3), ("f32", 37, 24000, 0)):
        rq.set_tuning(0, 0, grid)
        w = workloads.Workload("wide", "residual_rmsnorm_fp4", rows, hidden, dt, 95, eps=1e-6, fp4_block=block,
                               fp4_scale=fmt, fp4_swizzled=swz, fp4_round_product=rp)
        inp = _inputs(rows, hidden, dt, seed=hidden + block + rows, resid=True)
        say(f"[wide fp4 registers, residual] {dt} {rows}x{hidden} block={block} {fmt} swizzled={swz} "
            f"round_product={rp} grid={grid or 'auto'}")
        check_fp4(w, inp, _gs(inp, w), label=f"wide registers residual {dt} {rows}x{hidden} {block} {fmt}")


def test_fp8_wide_strided_rows():
    rows, hidden, stride = 21, 40000, 40960
    inp = _inputs(rows, hidden, "bf16", seed=9, resid=True)
    buf = torch.zeros((rows, stride), dtype=torch.bfloat16, device=DEV)
    rbuf = torch.zeros_like(buf)
    obuf = torch.full((rows, stride), 0xA5, dtype=torch.uint8, device=DEV)
    x, r, out = buf[:, :hidden], rbuf[:, :hidden], obuf[:, :hidden]
    x.copy_(inp["x"].to(DEV))
    r.copy_(inp["residual"].to(DEV))
    say("[wide fp8] strided rows")
    codes, scales, ro = rq.rmsnorm_fp8_strided(x, inp["gamma"].to(DEV), residual=r, scale_ub=1200.0, out=out)
    torch.cuda.synchronize()
    assert torch.all(obuf[:, hidden:] == 0xA5), "codes written outside the row views"
    w = workloads.Workload("wide", "residual_rmsnorm_fp8", rows, hidden, "bf16", 95, eps=1e-6)
    xb, rb, gb = (workloads.bits(inp[k]) for k in ("x", "residual", "gamma"))
    ref = oracle.rmsnorm_fp8(xb, gb, residual=rb, in_dtype="bf16", eps=1e-6, weight_offset=0.0, scale_ub=1200.0,
                             out_fmt="e4m3fn", scales_dtype="f32")
    y = oracle.rmsnorm_y(xb, gb, residual=rb, in_dtype="bf16", eps=1e-6, weight_offset=0.0)["y"]
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref, y, out_fmt="e4m3fn",
                      scales_dtype="f32", gpu_residual_out=workloads.bits(ro.cpu()))
    say(f"  parity {w.op} strided: {rep}")


def test_fp4_wide_strided_rows_with_residual():
    """Strided 45056-wide rows with a residual through the FP4 entry point
    (held in registers, 6 vectors per lane): byte-identical to the contiguous
    call, nothing written outside the row views."""
    rows, hidden, stride = 21, 45056, 46080
    inp = _inputs(rows, hidden, "bf16", seed=12, resid=True)
    buf = torch.zeros((rows, stride), dtype=torch.bfloat16, device=DEV)
    rbuf = torch.zeros_like(buf)
    obuf = torch.full((rows, stride // 2), 0xA5, dtype=torch.uint8, device=DEV)
    x, r, out = buf[:, :hidden], rbuf[:, :hidden], obuf[:, :hidden // 2]
    x.copy_(inp["x"].to(DEV))
    r.copy_(inp["residual"].to(DEV))
    g = inp["gamma"].to(DEV)
    gs = torch.tensor([30.0], dtype=torch.float32, device=DEV)
    say("[wide fp4 registers, residual] strided rows")
    c_p, c_s, c_ro = rq.residual_rmsnorm_fp4quant(x.contiguous(), r.contiguous(), g, global_scale=gs)
    s_p, s_s, s_ro = rq.rmsnorm_fp4quant_strided(x, g, residual=r, global_scale=gs, out=out)
    torch.cuda.synchronize()
    assert torch.equal(s_p, c_p) and torch.equal(s_s, c_s) and torch.equal(s_ro, c_ro)
    assert bool((obuf[:, hidden // 2:] == 0xA5).all()), "codes written outside the row views"


def test_fp8_strided_rows_held_in_registers():
    rows, hidden, stride = 21, 65536, 66560
    inp = _inputs(rows, hidden, "bf16", seed=10, resid=False)
    buf = torch.zeros((rows, stride), dtype=torch.bfloat16, device=DEV)
    obuf = torch.full((rows, stride), 0xA5, dtype=torch.uint8, device=DEV)
    x, out = buf[:, :hidden], obuf[:, :hidden]
    x.copy_(inp["x"].to(DEV))
    say("[wide fp8 registers] strided rows")
    codes, scales, _ = rq.rmsnorm_fp8_strided(x, inp["gamma"].to(DEV), scale_ub=1200.0, out=out)
    torch.cuda.synchronize()
    assert torch.all(obuf[:, hidden:] == 0xA5), "codes written outside the row views"
    xb, gb = workloads.bits(inp["x"]), workloads.bits(inp["gamma"])
    ref = oracle.rmsnorm_fp8(xb, gb, in_dtype="bf16", eps=1e-6, weight_offset=0.0, scale_ub=1200.0,
                             out_fmt="e4m3fn", scales_dtype="f32")
    y = oracle.rmsnorm_y(xb, gb, in_dtype="bf16", eps=1e-6, weight_offset=0.0)["y"]
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref, y, out_fmt="e4m3fn",
                      scales_dtype="f32")
    say(f"  parity rmsnorm_fp8 strided (registers): {rep}")


def test_beyond_the_widest_row_is_refused():
    x = torch.zeros((2, MAX16 + 16), dtype=torch.bfloat16, device=DEV)  # one FP4 block past the widest row
    g = torch.ones(MAX16 + 16, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rq.RmsqError, match="UNSUPPORTED"):
        rq.rmsnorm_fp8(x, g)
    with pytest.raises(rq.RmsqError, match="UNSUPPORTED"):
        rq.rmsnorm_fp4quant(x, g)
