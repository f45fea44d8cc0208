"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

* Every workload at a reduced row count, element by element (sizes that span
  several blocks of the persistent grid and leave ragged tails).
* Every workload at its full size, in the launch configuration the benchmark
  times, every row compared (the oracle runs over row chunks); the boundary
  flips of the whole tensor are held to the 0.01% cap.
* Edge cases: empty input, ragged and minimal hidden sizes, the largest
  hidden, constant / zero / gamma=0 rows, negative zeros, binding scale_ub,
  in-place residual updates, every dtype/format/scale-dtype combination,
  determinism, agreement across launch shapes, non-default streams.
The comparison rule is in tests/parity.py.
"""
import json
import os

import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import oracle
import workloads
from gpu_common import DEV, check_fp4, check_fp8, check_whole, run_fp8, say

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
W = workloads.WORKLOADS
FP8_NAMES = [n for n, w in W.items() if not w.fp4]
SMALL_ROWS = {"rmsnorm_fp8_bf16_16x512": 16, "residual_rmsnorm_fp8_bf16_8192x4096": 301,
              "allreduce_residual_rmsnorm_fp8_bf16_8x8192x4096": 97,
              "rmsnorm_fp8_f16_decode_1x8192": 1, "rmsnorm_fp8_f16_decode_8x8192": 8,
              "rmsnorm_fp8_f16_decode_64x8192": 64, "residual_rmsnorm_fp8_bf16_32768x8192": 203,
              "residual_rmsnorm_fp8_f32_32768x8192": 203, "rmsnorm_fp4_bf16_16384x7168": 157,
              "rmsnorm_mxfp4_bf16_16384x7168": 157, "rmsnorm_fp4_swizzled_bf16_16384x7168": 300,
              "residual_rmsnorm_fp4_bf16_16384x7168": 157}


def golden_gs(name):
    entry = json.load(open(os.path.join(HERE, "golden", "fp4_global_scale.json")))["workloads"].get(name)
    return entry["global_scale"] if entry else 1.0


def fp4_gs_for(inp, w=None):
    w = w or inp["workload"]
    amax = oracle.absmax(workloads.bits(inp["x"]), workloads.bits(inp["gamma"]), in_dtype=w.in_dtype, eps=w.eps,
                         weight_offset=w.weight_offset)
    return float(np.float32(448 * 6 / amax))


@pytest.fixture(autouse=True)
def default_shape():
    rq.set_tuning(0, 0, 0)
    yield
    rq.set_tuning(0, 0, 0)


@pytest.mark.parametrize("name", list(SMALL_ROWS))
def test_workload_small_all_elements(name):
    w = W[name]
    inp = workloads.make(name, rows=SMALL_ROWS[name])
    say(f"[small] {name} rows={SMALL_ROWS[name]} shape={rq.query_shape(SMALL_ROWS[name], w.hidden, workloads.TORCH_DTYPES[w.in_dtype], w.fp4, w.residual)}")
    if w.fp4:
        check_fp4(w, inp, fp4_gs_for(inp))
    else:
        check_fp8(w, inp)


@pytest.mark.parametrize("name", list(W))
def test_workload_full_size_every_row(name):
    """Every workload at its full size, every row compared: the boundary
    flips of the whole tensor must be at most 0.01% of its codes."""
    w = W[name]
    say(f"[full] {name} rows={w.rows} hidden={w.hidden} "
        f"shape={rq.query_shape(w.rows, w.hidden, workloads.TORCH_DTYPES[w.in_dtype], w.fp4, w.residual, summed=w.ninputs > 1)}")
    inp = workloads.make(name)
    check_whole(w, inp, golden_gs(name) if w.fp4 else None)


def _rand_inputs(rows, hidden, dt, seed=0, resid=False, gamma=None, scale=1.0):
    rng = np.random.default_rng(seed)
    td = workloads.TORCH_DTYPES[dt]
    x = torch.from_numpy(rng.standard_normal((rows, hidden)) * scale).to(td)
    r = torch.from_numpy(rng.standard_normal((rows, hidden))).to(td) if resid else None
    g = torch.from_numpy(rng.uniform(0.5, 1.5, hidden) if gamma is None else np.broadcast_to(gamma, hidden).copy()).to(td)
    return {"x": x, "residual": r, "gamma": g}


def _wl(op, rows, hidden, dt, **kw):
    return workloads.Workload("custom", op, rows, hidden, dt, 99, eps=kw.pop("eps", 1e-6), **kw)


def test_zero_rows_is_a_noop():
    x = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    out = torch.empty((0, 512), dtype=torch.uint8, device=DEV)
    sc = torch.empty((0,), dtype=torch.float32, device=DEV)
    rq.rmsnorm_fp8(x, g, out=out, scales=sc)
    rq.residual_rmsnorm_fp8(x, x, g, out=out, scales=sc, residual_out=x)
    rq.rmsnorm_fp4(x, g)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt,hiddens", [("bf16", [8, 16, 24, 520, 1576, 4104, 8200]),
                                        ("f16", [8, 136, 2056]),
                                        ("f32", [4, 12, 1028, 4100])])
@pytest.mark.parametrize("rows", [1, 3, 67])
def test_ragged_hidden_and_rows(dt, hiddens, rows):
    for h in hiddens:
        for resid in (False, True):
            op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
            w = _wl(op, rows, h, dt)
            say(f"[ragged] {op} {dt} rows={rows} hidden={h}")
            check_fp8(w, _rand_inputs(rows, h, dt, seed=h + rows, resid=resid), label=f"{op} {dt} {rows}x{h}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("rows,hidden", [(1, 16), (3, 32), (67, 528), (5, 7168 + 16), (129, 1024)])
def test_fp4_ragged(dt, rows, hidden):
    w = _wl("rmsnorm_fp4", rows, hidden, dt)
    inp = _rand_inputs(rows, hidden, dt, seed=rows * hidden)
    say(f"[fp4 ragged] {dt} rows={rows} hidden={hidden}")
    check_fp4(w, inp, fp4_gs_for(inp, w), label=f"fp4 {dt} {rows}x{hidden}")
    check_fp4(w, inp, None, label=f"fp4 {dt} {rows}x{hidden} gs=None")


@pytest.mark.parametrize("dt,hidden", [("bf16", 5120), ("bf16", 6144), ("bf16", 16384), ("f16", 3072),
                                       ("f32", 3072), ("f32", 7168)])
def test_automatic_large_batch_shapes(dt, hidden):
    """Batches above 256 rows of widths whose automatic shapes differ by
    path (4 x 4, 8 x 2, 8 x 4, 12 x 1, 16 x 1 ...), every element checked."""
    rows = 260
    for op in ("rmsnorm_fp8", "residual_rmsnorm_fp8", "rmsnorm_fp4", "residual_rmsnorm_fp4"):
        fp4, resid = op.endswith("fp4"), op.startswith("residual")
        if fp4 and dt == "f32" and hidden > 8192:
            continue
        w = _wl(op, rows, hidden, dt)
        inp = _rand_inputs(rows, hidden, dt, seed=hidden + len(op), resid=resid)
        s = rq.query_shape(rows, hidden, workloads.TORCH_DTYPES[dt], fp4, resid)
        say(f"[large batch] {op} {dt} {rows}x{hidden} shape {s}")
        if fp4:
            check_fp4(w, inp, fp4_gs_for(inp, w), label=f"{op} {dt} {hidden} {s}")
        else:
            check_fp8(w, inp, label=f"{op} {dt} {hidden} {s}")


@pytest.mark.parametrize("dt,hidden", [("bf16", 4096), ("f16", 2560), ("bf16", 5120), ("f16", 6144)])
def test_wave_per_row_fp4_formats(dt, hidden):
    """The one-wavefront-per-row FP4 kernel (16-bit rows of 257..768
    vectors, large batches: 8 or 12 vectors per lane, whole or ragged) in
    every scale format and block size, on 1000 rows: the swizzled layout's
    row map covers 768 rows and leaves a tail of 232."""
    rows = 1000
    s = rq.query_shape(rows, hidden, workloads.TORCH_DTYPES[dt], True, False)
    assert s["waves_per_row"] == 1 and s["rows_per_block"] == 4, s
    inp = _rand_inputs(rows, hidden, dt, seed=hidden + 7)
    for kw in ({}, {"fp4_block": 32}, {"fp4_scale": "ue8m0", "fp4_block": 32}, {"fp4_swizzled": True},
               {"fp4_round_product": True, "weight_offset": 1.0}):
        w = _wl("rmsnorm_fp4", rows, hidden, dt, **kw)
        say(f"[fp4 wave row] {dt} {rows}x{hidden} {kw} shape {s}")
        gs = None if w.fp4_scale == "ue8m0" else fp4_gs_for(inp, w)
        check_fp4(w, inp, gs, label=f"fp4 wave row {dt} {hidden} {kw}")


@pytest.mark.parametrize("dt,hidden", [("bf16", 32768), ("f16", 32768), ("f32", 16384)])
def test_largest_hidden(dt, hidden):
    w = _wl("residual_rmsnorm_fp8", 5, hidden, dt)
    say(f"[max hidden] {dt} {hidden}")
    check_fp8(w, _rand_inputs(5, hidden, dt, seed=3, resid=True), label=f"max {dt} {hidden}")
    if dt != "f32":
        w4 = _wl("rmsnorm_fp4", 5, hidden, dt)
        inp = _rand_inputs(5, hidden, dt, seed=4)
        check_fp4(w4, inp, fp4_gs_for(inp, w4), label=f"fp4 max {dt} {hidden}")


def test_special_rows():
    h = 1024
    rows = []
    rows.append(np.full(h, 3.0))                      # constant row
    rows.append(np.zeros(h))                          # zero row (eps > 0): scale 0
    neg0 = np.zeros(h); neg0[::2] = -0.0              # negative zeros
    rows.append(neg0)
    big = np.random.default_rng(1).standard_normal(h) * 1e4
    rows.append(big)                                  # large values
    tiny = np.random.default_rng(2).standard_normal(h) * 1e-3
    rows.append(tiny)                                 # eps comparable to mean(x^2)
    onehot = np.zeros(h); onehot[17] = -5.0
    rows.append(onehot)
    # zeros of both signs among nonzero values (a nonzero scale), every
    # fourth gamma zero and some gammas negative below: zero products of
    # both signs, whose codes keep the product's sign bit
    mixed = np.random.default_rng(4).standard_normal(h)
    mixed[1::5] = 0.0
    mixed[3::5] = -0.0
    rows.append(mixed)
    rows.append(-mixed)
    x = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    gmix = np.random.default_rng(3).uniform(0.5, 1.5, h)
    gmix[::4] = 0.0
    gmix[2::7] *= -1.0
    for dt in ("bf16", "f16", "f32"):
        inp = {"x": x.to(workloads.TORCH_DTYPES[dt]), "residual": None,
               "gamma": torch.from_numpy(np.random.default_rng(3).uniform(0.5, 1.5, h)).to(workloads.TORCH_DTYPES[dt])}
        for fmt in ("e4m3fn", "e4m3fnuz"):
            w = _wl("rmsnorm_fp8", len(rows), h, dt, out_fmt=fmt)
            say(f"[special] {dt} {fmt}")
            check_fp8(w, inp, label=f"special {dt} {fmt}")
        inpm = dict(inp, gamma=torch.from_numpy(gmix).to(workloads.TORCH_DTYPES[dt]))
        for off in (0.0, 0.5):
            w = _wl("rmsnorm_fp8", len(rows), h, dt, weight_offset=off)
            say(f"[special] {dt} zero products, weight_offset {off}")
            check_fp8(w, inpm, label=f"special {dt} zero products off={off}")
        inp0 = dict(inp, gamma=torch.zeros(h, dtype=workloads.TORCH_DTYPES[dt]))
        check_fp8(_wl("rmsnorm_fp8", len(rows), h, dt), inp0, label=f"gamma=0 {dt}")
        w4 = _wl("rmsnorm_fp4", len(rows), h, "bf16")
        if dt == "bf16":
            check_fp4(w4, inpm, 1.0, label="fp4 zero products")
            check_fp4(w4, inp, 1.0, label="fp4 special gs=1")
            check_fp4(w4, inp0, 1.0, label="fp4 gamma=0")


@pytest.mark.parametrize("ub", [1e-3, 1e-2, 0.05])
def test_scale_ub_binds(ub):
    w = _wl("residual_rmsnorm_fp8", 33, 2048, "bf16", scale_ub=ub)
    inp = _rand_inputs(33, 2048, "bf16", seed=11, resid=True)
    say(f"[ub] {ub}")
    check_fp8(w, inp, label=f"ub={ub}")
    c, s, _ = run_fp8(w, inp)
    if ub <= 1e-3:  # below every row's natural scale: the bound binds everywhere
        assert np.all(s == np.float32(ub))


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_dtype_format_scale_matrix(dt, fmt, sdt):
    for resid in (False, True):
        op = "residual_rmsnorm_fp8" if resid else "rmsnorm_fp8"
        w = _wl(op, 70, 2048, dt, out_fmt=fmt, scales_dtype=sdt, weight_offset=0.5)
        say(f"[matrix] {op} {dt} {fmt} {sdt}")
        check_fp8(w, _rand_inputs(70, 2048, dt, seed=5, resid=resid), label=f"{op} {dt} {fmt} {sdt}")


@pytest.mark.parametrize("where", ["x", "residual"])
def test_in_place_residual(where):
    w = W["residual_rmsnorm_fp8_bf16_8192x4096"]
    inp = workloads.make(w.name, rows=130)
    say(f"[in place] residual_out = {where}")
    check_fp8(w, inp, in_place=where, label=f"in place over {where}")


def test_deterministic_and_shape_independent():
    w = W["residual_rmsnorm_fp8_bf16_8192x4096"]
    inp = workloads.make(w.name, rows=257)
    base = run_fp8(w, inp)
    again = run_fp8(w, inp)
    assert all(np.array_equal(a, b) for a, b in zip(base[:2], again[:2]))
    for waves in (1, 2, 4, 8, 16):
        for vpt in (1, 2, 4):
            if waves * 64 * vpt * 8 < w.hidden:
                continue
            for blocks in (0, 7):
                rq.set_tuning(waves, vpt, blocks)
                say(f"[shape] waves={waves} vpt={vpt} max_blocks={blocks}")
                rep = check_fp8(w, inp, label=f"shape {waves}x{vpt}/{blocks}")
                c, s, ro = run_fp8(w, inp)
                assert np.array_equal(ro, base[2])
                # codes may differ from the default shape only at rounding boundaries
                assert (c != base[0]).mean() <= 1e-4
    rq.set_tuning(0, 0, 0)


def test_fp4_shapes_and_offset():
    w = W["rmsnorm_fp4_bf16_16384x7168"]
    inp = workloads.make(w.name, rows=90)
    gs = fp4_gs_for(inp)
    for waves, vpt in ((4, 4), (8, 2), (8, 4), (16, 1), (16, 2)):
        if waves * 64 * vpt * 8 < w.hidden:
            continue
        rq.set_tuning(waves, vpt, 5)
        say(f"[fp4 shape] waves={waves} vpt={vpt}")
        check_fp4(w, inp, gs, label=f"fp4 shape {waves}x{vpt}")
    rq.set_tuning(0, 0, 0)
    check_fp4(w, inp, gs, weight_offset=0.25, label="fp4 weight_offset=0.25")


def test_non_default_stream_and_3d_input():
    w = W["rmsnorm_fp8_bf16_16x512"]
    inp = workloads.make(w.name)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rep = check_fp8(w, inp, stream=s, label="side stream")
    x3 = inp["x"].reshape(4, 4, 512).to(DEV)
    g = inp["gamma"].to(DEV)
    c3, s3 = rq.rmsnorm_fp8(x3, g, eps=w.eps, scale_ub=w.scale_ub)
    c2, s2 = rq.rmsnorm_fp8(x3.reshape(16, 512), g, eps=w.eps, scale_ub=w.scale_ub)
    torch.cuda.synchronize()
    assert c3.shape == (4, 4, 512) and s3.shape == (4, 4)
    assert torch.equal(c3.reshape(16, 512), c2) and torch.equal(s3.reshape(16), s2)
