"""GPU parity of rmsnorm_fp4quant and residual_rmsnorm_fp4quant (through the
C ABI) against the oracle for every block size (16, 32), scale format (E4M3,
UE8M0) and scale layout (row-major, swizzled 128 x 4 tiles), on bf16, fp16
and fp32 inputs (fp32 puts a 16-element block on 4 lanes and a 32-element
block on 8):

* row counts that leave a ragged last 128-row tile and hidden sizes whose
  scale columns leave a ragged last 4-column tile (swizzled padding must keep
  its bytes);
* the hand-worked rows of tests/golden/hand_rows.json (fp4_block_rows),
  byte for byte;
* forced launch shapes (1-16 waves per row, 1-4 vectors per lane), so the
  2-, 4- and 8-lane block reductions run in every mapping;
* residual_out bit-exact, including in-place updates over x or residual;
* the 16-element E4M3 row-major case equals rmsnorm_fp4 bit for bit.
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
from gpu_common import DEV, check_fp4, say

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "hand_rows.json")))
TD = workloads.TORCH_DTYPES


@pytest.fixture(autouse=True)
def default_shape():
    rq.set_tuning(0, 0, 0)
    yield
    rq.set_tuning(0, 0, 0)


def _inputs(rows, hidden, dt, seed, resid=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, hidden))
    heavy = rng.choice(hidden, size=max(1, hidden // 100), replace=False)
    x[:, heavy] = rng.standard_t(3.0, size=(rows, heavy.size))
    mag = np.exp2(rng.integers(-8, 8, (rows, 1)))  # rows of different magnitude
    r = torch.from_numpy(rng.standard_normal((rows, hidden)) * mag).to(TD[dt]) if resid else None
    return {"x": torch.from_numpy(x * mag).to(TD[dt]), "residual": r,
            "gamma": torch.from_numpy(rng.uniform(0.8, 1.2, hidden)).to(TD[dt])}


def _wl(rows, hidden, dt, block, fmt, swz, offset=0.0, resid=False, round_product=False):
    op = "residual_rmsnorm_fp4" if resid else "rmsnorm_fp4"
    return workloads.Workload("fp4quant", op, rows, hidden, dt, 98, eps=1e-6, weight_offset=offset,
                              fp4_block=block, fp4_scale=fmt, fp4_swizzled=swz, fp4_round_product=round_product)


def _gs(inp, w):
    amax = oracle.absmax(workloads.bits(inp["x"]), workloads.bits(inp["gamma"]), in_dtype=w.in_dtype, eps=w.eps,
                         weight_offset=w.weight_offset)
    return float(np.float32(448 * 6 / amax))


@pytest.mark.parametrize("swz", [False, True], ids=["rowmajor", "swizzled"])
@pytest.mark.parametrize("fmt", ["e4m3", "ue8m0"])
@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_every_variant(dt, block, fmt, swz):
    # 256 x 3072: a whole number of 256-row runs of the swizzled row map
    for rows, hidden in ((300, 160), (131, 7168), (257, 2080), (256, 3072)):
        w = _wl(rows, hidden, dt, block, fmt, swz)
        inp = _inputs(rows, hidden, dt, seed=rows + hidden + block)
        say(f"[fp4quant] {dt} block={block} {fmt} swizzled={swz} rows={rows} hidden={hidden}")
        check_fp4(w, inp, _gs(inp, w), label=f"{dt} {block} {fmt} swz={swz} {rows}x{hidden}")


@pytest.mark.parametrize("fmt", ["e4m3", "ue8m0"])
def test_swizzled_tile_slots_widest_row(fmt):
    # the widest bf16 row with 16-element blocks: 2048 scale columns per row
    rows, hidden = 256, 32768
    w = _wl(rows, hidden, "bf16", 16, fmt, True)
    inp = _inputs(rows, hidden, "bf16", seed=11)
    say(f"[fp4quant widest swizzled] {fmt} rows={rows} hidden={hidden}")
    check_fp4(w, inp, _gs(inp, w), label=f"widest swizzled {fmt}")


# Swizzled scales over many 256-row runs of the row map that keeps each
# 32-row group (the rows whose scales share 128-byte lines) on one XCD:
# ragged last 128-row tiles (partial and empty groups), ragged 4-column tiles,
# each input type, the residual variant, and forced shapes and grids.
MANY_RUNS = [  # dt, block, fmt, rows, hidden, resid, (waves, vpt, blocks)
    ("bf16", 16, "e4m3", 8229, 112, False, (0, 0, 0)),     # 7 scale columns, 37-row last tile
    ("bf16", 16, "e4m3", 8192, 7168, False, (0, 0, 0)),    # the 16384 x 7168 workload's row
    ("f16", 32, "ue8m0", 8292, 1056, True, (0, 0, 0)),     # 33 columns, residual, 100-row last tile
    ("f32", 16, "e4m3", 8200, 256, False, (0, 0, 0)),      # 8-row last tile: 3 empty groups
    ("bf16", 32, "e4m3", 8229, 2048, False, (1, 4, 0)),    # one wave per row
    ("bf16", 16, "ue8m0", 8229, 2048, True, (4, 1, 7)),    # 7 blocks: not a multiple of 8
    ("f16", 16, "e4m3", 8300, 4096, False, (16, 1, 0)),    # 16 waves per row: one row per block
]


@pytest.mark.parametrize("case", MANY_RUNS, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}-{c[3]}x{c[4]}-r{int(c[5])}-{c[6]}")
def test_swizzled_many_row_runs(case):
    dt, block, fmt, rows, hidden, resid, tune = case
    w = _wl(rows, hidden, dt, block, fmt, True, resid=resid)
    inp = _inputs(rows, hidden, dt, seed=rows + hidden, resid=resid)
    rq.set_tuning(*tune)
    say(f"[fp4quant swizzled row runs] {case}")
    check_fp4(w, inp, _gs(inp, w), label=f"swizzled row runs {case}")


@pytest.mark.parametrize("row", GOLDEN["fp4_block_rows"], ids=lambda r: r["id"])
def test_hand_rows_byte_exact(row):
    dt = row["in_dtype"]
    if dt == "f32":
        dt = "bf16"  # every value of these rows is exact in bf16 (powers of two times 1, 3)
    n = len(row["x"])
    x = torch.tensor([row["x"]], dtype=torch.float64).to(TD[dt]).to(DEV)
    g = torch.ones(n, dtype=TD[dt], device=DEV)
    gst = torch.tensor([row["global_scale"]], dtype=torch.float32, device=DEV)
    say(f"[fp4quant hand row] {row['id']}")
    for swz in (False, True):
        packed, bs = rq.rmsnorm_fp4quant(x, g, eps=row["eps"], weight_offset=row["weight_offset"], global_scale=gst,
                                         block_size=row["block_size"], scale_format=row["scale_format"],
                                         swizzled=swz)
        torch.cuda.synchronize()
        got_p = [f"0x{v:02X}" for v in packed.cpu().numpy()[0]]
        b = bs.cpu().numpy()
        if swz:
            b = b[oracle.swizzled_offset(0, np.arange(n // row["block_size"]), n // row["block_size"])]
        got_s = [f"0x{v:02X}" for v in np.ravel(b)[: n // row["block_size"]]]
        assert got_s == row["expect_block_scales"]
        assert got_p == row["expect_packed"]


@pytest.mark.parametrize("fmt", ["e4m3", "ue8m0"])
def test_forced_launch_shapes_block32(fmt):
    hidden = 4096  # 512 vectors
    inp = _inputs(70, hidden, "bf16", seed=3)
    w = _wl(70, hidden, "bf16", 32, fmt, False)
    gs = _gs(inp, w)
    for waves, vpt in ((1, 4), (2, 4), (2, 2), (4, 2), (8, 1), (3, 4), (16, 1), (12, 1), (5, 2)):
        if waves * 64 * vpt * 8 < hidden:
            continue
        rq.set_tuning(waves, vpt, 7)
        say(f"[fp4quant shape] {fmt} waves={waves} vpt={vpt}")
        check_fp4(w, inp, gs, label=f"block32 {fmt} {waves}x{vpt}")
    rq.set_tuning(0, 0, 0)


@pytest.mark.parametrize("swz", [False, True], ids=["rowmajor", "swizzled"])
@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "ue8m0"), (32, "e4m3"), (16, "ue8m0")])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_residual_variants(dt, block, fmt, swz):
    for rows, hidden in ((300, 160), (131, 7168), (512, 3072)):
        w = _wl(rows, hidden, dt, block, fmt, swz, resid=True)
        inp = _inputs(rows, hidden, dt, seed=rows + hidden + block + 1, resid=True)
        say(f"[fp4quant residual] {dt} block={block} {fmt} swizzled={swz} rows={rows} hidden={hidden}")
        check_fp4(w, inp, _gs(inp, w), label=f"residual {dt} {block} {fmt} swz={swz} {rows}x{hidden}")


@pytest.mark.parametrize("where", ["x", "residual"])
def test_residual_in_place(where):
    rows, hidden = 77, 2048
    inp = _inputs(rows, hidden, "bf16", seed=5, resid=True)
    x, r, g = inp["x"].to(DEV), inp["residual"].to(DEV), inp["gamma"].to(DEV)
    want_p, want_s, want_ro = rq.residual_rmsnorm_fp4quant(x.clone(), r.clone(), g, block_size=32)
    target = x if where == "x" else r
    p, sc, ro = rq.residual_rmsnorm_fp4quant(x, r, g, block_size=32, residual_out=target)
    torch.cuda.synchronize()
    say(f"[fp4quant in place] residual_out over {where}")
    assert ro.data_ptr() == target.data_ptr()
    assert torch.equal(ro, want_ro) and torch.equal(p, want_p) and torch.equal(sc, want_s)


@pytest.mark.parametrize("resid", [False, True])
@pytest.mark.parametrize("block", [16, 32])
def test_forced_launch_shapes_f32(block, resid):
    hidden = 2048  # 512 fp32 vectors
    inp = _inputs(70, hidden, "f32", seed=13, resid=resid)
    w = _wl(70, hidden, "f32", block, "ue8m0" if block == 32 else "e4m3", False, resid=resid)
    gs = _gs(inp, w)
    for waves, vpt in ((1, 4), (2, 4), (2, 2), (4, 2), (8, 1), (3, 4), (16, 1), (12, 1)):
        if waves * 64 * vpt * 4 < hidden:
            continue
        rq.set_tuning(waves, vpt, 7)
        say(f"[fp4quant f32 shape] block={block} resid={resid} waves={waves} vpt={vpt}")
        check_fp4(w, inp, gs, label=f"f32 block{block} resid={resid} {waves}x{vpt}")
    rq.set_tuning(0, 0, 0)


@pytest.mark.parametrize("resid", [False, True])
@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "ue8m0")])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_round_product_mode(dt, block, fmt, resid):
    """The page's numerics (x * w rounded to the input type) against the
    oracle's same mode."""
    for rows, hidden in ((150, 2080), (64, 7168)):
        w = _wl(rows, hidden, dt, block, fmt, False, resid=resid, round_product=True)
        inp = _inputs(rows, hidden, dt, seed=rows + block + 7, resid=resid)
        say(f"[fp4quant round_product] {dt} block={block} {fmt} resid={resid} {rows}x{hidden}")
        check_fp4(w, inp, _gs(inp, w), label=f"round_product {dt} {block} {fmt} resid={resid}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("row", GOLDEN["fp4_compat_rows"], ids=lambda r: r["id"])
def test_round_product_hand_row(row, dt):
    n = len(row["x"])
    x = torch.tensor([row["x"]], dtype=torch.float64).to(TD[dt]).to(DEV)
    g = torch.tensor(row["gamma"], dtype=torch.float64).to(TD[dt]).to(DEV)
    say(f"[fp4quant round_product hand row] {row['id']} {dt}")
    for rp, key in ((False, "expect_packed_exact"), (True, "expect_packed_compat")):
        packed, bs = rq.rmsnorm_fp4quant(x, g, eps=row["eps"], block_size=row["block_size"],
                                         scale_format=row["scale_format"], round_product=rp)
        torch.cuda.synchronize()
        assert [f"0x{v:02X}" for v in bs.cpu().numpy()[0]] == row["expect_block_scales"]
        assert [f"0x{v:02X}" for v in packed.cpu().numpy()[0]] == row[key], (rp, key)


def test_weight_offset_and_f16_block32():
    inp = _inputs(90, 7168, "f16", seed=11)
    w = _wl(90, 7168, "f16", 32, "ue8m0", True, offset=0.25)
    check_fp4(w, inp, 1.0, label="f16 block32 ue8m0 swizzled offset 0.25")


def test_default_variant_equals_rmsnorm_fp4():
    inp = _inputs(200, 7168, "bf16", seed=12)
    x, g = inp["x"].to(DEV), inp["gamma"].to(DEV)
    gst = torch.tensor([37.5], dtype=torch.float32, device=DEV)
    p1, s1 = rq.rmsnorm_fp4(x, g, global_scale=gst)
    p2, s2 = rq.rmsnorm_fp4quant(x, g, global_scale=gst, block_size=16, scale_format="e4m3")
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(s1, s2)
