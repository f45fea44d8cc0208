"""Pins for the oracle's block-size / scale-format generalization of the FP4
path and for the swizzled scale layout.

Sources: FlashInfer rmsnorm_fp4quant.py -- section "UE8M0 Intrinsics (for
MXFP4)" (code = ceil(log2 v) + 127 clamped to [0, 255], 0 for v <= 0; element
factor 2^(127 - code), 0 for code 0), the kernel's Phase 3 (scale from the
block amax / 6; E4M3 scales use the global scale, UE8M0 scales do not), the
constructor (block_size 16 or 32, scale_format e4m3 or ue8m0) and the
swizzled scale store / API docstring (128 x 4 tiles).

What pins what:
  * UE8M0 encoding against its definition by exhaustive search (the smallest
    code whose power of two is >= v), on every power of two of the range,
    its fp64 neighbours and random values; decoding in closed form.
  * Hand-worked rows (tests/golden/hand_rows.json, fp4_block_rows) for
    32-element UE8M0 and E4M3 blocks, 16-element UE8M0 blocks, a block whose
    scale underflows to code 0 and one whose amax/6 lies in (2^-128, 2^-127]
    (code 0 by the ceil rule itself, factor 0 by the zero check).
  * Block-size consistency: a 32-element E4M3 block scale is the larger of
    its two 16-element halves' scales (before rounding).
  * UE8M0 invariants on random rows: the scale is the smallest power of two
    >= amax/6, no element saturates, every code is within half a step.
  * The swizzled offsets worked by hand, and equal to the 5-axis tile view
    [m_tile][k_tile][outer_m][inner_m][inner_k] of the padded row-major matrix
    (the docstring's description), which is a bijection onto the non-padding
    positions.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")))
TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def as_bits(vals, dt):
    return workloads.bits(torch.tensor(vals, dtype=torch.float64).to(TD[dt]))


def hexes(a):
    return [f"0x{int(v):02X}" for v in a]


# ---- UE8M0 ------------------------------------------------------------------

def ue8m0_by_search(v: float) -> int:
    """Smallest code c in [0, 255] with 2^(c - 127) >= v; 0 for v <= 0."""
    if not v > 0:
        return 0
    for c in range(256):
        if 2.0 ** (c - 127) >= v:
            return c
    return 255


def test_ue8m0_encode_matches_search():
    vals = [0.0, -1.0, -0.0, float("inf")]
    for k in range(-170, 140):
        p = 2.0 ** k
        vals += [p, np.nextafter(p, 0.0), np.nextafter(p, np.inf), 1.5 * p, 0.75 * p]
    rng = np.random.default_rng(5)
    vals += list(np.exp2(rng.uniform(-160, 130, 4000)))
    vals = np.array(vals, np.float64)
    got = oracle.encode("ue8m0", vals)
    want = np.array([ue8m0_by_search(float(v)) for v in vals])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(vals[i], got[i], want[i]) for i in bad[:5]]


def test_ue8m0_decode_closed_form():
    c = np.arange(256)
    assert np.array_equal(oracle.decode("ue8m0", c), np.ldexp(1.0, c - 127))
    assert oracle.decode("ue8m0", [127])[0] == 1.0


@pytest.mark.parametrize("row", GOLDEN["fp4_block_rows"], ids=lambda r: r["id"])
def test_fp4_block_hand_rows(row):
    dt = row["in_dtype"]
    n = len(row["x"])
    r = oracle.rmsnorm_fp4(as_bits([row["x"]], dt), as_bits([1.0] * n, dt), in_dtype=dt, eps=row["eps"],
                           weight_offset=row["weight_offset"], global_scale=row["global_scale"],
                           block_size=row["block_size"], scale_format=row["scale_format"])
    assert hexes(r["block_scales"][0]) == row["expect_block_scales"]
    assert hexes(r["packed"][0]) == row["expect_packed"]


def test_default_is_16_element_e4m3():
    rng = np.random.default_rng(8)
    x = as_bits(rng.standard_normal((6, 256)).tolist(), "bf16")
    g = as_bits(rng.uniform(0.5, 1.5, 256).tolist(), "bf16")
    a = oracle.rmsnorm_fp4(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=300.0)
    b = oracle.rmsnorm_fp4(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=300.0,
                           block_size=16, scale_format="e4m3")
    for k in ("packed", "block_scales"):
        assert np.array_equal(a[k], b[k])


def test_32_element_e4m3_scale_is_max_of_halves():
    rng = np.random.default_rng(9)
    x = as_bits(rng.standard_normal((8, 512)).tolist(), "bf16")
    g = as_bits(rng.uniform(0.5, 1.5, 512).tolist(), "bf16")
    kw = dict(in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=500.0)
    r16 = oracle.rmsnorm_fp4(x, g, block_size=16, **kw)
    r32 = oracle.rmsnorm_fp4(x, g, block_size=32, **kw)
    halves = r16["sf"].reshape(8, -1, 2).max(axis=2)
    assert np.array_equal(r32["sf"], halves)


@pytest.mark.parametrize("block", [16, 32])
def test_ue8m0_invariants_random_rows(block):
    rng = np.random.default_rng(10 + block)
    rows, h = 16, 1024
    xs = rng.standard_normal((rows, h)) * np.exp2(rng.integers(-20, 20, (rows, 1)))
    x = as_bits(xs.tolist(), "bf16")
    g = as_bits(rng.uniform(0.5, 1.5, h).tolist(), "bf16")
    r = oracle.rmsnorm_fp4(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=123.0,
                           block_size=block, scale_format="ue8m0")
    y = oracle.rmsnorm_y(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0)["y"]
    amax = np.abs(y).reshape(rows, -1, block).max(axis=2)
    v = (amax / 6).astype(np.float32).astype(np.float64)
    S = r["block_scales"].astype(np.int64)
    # the smallest power of two >= v (no clamp binds for these magnitudes)
    assert np.all(np.ldexp(1.0, S - 127) >= v)
    assert np.all(np.ldexp(1.0, S - 128) < v)
    # q = y * 2^(127 - S) never exceeds 6 in magnitude (no saturation)
    assert np.abs(r["q"]).max() <= 6.0 * (1 + 2 ** -23)
    # every code is within half a code step of q
    codes = np.stack([r["packed"] & 0xF, r["packed"] >> 4], axis=-1).reshape(rows, h)
    dec = oracle.decode("e2m1", codes)
    mags = oracle.decode("e2m1", np.arange(8))
    steps = np.diff(mags)
    a = np.abs(r["q"])
    idx = np.clip(np.searchsorted(mags, a) - 1, 0, 6)
    assert np.all(np.abs(dec - r["q"]) <= steps[idx] / 2 * (1 + 1e-6))
    # the global scale plays no part
    r2 = oracle.rmsnorm_fp4(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=1.0,
                            block_size=block, scale_format="ue8m0")
    assert np.array_equal(r["packed"], r2["packed"]) and np.array_equal(r["block_scales"], r2["block_scales"])


def test_bad_block_or_format_is_rejected():
    x = as_bits([[1.0] * 48], "bf16")
    g = as_bits([1.0] * 48, "bf16")
    with pytest.raises(ValueError):
        oracle.rmsnorm_fp4(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=1.0, block_size=32)
    with pytest.raises(ValueError):
        oracle.rmsnorm_fp4(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=1.0, block_size=8)
    with pytest.raises(ValueError):
        oracle.rmsnorm_fp4(x, g, in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=1.0,
                           scale_format="e8m0")


# ---- swizzled layout ----------------------------------------------------------

def test_swizzle_hand_offsets():
    s = GOLDEN["swizzle_offsets"]
    assert oracle.swizzled_size(s["rows"], s["sf_per_row"]) == s["size"]
    for row, sf, off in s["cases"]:
        assert int(oracle.swizzled_offset(row, sf, s["sf_per_row"])) == off, (row, sf)


@pytest.mark.parametrize("rows,nsf", [(1, 1), (128, 4), (130, 5), (257, 448), (300, 14), (64, 7)])
def test_swizzle_is_the_tile_view_and_a_bijection(rows, nsf):
    rng = np.random.default_rng(rows * 1000 + nsf)
    m = rng.integers(0, 255, (rows, nsf), dtype=np.uint8)
    got = oracle.swizzle_scales(m, fill=255)
    # the docstring's tile view: pad to [Mt*128, Kt*4], split rows into
    # (m_tile, inner_m, outer_m) and columns into (k_tile, inner_k), then
    # order the axes as [m_tile][k_tile][outer_m][inner_m][inner_k]
    mt, kt = -(-rows // 128), -(-nsf // 4)
    pad = np.full((mt * 128, kt * 4), 255, np.uint8)
    pad[:rows, :nsf] = m
    view = pad.reshape(mt, 4, 32, kt, 4).transpose(0, 3, 2, 1, 4).reshape(-1)
    assert np.array_equal(got, view)
    r, c = np.meshgrid(np.arange(rows), np.arange(nsf), indexing="ij")
    offs = oracle.swizzled_offset(r, c, nsf).reshape(-1)
    assert len(np.unique(offs)) == offs.size and offs.min() >= 0 and offs.max() < got.size


# ---- residual input and fp32 input (the FP4 quantizer on the residual page's
# pre-norm sum; the quantizer itself is unchanged) --------------------------------

def test_fp4_residual_hand_row():
    """x + r reproduces the mx32 hand row exactly: r = 0.5 everywhere and
    x = row - 0.5 (all exact in bf16), so residual_out holds the row's bf16
    bits and the codes equal the hand row's."""
    base = next(r for r in GOLDEN["fp4_block_rows"] if r["id"] == "mx32_ue8m0")
    n = len(base["x"])
    x = [v - 0.5 for v in base["x"]]
    r = oracle.rmsnorm_fp4(as_bits([x], "bf16"), as_bits([1.0] * n, "bf16"), in_dtype="bf16", eps=0.0,
                           weight_offset=0.0, global_scale=1.0, block_size=32, scale_format="ue8m0",
                           residual=as_bits([[0.5] * n], "bf16"))
    # bf16 bits: 4 = 0x4080, 2 = 0x4000, -2 = 0xC000, 3 = 0x4040, -3 = 0xC040, 1 = 0x3F80, 0 = 0
    want = [0x4080, 0x4000, 0xC000, 0x4000, 0xC000] + [0] * 27 + [0x4040, 0x4040, 0xC040] + [0x3F80] * 5 + [0] * 24
    assert [int(v) for v in r["residual_out"][0]] == want
    assert hexes(r["block_scales"][0]) == base["expect_block_scales"]
    assert hexes(r["packed"][0]) == base["expect_packed"]


@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "ue8m0"), (32, "e4m3"), (16, "ue8m0")])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_fp4_residual_is_fp4_of_the_stored_sum(dt, block, fmt):
    rng = np.random.default_rng(30 + block)
    rows, h = 12, 512
    x = as_bits(rng.standard_normal((rows, h)).tolist(), dt)
    res = as_bits(rng.standard_normal((rows, h)).tolist(), dt)
    g = as_bits(rng.uniform(0.5, 1.5, h).tolist(), dt)
    kw = dict(in_dtype=dt, eps=1e-6, weight_offset=0.0, global_scale=250.0, block_size=block, scale_format=fmt)
    a = oracle.rmsnorm_fp4(x, g, residual=res, **kw)
    # the stored sum is torch's correctly rounded (fp32 holds the exact sum of two 16-bit values)
    tx = workloads.from_bits(x, dt).to(torch.float64)
    tr = workloads.from_bits(res, dt).to(torch.float64)
    assert np.array_equal(a["residual_out"], workloads.bits((tx + tr).to(TD[dt])))
    b = oracle.rmsnorm_fp4(a["residual_out"], g, **kw)
    for k in ("packed", "block_scales"):
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "ue8m0")])
def test_fp4_fp32_input_of_bf16_values_matches_bf16(block, fmt):
    """Widening bf16 values to fp32 changes no value, so no code."""
    rng = np.random.default_rng(40 + block)
    xb = torch.from_numpy(rng.standard_normal((9, 768))).to(torch.bfloat16)
    gb = torch.from_numpy(rng.uniform(0.5, 1.5, 768)).to(torch.bfloat16)
    kw = dict(eps=1e-6, weight_offset=0.0, global_scale=77.0, block_size=block, scale_format=fmt)
    a = oracle.rmsnorm_fp4(workloads.bits(xb), workloads.bits(gb), in_dtype="bf16", **kw)
    b = oracle.rmsnorm_fp4(workloads.bits(xb.float()), workloads.bits(gb.float()), in_dtype="f32", **kw)
    for k in ("packed", "block_scales"):
        assert np.array_equal(a[k], b[k])


# ---- the FP4 page's numerics (16-bit x * w), optional ------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("row", GOLDEN["fp4_compat_rows"], ids=lambda r: r["id"])
def test_fp4_compat_hand_row(row, dt):
    x, g = as_bits([row["x"]], dt), as_bits(row["gamma"], dt)
    kw = dict(in_dtype=dt, eps=row["eps"], weight_offset=0.0, global_scale=row["global_scale"],
              block_size=row["block_size"], scale_format=row["scale_format"])
    exact = oracle.rmsnorm_fp4(x, g, **kw)
    compat = oracle.rmsnorm_fp4(x, g, round_product=True, **kw)
    assert hexes(exact["block_scales"][0]) == row["expect_block_scales"]
    assert hexes(compat["block_scales"][0]) == row["expect_block_scales"]
    assert hexes(exact["packed"][0]) == row["expect_packed_exact"]
    assert hexes(compat["packed"][0]) == row["expect_packed_compat"]


@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "ue8m0")])
def test_fp4_compat_equals_exact_when_products_are_exact(block, fmt):
    """With gamma a power of two every bf16 product x * gamma is a bf16 value,
    so rounding it changes nothing."""
    rng = np.random.default_rng(50 + block)
    x = as_bits(rng.standard_normal((10, 640)).tolist(), "bf16")
    g = as_bits(np.exp2(rng.integers(-3, 4, 640)).tolist(), "bf16")
    kw = dict(in_dtype="bf16", eps=1e-6, weight_offset=0.0, global_scale=150.0, block_size=block, scale_format=fmt)
    a = oracle.rmsnorm_fp4(x, g, **kw)
    b = oracle.rmsnorm_fp4(x, g, round_product=True, **kw)
    for k in ("packed", "block_scales", "q"):
        assert np.array_equal(a[k], b[k])


def test_fp4_compat_y_is_rounded_product_times_rstd():
    rng = np.random.default_rng(60)
    xs, gs = rng.standard_normal((6, 256)), rng.uniform(0.5, 1.5, 256)
    x, g = as_bits(xs.tolist(), "bf16"), as_bits(gs.tolist(), "bf16")
    kw = dict(in_dtype="bf16", eps=1e-6, weight_offset=0.0)
    plain = oracle.rmsnorm_y(x, g, **kw)
    comp = oracle.rmsnorm_y(x, g, round_product=True, **kw)
    xv = workloads.from_bits(x, "bf16").to(torch.float64)
    gv = workloads.from_bits(g, "bf16").to(torch.float64)
    prod = (xv * gv).to(torch.bfloat16).to(torch.float64).numpy()  # torch: one RNE rounding
    assert np.array_equal(comp["rstd"], plain["rstd"])
    assert np.array_equal(comp["y"], prod * comp["rstd"][:, None])
