"""Pins for the oracle's row pipeline: hand-worked rows, closed forms and invariants.

The hand rows (tests/golden/hand_rows.json) were derived by hand from the
definitions; scale closed forms are evaluated here at 60 decimal digits.
Invariants follow from the definitions alone:
  * FP8 codes equal ENC(FMAX * s*g' / max|s*g'|) when scale_ub does not bind
    (rstd and eps cancel), so they are independent of rstd.
  * Scaling a row by 2^k leaves the FP8 codes unchanged.
  * (gamma, weight_offset) is the same as (gamma + weight_offset, 0).
  * The residual output is torch's (x.float() + r.float()).to(dtype)
    (a correctly rounded sum: fp32 holds at least 2p+2 bits of a bf16/fp16 sum).
  * The fused residual path equals the plain path run on residual_out.
  * Dequantization error is at most half a code step (unsaturated codes).
Sources: Mojo docs rms_norm_fused_fp8 (Args) and allreduce_residual_rmsnorm_fp8
(Args: residual, residual_output, weight_offset); FlashInfer rmsnorm_fp4quant.py
(Constants, FP8 E4M3 Intrinsics, E2M1 Conversion, kernel Phase 2 / Phase 3).
"""
import json
import math
import os
from decimal import Decimal as D, getcontext

import numpy as np
import pytest
import torch

import oracle
import workloads

getcontext().prec = 60
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")))
TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def as_bits(vals, dt):
    return workloads.bits(torch.tensor(vals, dtype=torch.float64).to(TD[dt]))


def hexes(a):
    return [f"0x{int(v):02X}" for v in a]


def eval_closed_form(expr, row):
    env = {"D": D, "sqrt": lambda d: D(d).sqrt(), "EPS": D(float(np.float32(row["eps"]))),
           "F32_UB": float(np.float32(row["scale_ub"]))}
    return eval(expr, {"__builtins__": {}}, env)


@pytest.mark.parametrize("row", GOLDEN["fp8_rows"], ids=lambda r: r["id"])
def test_fp8_hand_rows(row):
    dt = row["in_dtype"]
    r = oracle.rmsnorm_fp8(as_bits([row["x"]], dt), as_bits(row["gamma"], dt), in_dtype=dt, eps=row["eps"],
                           weight_offset=row["weight_offset"], scale_ub=row["scale_ub"], out_fmt=row["out_fmt"],
                           scales_dtype=row["scales_dtype"])
    assert hexes(r["codes"][0]) == row["expect_codes"]
    if "expect_q" in row:
        q_exact = np.array(row["expect_q"], np.float64)
        # the stored fp32 scale carries one rounding: q within 2^-23 relative of exact
        assert np.allclose(r["q"][0], q_exact, rtol=2.0**-23, atol=0)
    if "expect_scale" in row:
        exact = eval_closed_form(row["expect_scale"], row)
        got = D(float(r["scales"][0]))
        # stored fp32 scale = exact scale rounded once to fp32
        assert abs(got - exact) <= abs(exact) * D(2.0**-24), (got, exact)
        assert r["scales"][0] == np.float32(float(exact))
    if "expect_scale_bits" in row:
        assert f"0x{int(r['scales'][0]):04X}" == row["expect_scale_bits"]


@pytest.mark.parametrize("row", GOLDEN["residual_rows"], ids=lambda r: r["id"])
def test_residual_hand_rows(row):
    dt = row["in_dtype"]
    r = oracle.rmsnorm_fp8(as_bits([row["x"]], dt), as_bits(row["gamma"], dt), in_dtype=dt, eps=row["eps"],
                           weight_offset=row["weight_offset"], scale_ub=row["scale_ub"], out_fmt=row["out_fmt"],
                           scales_dtype=row["scales_dtype"], residual=as_bits([row["residual"]], dt))
    assert [f"0x{int(v):04X}" for v in r["residual_out"][0]] == row["expect_residual_out_bits"]
    if "expect_codes" in row:
        assert hexes(r["codes"][0]) == row["expect_codes"]


@pytest.mark.parametrize("row", GOLDEN["fp4_rows"], ids=lambda r: r["id"])
def test_fp4_hand_rows(row):
    dt = row["in_dtype"]
    n = len(row["x"])
    gamma = [1.0] * n if row["gamma"] == "ones" else row["gamma"]
    r = oracle.rmsnorm_fp4(as_bits([row["x"]], dt), as_bits(gamma, dt), in_dtype=dt, eps=row["eps"],
                           weight_offset=row["weight_offset"], global_scale=row["global_scale"])
    assert hexes(r["block_scales"][0]) == row["expect_block_scales"]
    assert hexes(r["packed"][0]) == row["expect_packed"]


def test_fp4_hand_row_global_scale_is_derived():
    """The fixture's global scale is fp32(448*6 / global amax), global amax = 6*rstd."""
    row = GOLDEN["fp4_rows"][0]
    s2 = sum(D(v) * D(v) for v in row["x"])
    rstd = 1 / (s2 / len(row["x"]) + D(float(np.float32(row["eps"])))).sqrt()
    assert float(np.float32(float(D(448 * 6) / (6 * rstd)))) == row["global_scale"]
    x = as_bits([row["x"]], "f32")
    gm = oracle.absmax(x, as_bits([1.0] * len(row["x"]), "f32"), in_dtype="f32", eps=row["eps"], weight_offset=0)
    assert abs(D(gm) - 6 * rstd) <= 6 * rstd * D(1e-15)


# ---- closed forms on random rows -----------------------------------------

def _random_case(seed, rows, hidden, dt, gamma_lo=0.5, gamma_hi=1.5, scale=1.0):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((rows, hidden)) * scale).to(TD[dt])
    g = torch.from_numpy(rng.uniform(gamma_lo, gamma_hi, hidden)).to(TD[dt])
    return x, g


def _near_midpoint(fmt, q, rel=1e-9):
    """True where |q| lies within rel of a midpoint between adjacent codes."""
    maxc = {"e4m3fn": 0x7E, "e4m3fnuz": 0x7F, "e2m1": 7}[fmt]
    mags = oracle.decode(fmt, np.arange(maxc + 1))
    mids = (mags[:-1] + mags[1:]) / 2
    a = np.abs(q)[..., None]
    return np.any(np.abs(a - mids) <= rel * mids, axis=-1)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
def test_fp8_codes_match_rstd_free_closed_form(dt, fmt):
    """q_j = FMAX * s_j g'_j / max|s g'| exactly; the oracle's rounded path must agree."""
    x, g = _random_case(5, 24, 256, dt)
    off = 0.25
    r = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), in_dtype=dt, eps=1e-5, weight_offset=off,
                           scale_ub=1e9, out_fmt=fmt, scales_dtype="f32")
    fmax = oracle.decode(fmt, [{"e4m3fn": 0x7E, "e4m3fnuz": 0x7F}[fmt]])[0]
    sg = x.to(torch.float64).numpy() * (g.to(torch.float64).numpy() + off)
    q = fmax * sg / np.abs(sg).max(axis=1, keepdims=True)
    expect = oracle.encode(fmt, q)
    near = _near_midpoint(fmt, q, 1e-6)
    assert np.array_equal(r["codes"][~near], expect[~near])
    # every row's largest element maps to +-FMAX
    j = np.abs(sg).argmax(axis=1)
    top = r["codes"][np.arange(sg.shape[0]), j] & 0x7F
    assert np.all(top == {"e4m3fn": 0x7E, "e4m3fnuz": 0x7F}[fmt])


def test_fp8_scale_closed_form_constant_rows():
    """Constant row c with gamma g: rstd = 1/sqrt(c^2 + eps), scale = |c| g rstd / FMAX."""
    for c, gval, eps in [(3.0, 1.0, 1e-6), (0.5, 2.0, 0.75), (-7.0, 0.5, 1e-5), (1e-3, 1.0, 1e-6)]:
        x = as_bits([[c] * 64], "f32")
        g = as_bits([gval] * 64, "f32")
        r = oracle.rmsnorm_fp8(x, g, in_dtype="f32", eps=eps, weight_offset=0, scale_ub=1e9,
                               out_fmt="e4m3fn", scales_dtype="f32")
        e = D(float(np.float32(eps)))
        cc = D(float(np.float32(c)))
        exact = abs(cc) * D(gval) / (cc * cc + e).sqrt() / 448
        assert abs(D(float(r["sc"][0])) - exact) <= exact * D(1e-15)
        assert np.all((r["codes"][0] & 0x7F) == 0x7E)
        assert np.all((r["codes"][0] >> 7) == (1 if c < 0 else 0))


def test_fp8_scale_ub_binds():
    x, g = _random_case(9, 8, 128, "bf16")
    ub = 1e-3
    r = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0,
                           scale_ub=ub, out_fmt="e4m3fn", scales_dtype="f32")
    assert np.all(r["scales"] == np.float32(ub))
    y = oracle.rmsnorm_y(workloads.bits(x), workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0)["y"]
    q = y / float(np.float32(ub))
    assert np.allclose(r["q"], q, rtol=1e-15, atol=0)
    sat = np.abs(q) >= 448
    assert np.all((r["codes"][sat] & 0x7F) == 0x7E)


def test_gamma_zero_gives_zero_codes():
    x, _ = _random_case(2, 4, 64, "bf16")
    g = torch.zeros(64, dtype=torch.bfloat16)
    for fmt in ("e4m3fn", "e4m3fnuz"):
        r = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0,
                               scale_ub=1200, out_fmt=fmt, scales_dtype="f32")
        assert np.all(r["scales"] == 0)
        assert np.all((r["codes"] & 0x7F) == 0)
        if fmt == "e4m3fn":
            neg = x.to(torch.float32).numpy() < 0
            assert np.array_equal(r["codes"] == 0x80, neg)


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_power_of_two_scaling_leaves_fp8_codes(k):
    x, g = _random_case(4, 16, 512, "bf16")
    base = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0,
                              scale_ub=1e9, out_fmt="e4m3fn", scales_dtype="f32")
    xs = (x.to(torch.float64) * 2.0**k).to(torch.bfloat16)
    sc = oracle.rmsnorm_fp8(workloads.bits(xs), workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0,
                            scale_ub=1e9, out_fmt="e4m3fn", scales_dtype="f32")
    near = _near_midpoint("e4m3fn", base["q"], 1e-6)
    assert np.array_equal(base["codes"][~near], sc["codes"][~near])


def test_weight_offset_folds_into_gamma():
    x, g = _random_case(6, 8, 256, "f32")
    g = g.to(torch.bfloat16).to(torch.float32)  # 8 significant bits, so g + 0.5 is exact in fp32
    off = 0.5
    r1 = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), in_dtype="f32", eps=1e-6, weight_offset=off,
                            scale_ub=1200, out_fmt="e4m3fn", scales_dtype="f32")
    g2 = (g.to(torch.float64) + off).to(torch.float32)  # exact for these magnitudes
    assert torch.equal(g2.to(torch.float64), g.to(torch.float64) + off)
    r2 = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g2), in_dtype="f32", eps=1e-6, weight_offset=0,
                            scale_ub=1200, out_fmt="e4m3fn", scales_dtype="f32")
    assert np.array_equal(r1["codes"], r2["codes"]) and np.array_equal(r1["scales"], r2["scales"])


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_residual_out_matches_torch_sum(dt):
    rng = np.random.default_rng(21)
    x = torch.from_numpy(rng.standard_normal((8, 256)) * np.exp2(rng.integers(-12, 12, (8, 256)))).to(TD[dt])
    r = torch.from_numpy(rng.standard_normal((8, 256)) * np.exp2(rng.integers(-12, 12, (8, 256)))).to(TD[dt])
    g = torch.ones(256, dtype=TD[dt])
    out = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), in_dtype=dt, eps=1e-6, weight_offset=0,
                             scale_ub=1200, out_fmt="e4m3fn", scales_dtype="f32", residual=workloads.bits(r))
    ref = workloads.bits((x.float() + r.float()).to(TD[dt]))
    assert np.array_equal(out["residual_out"], ref)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_residual_path_equals_plain_path_on_sum(dt):
    x, g = _random_case(8, 12, 384, dt)
    res, _ = _random_case(18, 12, 384, dt)
    kw = dict(in_dtype=dt, eps=1e-5, weight_offset=0, scale_ub=1200, out_fmt="e4m3fn", scales_dtype="f32")
    fused = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), residual=workloads.bits(res), **kw)
    plain = oracle.rmsnorm_fp8(fused["residual_out"], workloads.bits(g), **kw)
    assert np.array_equal(fused["codes"], plain["codes"])
    assert np.array_equal(fused["scales"], plain["scales"])


def test_row_permutation_permutes_outputs():
    x, g = _random_case(3, 10, 128, "bf16")
    kw = dict(in_dtype="bf16", eps=1e-6, weight_offset=0, scale_ub=1200, out_fmt="e4m3fn", scales_dtype="bf16")
    a = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), **kw)
    perm = np.random.default_rng(0).permutation(10)
    b = oracle.rmsnorm_fp8(workloads.bits(x)[perm], workloads.bits(g), **kw)
    assert np.array_equal(a["codes"][perm], b["codes"]) and np.array_equal(a["scales"][perm], b["scales"])


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_fp8_dequant_error_within_half_step(fmt, sdt):
    x, g = _random_case(12, 16, 256, "bf16")
    r = oracle.rmsnorm_fp8(workloads.bits(x), workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0,
                           scale_ub=1200, out_fmt=fmt, scales_dtype=sdt)
    y = oracle.rmsnorm_y(workloads.bits(x), workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0)["y"]
    scale = oracle.value_of(sdt, r["scales"])[:, None]
    deq = oracle.decode(fmt, r["codes"]) * scale
    maxc = {"e4m3fn": 0x7E, "e4m3fnuz": 0x7F}[fmt]
    mags = oracle.decode(fmt, np.arange(maxc + 1))
    m = (r["codes"] & 0x7F).astype(int)
    step = np.where(m < maxc, mags[np.minimum(m + 1, maxc)] - mags[m], mags[m] - mags[m - 1])
    step_below = np.where(m > 0, mags[m] - mags[np.maximum(m - 1, 0)], step)
    bound = 0.5 * np.maximum(step, step_below) * scale * (1 + 1e-6)
    fmax = mags[maxc]
    unsat = np.abs(y / scale) <= fmax
    assert np.all(np.abs(deq - y)[unsat] <= bound[unsat])
    assert np.all(np.abs(oracle.decode(fmt, r["codes"])) <= fmax)


def test_fp4_dequant_error_and_global_amax_block():
    """Every E2M1 code is within half a step of y*gs/d; the block holding the
    global amax gets scale code 0x7E when gs = 448*6/global_amax."""
    rng = np.random.default_rng(31)
    x = torch.from_numpy(rng.standard_t(3, (8, 512))).to(torch.bfloat16)
    g = torch.from_numpy(rng.uniform(0.8, 1.2, 512)).to(torch.bfloat16)
    xb, gb = workloads.bits(x), workloads.bits(g)
    amax = oracle.absmax(xb, gb, in_dtype="bf16", eps=1e-6, weight_offset=0)
    gs = float(np.float32(448 * 6 / amax))
    r = oracle.rmsnorm_fp4(xb, gb, in_dtype="bf16", eps=1e-6, weight_offset=0, global_scale=gs)
    y = oracle.rmsnorm_y(xb, gb, in_dtype="bf16", eps=1e-6, weight_offset=0)["y"]
    codes = np.stack([r["packed"] & 0xF, r["packed"] >> 4], axis=-1).reshape(8, 512)
    d = oracle.decode("e4m3fn", r["block_scales"])
    assert np.all(d <= 448)
    dd = np.repeat(d, 16, axis=1)
    deq = oracle.decode("e2m1", codes) * dd / gs
    qexact = y * gs / dd
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    m = (codes & 7).astype(np.int64)
    gap = np.where(m < 7, mags[np.minimum(m + 1, 7)] - mags[m], 2.0)
    gap = np.maximum(gap, np.where(m > 0, mags[m] - mags[np.maximum(m - 1, 0)], gap))
    unsat = np.abs(qexact) <= 6
    assert np.all(np.abs(deq - y)[unsat] <= (0.5 * gap * dd / gs * (1 + 1e-6))[unsat])
    # block holding the global maximum
    row, col = np.unravel_index(np.abs(y).argmax(), y.shape)
    assert r["block_scales"][row, col // 16] == 0x7E
    assert (codes[row, col] & 7) == 7


def test_fp4_blocks_are_16_contiguous_elements():
    """A single large element raises only its own 16-element block's scale."""
    x = np.zeros((1, 64), np.float32)
    x[0, :] = 1.0
    x[0, 37] = 100.0  # block 2 (elements 32..47)
    g = np.ones(64, np.float32)
    r = oracle.rmsnorm_fp4(x, g, in_dtype="f32", eps=1e-6, weight_offset=0, global_scale=1.0)
    s = oracle.decode("e4m3fn", r["block_scales"][0])
    assert s[2] > 10 * s[0] and s[0] == s[1] == s[3]
    assert (r["packed"][0, 37 // 2] >> 4) == 7  # odd element -> high nibble, saturating code


def test_workload_generators_are_deterministic_and_shaped():
    for name, w in workloads.WORKLOADS.items():
        rows = min(w.rows, 64)
        a = workloads.make(name, rows=rows)
        b = workloads.make(name, rows=rows)
        assert a["x"].shape == (rows, w.hidden) and a["gamma"].shape == (w.hidden,)
        assert torch.equal(a["x"].view(torch.uint8) if a["x"].dtype != torch.float32 else a["x"],
                           b["x"].view(torch.uint8) if b["x"].dtype != torch.float32 else b["x"])
        assert (a["residual"] is not None) == w.residual
        assert a["x"].dtype == workloads.TORCH_DTYPES[w.in_dtype]
        assert torch.isfinite(a["x"].float()).all()
    c3 = workloads.make("residual_rmsnorm_fp8_bf16_32768x8192", rows=64)
    c3b = workloads.make("residual_rmsnorm_fp8_f32_32768x8192", rows=64)
    assert torch.equal(c3["x"].float(), c3b["x"]) and torch.equal(c3["residual"].float(), c3b["residual"])
    assert math.isclose(workloads.WORKLOADS["rmsnorm_fp4_bf16_16384x7168"].hidden * 0.01, 71.68)
