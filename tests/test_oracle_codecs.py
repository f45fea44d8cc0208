"""Pins for the oracle's format codecs, against things other than the oracle.

* torch's float8_e4m3fn / float8_e4m3fnuz decode and (in-range) RNE casts,
* torch's fp32 -> bf16 / fp16 casts and numpy's float64 -> float16 cast,
* brute-force nearest-value search for E2M1 (torch has no fp32 -> fp4 cast),
* closed forms: midpoints between adjacent codes, saturation, signed zeros.

Format facts used: E4M3 max 448 and E2M1 max 6 (FlashInfer rmsnorm_fp4quant.py,
"Constants"); round-to-nearest-even with saturation to the largest finite
value (same file, "FP8 E4M3 Intrinsics" and "E2M1 Conversion"); e4m3fnuz is
one of the output types of the Mojo rms_norm_fused_fp8 page (Parameters).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")
TORCH_FP8 = {"e4m3fn": torch.float8_e4m3fn, "e4m3fnuz": torch.float8_e4m3fnuz}
MAX_CODE = {"e4m3fn": 0x7E, "e4m3fnuz": 0x7F, "e2m1": 0x7}


def torch_decode(fmt, codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(TORCH_FP8[fmt]).to(torch.float64).numpy()


def torch_encode(fmt, values_f32):
    return torch.from_numpy(np.asarray(values_f32, np.float32)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
def test_fp8_decode_all_codes_matches_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode(fmt, codes)
    ref = torch_decode(fmt, codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # signed zero where the format has one
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_format_maxima():
    assert oracle.decode("e4m3fn", [0x7E])[0] == 448.0
    assert oracle.decode("e4m3fnuz", [0x7F])[0] == 240.0
    assert oracle.decode("e2m1", [0x7])[0] == 6.0
    assert np.isnan(oracle.decode("e4m3fn", [0x7F])[0])
    assert np.isnan(oracle.decode("e4m3fnuz", [0x80])[0])


def test_e2m1_decode_table():
    # 2 exponent bits, 1 mantissa bit, bias 1 (OCP MX E2M1): the eight magnitudes
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = oracle.decode("e2m1", np.arange(16))
    assert list(vals[:8]) == mags
    assert list(-vals[8:]) == mags
    assert np.signbit(vals[8])


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz", "e2m1"])
def test_round_trip_every_code(fmt):
    n = 16 if fmt == "e2m1" else 256
    codes = np.arange(n, dtype=np.uint8)
    vals = oracle.decode(fmt, codes)
    ok = ~np.isnan(vals)
    back = oracle.encode(fmt, vals[ok])
    expect = codes[ok].copy()
    if fmt == "e4m3fnuz":
        pass  # 0x80 is NaN, so every finite code is its own image
    assert np.array_equal(back, expect)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz", "e2m1"])
def test_midpoints_ties_to_even_and_neighbours(fmt):
    mags = oracle.decode(fmt, np.arange(MAX_CODE[fmt] + 1)) if fmt == "e2m1" else \
        torch_decode(fmt, np.arange(MAX_CODE[fmt] + 1))
    lo, hi = mags[:-1], mags[1:]
    mid = (lo + hi) / 2.0  # exact in float64
    m = np.arange(len(lo))
    even = np.where(m % 2 == 0, m, m + 1)
    assert np.array_equal(oracle.encode(fmt, mid), even)
    assert np.array_equal(oracle.encode(fmt, np.nextafter(mid, np.inf)), m + 1)
    assert np.array_equal(oracle.encode(fmt, np.nextafter(mid, -np.inf)), m)
    sign = 0x8 if fmt == "e2m1" else 0x80
    neg = oracle.encode(fmt, -mid)
    expect = even | sign
    if fmt == "e4m3fnuz":
        expect = np.where(even == 0, 0, expect)  # no negative zero in fnuz
    assert np.array_equal(neg, expect)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz", "e2m1"])
def test_saturation(fmt):
    fmax = oracle.decode(fmt, [MAX_CODE[fmt]])[0]
    big = np.array([fmax, fmax * (1 + 1e-9), fmax * 1.0625, fmax * 2, 1e30, np.inf])
    assert np.all(oracle.encode(fmt, big) == MAX_CODE[fmt])
    sign = 0x8 if fmt == "e2m1" else 0x80
    assert np.all(oracle.encode(fmt, -big) == MAX_CODE[fmt] | sign)


def test_signed_zero():
    z = np.array([0.0, -0.0, -1e-300, 1e-300])
    assert list(oracle.encode("e4m3fn", z)) == [0x00, 0x80, 0x80, 0x00]
    assert list(oracle.encode("e4m3fnuz", z)) == [0, 0, 0, 0]
    assert list(oracle.encode("e2m1", z)) == [0x0, 0x8, 0x8, 0x0]


@pytest.mark.parametrize("fmt,limit", [("e4m3fn", 464.0), ("e4m3fnuz", 248.0)])
def test_fp8_encode_matches_torch_in_range(fmt, limit):
    """torch's cast is RNE but not saturating: compare where it returns a finite code."""
    rng = np.random.default_rng(1234)
    # log-uniform magnitudes across the whole normal + subnormal range, random signs
    mag = np.exp2(rng.uniform(-13.0, np.log2(limit), 400_000)).astype(np.float32)
    v = mag * rng.choice(np.array([-1, 1], np.float32), mag.size)
    # dense neighbourhoods of every midpoint between adjacent codes
    mags = torch_decode(fmt, np.arange(MAX_CODE[fmt] + 1))
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    around = [mid]
    for k in range(1, 4):
        around += [np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))]
        mid = around[-2]
    v = np.concatenate([v, *around, -np.concatenate(around)]).astype(np.float32)
    v = v[np.abs(v) < limit]
    mine = oracle.encode(fmt, v.astype(np.float64))
    ref = torch_encode(fmt, v)
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {v[bad[:5]]} -> {mine[bad[:5]]} vs {ref[bad[:5]]}"


def _e2m1_brute(v):
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    out = []
    for x in v:
        a = min(abs(x), 6.0)
        d = np.abs(mags - a)
        best = np.nonzero(d == d.min())[0]
        m = int(best[0]) if best.size == 1 else int([b for b in best if b % 2 == 0][0])
        if np.signbit(x):
            m |= 8
        out.append(m)
    return np.array(out, np.uint8)


def test_e2m1_brute_force_grid():
    grid = np.arange(-8.0, 8.0, 1.0 / 256)
    extra = []
    for m in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]:
        for s in (1, -1):
            extra += [s * m, s * np.nextafter(m, 0), s * np.nextafter(m, 10)]
    v = np.concatenate([grid, np.array(extra)])
    assert np.array_equal(oracle.encode("e2m1", v), _e2m1_brute(v))


def test_e2m1_ties_fixture():
    g = json.load(open(GOLDEN))["e2m1_ties"]
    codes = [int(c, 16) for c in g["codes"]]
    assert list(oracle.encode("e2m1", np.array(g["values"]))) == codes


# ---- IEEE half / bfloat16 rounding ----------------------------------------

def _random_f32(rng, n):
    b = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    f = b.view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("dt,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_round_from_fp32_matches_torch(dt, tdt):
    rng = np.random.default_rng(7)
    f = _random_f32(rng, 1_000_000)
    # values just around representable midpoints of the 16-bit grid
    base = rng.standard_normal(100_000).astype(np.float32)
    if dt == "bf16":
        half = base.view(np.uint32) & np.uint32(0xFFFF0000) | np.uint32(0x8000)
    else:
        half = base.astype(np.float16).astype(np.float32)
        half = (half.astype(np.float64) + np.abs(half.astype(np.float64)) * 2.0**-12).astype(np.float32)
    mids = half.view(np.float32) if dt == "bf16" else half
    f = np.concatenate([f, mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    if dt == "f16":
        f = f[np.abs(f) < 65520.0]  # beyond this the cast overflows to inf (checked separately)
    else:
        f = f[np.abs(f) < 3.3e38]
    mine = oracle.round_to(dt, f.astype(np.float64))
    ref = torch.from_numpy(f).to(tdt).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches e.g. {f[bad[:4]]}: {mine[bad[:4]]} vs {ref[bad[:4]]}"


def test_f16_round_from_float64_matches_numpy():
    """numpy converts float64 -> float16 with one rounding, straight from float64."""
    rng = np.random.default_rng(11)
    v = rng.standard_normal(300_000) * np.exp2(rng.uniform(-26, 16, 300_000))
    v = v[np.abs(v) < 65504.0]
    mine = oracle.round_to("f16", v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_value_of_round_trip():
    rng = np.random.default_rng(3)
    for dt, n in (("bf16", 65536), ("f16", 65536)):
        bits = np.arange(n, dtype=np.uint16)
        vals = oracle.value_of(dt, bits)
        finite = np.isfinite(vals)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float16
        ref = torch.from_numpy(bits.view(np.int16)).view(tdt).to(torch.float64).numpy()
        assert np.array_equal(vals[finite], ref[finite])
        back = oracle.round_to(dt, vals[finite])
        # +/-0 and every finite value map back to themselves
        assert np.array_equal(back, bits[finite])
    del rng


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz", "e2m1"])
def test_encoder_every_pattern_in_the_rounding_band(fmt):
    """The oracle's encoder over every fp32 pattern whose magnitude lies where
    the format rounds (all 2^23 mantissas of each exponent there, both signs),
    checked through the defining properties of saturating RNE on the decoded
    magnitudes (tests/codec_props.py); past the band, values saturate or round
    to zero, which test_saturation and test_signed_zero pin."""
    from concurrent.futures import ThreadPoolExecutor

    from codec_props import BANDS, band_values, check_codes

    def one(es):
        e, sign = es
        v = band_values(e, sign)
        return check_codes(fmt, v, oracle.encode(fmt, v.astype(np.float64)))

    jobs = [(e, s) for e in BANDS[fmt][2] for s in (0, 1)]
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        ties = sum(ex.map(one, jobs))
    assert ties > 0  # the band holds exact midpoints; they were met and went to even
