"""Pins of the oracle's gated producer (x = a * b rounded once to the input
type, the input_fn of Mojo docs "rms_norm_fused_fp8" that gated_rmsnorm_fp8
builds in), against exact rational arithmetic, a brute-force search over
every finite 16-bit value, hand-derived ties, and identities."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _grid(dt):
    """Every finite value of a 16-bit type with its bits, sorted by value
    (one entry per value: +0 stands for both zeros)."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    vals = oracle.value_of(dt, bits)
    keep = np.isfinite(vals) & ~((vals == 0) & (bits != 0))
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], bits[keep][order]


_GRIDS = {}


def brute_round(dt, exact: Fraction) -> int:
    """The bits of the value of dt nearest to `exact` (ties to the even
    significand), by search over the sorted grid; the sign of a zero result
    is the sign of `exact`."""
    if dt not in _GRIDS:
        _GRIDS[dt] = _grid(dt)
    vals, bits = _GRIDS[dt]
    i = int(np.searchsorted(vals, float(exact)))
    best = None
    for j in (i - 1, i, i + 1):
        if 0 <= j < len(vals):
            d = abs(Fraction(vals[j]) - exact)
            key = (d, int(bits[j]) & 1)  # a tie goes to the even last bit
            if best is None or key < best[0]:
                best = (key, int(bits[j]))
    b = best[1]
    if b == 0 and exact < 0:
        b = 0x8000
    return b


def bits16(dt, values):
    return oracle.round_to(dt, np.asarray(values, dtype=np.float64))


@pytest.mark.parametrize("dt,a,b,expect", [
    # bf16 has 8 significant bits: 1.0625^2 = 1.12890625 lies halfway between
    # 1.125 (even) and 1.1328125, and goes to 1.125
    ("bf16", 1.0625, 1.0625, 1.125),
    # (1 + 2^-7)^2 = 1 + 2^-6 + 2^-14: below the midpoint, down to 1 + 2^-6
    ("bf16", 1 + 2**-7, 1 + 2**-7, 1 + 2**-6),
    # f16 has 11: (1 + 2^-6)(1 + 2^-5) = 1 + 2^-5 + 2^-6 + 2^-11, a tie between
    # 1.046875 (even) and 1.046875 + 2^-10
    ("f16", 1 + 2**-6, 1 + 2**-5, 1.046875),
    # and one ulp of the fraction above the tie rounds up
    ("f16", 1 + 2**-6 + 2**-10, 1 + 2**-5, 1.046875 + 2**-10 * 2),
    ("bf16", -3.0, 0.5, -1.5),
    ("f16", -0.0, 2.0, -0.0),
])
def test_hand_rows(dt, a, b, expect):
    x = oracle.gated_product(bits16(dt, [a]), bits16(dt, [b]), in_dtype=dt)
    assert oracle.value_of(dt, x)[0] == expect
    assert np.signbit(oracle.value_of(dt, x)[0]) == np.signbit(expect)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_brute_force_over_every_16_bit_value(dt):
    rng = np.random.default_rng(11)
    n = 3000
    # magnitudes from far below to near the top of each range, both signs
    hi = 2.0 ** (60 if dt == "bf16" else 7)
    lo = 2.0 ** (-60 if dt == "bf16" else -12)
    mag = np.exp(rng.uniform(np.log(lo), np.log(hi), (2, n)))
    a = bits16(dt, mag[0] * rng.choice([-1.0, 1.0], n))
    b = bits16(dt, mag[1] * rng.choice([-1.0, 1.0], n))
    got = oracle.gated_product(a, b, in_dtype=dt)
    va, vb = oracle.value_of(dt, a), oracle.value_of(dt, b)
    for i in range(n):
        exact = Fraction(va[i]) * Fraction(vb[i])
        if abs(exact) > Fraction(oracle.value_of(dt, np.array([0x7F7F if dt == "bf16" else 0x7BFF], np.uint16))[0]):
            continue  # beyond the largest finite value: overflow, not part of the pin
        assert int(got[i]) == brute_round(dt, exact), (dt, va[i], vb[i])


def test_f32_products_round_once():
    rng = np.random.default_rng(5)
    a = rng.standard_normal(2000).astype(np.float32)
    b = (rng.standard_normal(2000) * 1e3).astype(np.float32)
    got = oracle.gated_product(a, b, in_dtype="f32")
    for i in range(a.size):
        exact = Fraction(float(a[i])) * Fraction(float(b[i]))
        # the exact product has at most 48 significant bits: float() of it is
        # exact, and numpy's float64 -> float32 cast rounds it once (RNE)
        assert float(exact) == Fraction(float(exact))
        assert got[i] == np.float32(float(exact))


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_identities(dt):
    rng = np.random.default_rng(3)
    v = rng.standard_normal((7, 64))
    a = oracle.round_to(dt, v)
    b = oracle.round_to(dt, rng.standard_normal((7, 64)))
    one = oracle.round_to(dt, np.ones_like(v))
    assert np.array_equal(oracle.gated_product(a, one, in_dtype=dt), a)
    assert np.array_equal(oracle.gated_product(a, b, in_dtype=dt), oracle.gated_product(b, a, in_dtype=dt))
    neg = oracle.round_to(dt, -oracle.value_of(dt, b))
    assert np.array_equal(oracle.value_of(dt, oracle.gated_product(a, neg, in_dtype=dt)),
                          -oracle.value_of(dt, oracle.gated_product(a, b, in_dtype=dt)))
