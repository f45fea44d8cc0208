"""Saturating round-to-nearest-even to E4M3FN / E4M3FNUZ / E2M1, checked
through the properties that define it rather than by a second encoder: on
the decoded magnitudes of every code (the oracle's decoder, pinned against
torch's float8 decode and the E2M1 table in test_oracle_codecs.py),
  * magnitudes at or past the largest finite one give the largest code;
  * no representable magnitude is nearer to |v| than the code's;
  * at an exact tie between two magnitudes the code is the even one;
  * the sign bit is v's (e4m3fnuz: zero magnitudes carry no sign).
Sources: FlashInfer rmsnorm_fp4quant.py (FP8 E4M3 Intrinsics, E2M1
Conversion: round to nearest even with saturation to the finite range); the
e4m3fnuz output type of the Mojo rms_norm_fused_fp8 page (Parameters)."""
import numpy as np

import oracle

# format: (largest magnitude code, sign bit, fp32 exponents where the format
# rounds: from below half its smallest subnormal to past its largest value)
BANDS = {
    "e4m3fn": (0x7E, 0x80, range(-11, 10)),    # 2^-9 smallest, 448 largest
    "e4m3fnuz": (0x7F, 0x80, range(-12, 9)),   # 2^-10 smallest, 240 largest
    "e2m1": (0x7, 0x8, range(-3, 4)),          # 0.5 smallest, 6 largest
}
MANTISSAS = np.arange(1 << 23, dtype=np.uint32)


def band_values(e: int, sign: int) -> np.ndarray:
    """All 2^23 fp32 values with exponent e and the given sign."""
    bits = (np.uint32(sign << 31) | np.uint32((e + 127) << 23)) + MANTISSAS
    return bits.view(np.float32)


def check_codes(fmt: str, v: np.ndarray, codes: np.ndarray) -> int:
    """Assert the properties for fp32 values v and their codes; returns the
    number of exact ties met."""
    maxc, sbit, _ = BANDS[fmt]
    mags = oracle.decode(fmt, np.arange(maxc + 1))
    assert np.all(np.diff(mags) > 0)
    m = (codes & (sbit - 1)).astype(np.int64)
    neg = (codes & sbit) != 0
    assert np.all(m <= maxc), "code beyond the largest finite magnitude"
    a = np.abs(v.astype(np.float64))
    got = mags[m]
    sat = a >= mags[maxc]
    assert np.all(m[sat] == maxc), f"saturation: {v[sat & (m != maxc)][:6]}"
    d = np.abs(a - got)
    d_lo = np.where(m > 0, np.abs(a - mags[np.maximum(m - 1, 0)]), np.inf)
    d_hi = np.where(m < maxc, np.abs(a - mags[np.minimum(m + 1, maxc)]), np.inf)
    far = (d > d_lo) | (d > d_hi)
    assert not far.any(), f"not the nearest magnitude: {v[far][:6]} -> codes {codes[far][:6]}"
    tie = ~sat & ((d == d_lo) | (d == d_hi))
    odd = tie & (m % 2 == 1)
    assert not odd.any(), f"tie not to even: {v[odd][:6]} -> codes {codes[odd][:6]}"
    if fmt == "e4m3fnuz":
        assert not (neg & (m == 0)).any(), "negative zero in e4m3fnuz"
        nz = m > 0
        assert np.array_equal(neg[nz], np.signbit(v)[nz])
    else:
        assert np.array_equal(neg, np.signbit(v))
    return int(tie.sum())
