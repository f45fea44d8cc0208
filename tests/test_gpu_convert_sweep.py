"""GPU: the device FP8 and E2M1 conversions (the codecs the fused kernels use)
over every fp32 bit pattern whose magnitude lies where the formats round:
from below half the smallest subnormal to past the largest finite value, all
2^23 mantissas of every such exponent, both signs.  Each code is checked to be
the saturating round-to-nearest-even result through the properties that
define it, on the oracle's decoded magnitude of every code:
  * magnitudes past the largest finite one give the largest finite code;
  * no representable magnitude is nearer to |v| than the code's;
  * at an exact tie between two magnitudes the code is the even one;
  * the sign bit is v's (e4m3fnuz: zero magnitudes carry no sign).
Outside the band every value rounds to zero or saturates; sampled patterns
there are checked against the oracle's encoder in test_gpu_convert.py.
Sources: FlashInfer rmsnorm_fp4quant.py (FP8 E4M3 Intrinsics, E2M1
Conversion: round to nearest even with saturation to the finite range)."""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import oracle
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

# format: (convert kind, largest magnitude code, sign bit, exponents of |v| swept)
FORMATS = {
    "e4m3fn": (rq.CVT_F32_TO_E4M3FN, 0x7E, 0x80, range(-11, 10)),    # 2^-9 smallest, 448 largest
    "e4m3fnuz": (rq.CVT_F32_TO_E4M3FNUZ, 0x7F, 0x80, range(-12, 9)),  # 2^-10 smallest, 240 largest
    "e2m1": (rq.CVT_F32_TO_E2M1, 0x7, 0x8, range(-3, 4)),             # 0.5 smallest, 6 largest
}


def check_codes(fmt, v, codes):
    _, maxc, sbit, _ = FORMATS[fmt]
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


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_every_pattern_in_the_rounding_band(fmt):
    kind, _, _, exps = FORMATS[fmt]
    mant = np.arange(1 << 23, dtype=np.uint32)
    n = mant.size
    src = torch.empty(n, dtype=torch.float32, device=DEV)
    dst = torch.empty(n // 2 if fmt == "e2m1" else n, dtype=torch.uint8, device=DEV)
    ties = 0
    for e in exps:
        for sign in (0, 1):
            bits = (np.uint32(sign << 31) | np.uint32((e + 127) << 23)) + mant
            v = bits.view(np.float32)
            src.copy_(torch.from_numpy(v))
            rq.convert(kind, src, dst)
            got = dst.cpu().numpy()
            if fmt == "e2m1":
                got = np.stack([got & 0xF, got >> 4], axis=-1).reshape(-1)
            ties += check_codes(fmt, v, got)
    say(f"[convert sweep] {fmt}: {len(exps) * 2 * n} patterns, {ties} exact ties")
