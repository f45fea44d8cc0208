"""GPU: the device FP8 and E2M1 conversions (the codecs the fused kernels use)
over every fp32 bit pattern whose magnitude lies where the formats round:
from below half the smallest subnormal to past the largest finite value, all
2^23 mantissas of every such exponent, both signs, each code checked to be
the saturating round-to-nearest-even result through the properties in
tests/codec_props.py.  Outside the band every value rounds to zero or
saturates; sampled patterns there are checked against the oracle's encoder
in test_gpu_convert.py."""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
from codec_props import BANDS, band_values, check_codes
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

KIND = {"e4m3fn": rq.CVT_F32_TO_E4M3FN, "e4m3fnuz": rq.CVT_F32_TO_E4M3FNUZ, "e2m1": rq.CVT_F32_TO_E2M1}


@pytest.mark.parametrize("fmt", list(BANDS))
def test_every_pattern_in_the_rounding_band(fmt):
    exps = BANDS[fmt][2]
    n = 1 << 23
    src = torch.empty(n, dtype=torch.float32, device=DEV)
    dst = torch.empty(n // 2 if fmt == "e2m1" else n, dtype=torch.uint8, device=DEV)
    ties = 0
    for e in exps:
        for sign in (0, 1):
            v = band_values(e, sign)
            src.copy_(torch.from_numpy(v))
            rq.convert(KIND[fmt], src, dst)
            got = dst.cpu().numpy()
            if fmt == "e2m1":
                got = np.stack([got & 0xF, got >> 4], axis=-1).reshape(-1)
            ties += check_codes(fmt, v, got)
    say(f"[convert sweep] {fmt}: {len(exps) * 2 * n} patterns, {ties} exact ties")
