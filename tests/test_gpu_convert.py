"""The device conversions (the exact codecs the fused kernels use) against the
oracle's encoders, bit-exact on fp32 inputs: both sides take the decision on
the same fp32 value, so no boundary tolerance applies here.

Inputs: every code's value, every midpoint between adjacent codes and its
fp32 neighbours (ties to even, both directions), signed zeros, values past
saturation, and random fp32 bit patterns.
"""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import oracle
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

MAXC = {"e4m3fn": 0x7E, "e4m3fnuz": 0x7F, "e2m1": 0x7}
KIND = {"e4m3fn": rq.CVT_F32_TO_E4M3FN, "e4m3fnuz": rq.CVT_F32_TO_E4M3FNUZ, "e2m1": rq.CVT_F32_TO_E2M1}


def structured_values(fmt, rng, n_random=1 << 20):
    mags = oracle.decode(fmt, np.arange(MAXC[fmt] + 1))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = [mags.astype(np.float32), mids]
    up, dn = mids.copy(), mids.copy()
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        vals += [up, dn]
    fmax = np.float32(mags[-1])
    vals.append(np.array([0.0, fmax * 1.01, fmax * 1.0625, fmax * 2, 1e6, 3e38, 1e-30, 1e-40], np.float32))
    # fnuz top-range boundaries (224 / 232 / 240)
    vals.append(np.array([224, 228, 232, np.nextafter(np.float32(232), np.float32(0)),
                          np.nextafter(np.float32(232), np.float32(1e9)), 236, 240, 244, 248], np.float32))
    bits = rng.integers(0, 2**32, n_random, dtype=np.uint64).astype(np.uint32)
    r = bits.view(np.float32)
    r = r[np.isfinite(r)]
    # random magnitudes on a log scale around the format's range
    lg = (rng.standard_normal(n_random) * 4).astype(np.float32)
    r2 = np.exp2(lg).astype(np.float32) * rng.choice(np.array([-1, 1], np.float32), n_random)
    v = np.concatenate(vals)
    v = np.concatenate([v, -v, r, r2]).astype(np.float32)
    if v.size % 2:
        v = np.append(v, np.float32(0))
    return v


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz", "e2m1"])
def test_quantize_matches_oracle_encoder(fmt):
    rng = np.random.default_rng(100 + MAXC[fmt])
    v = structured_values(fmt, rng)
    say(f"convert f32->{fmt}: {v.size} values")
    src = torch.from_numpy(v).to(DEV)
    n_out = v.size // 2 if fmt == "e2m1" else v.size
    dst = torch.empty(n_out, dtype=torch.uint8, device=DEV)
    rq.convert(KIND[fmt], src, dst)
    got = dst.cpu().numpy()
    if fmt == "e2m1":
        got = np.stack([got & 0xF, got >> 4], axis=-1).reshape(-1)
    expect = oracle.encode(fmt, v.astype(np.float64))
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {v[bad[:6]]}: gpu {got[bad[:6]]} oracle {expect[bad[:6]]}"


@pytest.mark.parametrize("dt,kind", [("bf16", rq.CVT_F32_TO_BF16), ("f16", rq.CVT_F32_TO_F16)])
def test_round_to_16bit_matches_oracle(dt, kind):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, 1 << 21, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    if dt == "f16":
        v = v[np.abs(v) < 65504.0]
        nrm = (rng.standard_normal(1 << 20) * 100).astype(np.float32)
    else:
        v = v[np.abs(v) < 3.3e38]
        nrm = rng.standard_normal(1 << 20).astype(np.float32)
    v = np.concatenate([v, nrm])
    say(f"convert f32->{dt}: {v.size} values")
    src = torch.from_numpy(v).to(DEV)
    dst = torch.empty(v.size, dtype=torch.int16, device=DEV)
    rq.convert(kind, src, dst)
    got = dst.cpu().numpy().view(np.uint16)
    expect = oracle.round_to(dt, v.astype(np.float64))
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {v[bad[:6]]}: gpu {got[bad[:6]]} oracle {expect[bad[:6]]}"


def test_e4m3fn_decode_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    src = codes.to(DEV)
    dst = torch.empty(256, dtype=torch.float32, device=DEV)
    rq.convert(rq.CVT_E4M3FN_TO_F32, src, dst)
    got = dst.cpu().numpy().astype(np.float64)
    expect = oracle.decode("e4m3fn", codes.numpy())
    ok = ~np.isnan(expect)
    assert np.array_equal(got[ok], expect[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(expect[ok]))


def test_convert_tail_lengths():
    """n not a multiple of the 8-element group: the tail is written, nothing past it."""
    for n in (1, 2, 7, 9, 15, 1001):
        v = torch.linspace(-500, 500, n, dtype=torch.float32)
        dst = torch.full((n + 16,), 0xAB, dtype=torch.uint8, device=DEV)
        rq.convert(rq.CVT_F32_TO_E4M3FN, v.to(DEV), dst[:n])
        got = dst.cpu().numpy()
        assert np.array_equal(got[:n], oracle.encode("e4m3fn", v.numpy().astype(np.float64)))
        assert np.all(got[n:] == 0xAB)
