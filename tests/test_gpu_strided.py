"""GPU: the strided entry points (rmsnorm_fp8_strided, rmsnorm_fp4quant_strided)
on row views of wider buffers give bit-identical results to the contiguous
entry points on the same values, write nothing outside their views, and
allow residual_out over x in place with the same stride.  The contiguous
entry points are checked against the oracle in the other GPU tests, so
identity with them carries that parity over."""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu
TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
CANARY = 0x5A


def _wide(rows, hidden, pad, dt, seed):
    """A [rows, hidden + pad] buffer of random values and its [:, :hidden] view."""
    g = torch.Generator().manual_seed(seed)
    buf = torch.randn((rows, hidden + pad), generator=g, dtype=torch.float64).to(TD[dt]).to(DEV)
    return buf, buf[:, :hidden]


def _canvas(rows, width, used, dtype=torch.uint8):
    """A [rows, width] output buffer filled with the canary and its [:, :used] view."""
    buf = torch.full((rows, width), CANARY, dtype=torch.uint8, device=DEV)
    if dtype != torch.uint8:
        buf = buf.view(dtype)
    return buf, buf[:, :used]


@pytest.mark.parametrize("resid", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_fp8_strided_matches_contiguous(dt, resid):
    rows, hidden = 259, 2048
    esz = torch.tensor([], dtype=TD[dt]).element_size()
    pad = 64 // esz * 3  # a row stride that is not a multiple of the row
    say(f"[strided fp8] {dt} resid={resid}")
    xb, x = _wide(rows, hidden, pad, dt, 1)
    rb, r = _wide(rows, hidden, pad + 16 // esz, dt, 2)
    g = torch.rand(hidden, dtype=torch.float64).add(0.5).to(TD[dt]).to(DEV)
    ob, out = _canvas(rows, hidden + 96, hidden)
    rob, ro = _canvas(rows, (hidden + 32 // esz) * esz, hidden * esz)
    ro = rob.view(TD[dt])[:, :hidden]
    if resid:
        c_out, c_sc, c_ro = rq.residual_rmsnorm_fp8(x.contiguous(), r.contiguous(), g)
        s_out, s_sc, s_ro = rq.rmsnorm_fp8_strided(x, g, residual=r, out=out, residual_out=ro)
    else:
        c_out, c_sc = rq.rmsnorm_fp8(x.contiguous(), g)
        s_out, s_sc, s_ro = rq.rmsnorm_fp8_strided(x, g, out=out)
    torch.cuda.synchronize()
    assert s_out.data_ptr() == out.data_ptr()
    assert torch.equal(s_out, c_out) and torch.equal(s_sc, c_sc)
    assert bool((ob[:, hidden:] == CANARY).all()), "bytes outside the code view were written"
    if resid:
        assert torch.equal(s_ro, c_ro)
        assert bool((rob[:, hidden * esz:] == CANARY).all()), "bytes outside residual_out's view were written"


@pytest.mark.parametrize("resid", [False, True])
@pytest.mark.parametrize("dt,block,fmt,swz", [("bf16", 16, "e4m3", False), ("bf16", 32, "ue8m0", True),
                                              ("f16", 32, "e4m3", False), ("f32", 16, "ue8m0", True)])
def test_fp4_strided_matches_contiguous(dt, block, fmt, swz, resid):
    rows, hidden = 300, 4096
    esz = torch.tensor([], dtype=TD[dt]).element_size()
    say(f"[strided fp4] {dt} block={block} {fmt} swizzled={swz} resid={resid}")
    xb, x = _wide(rows, hidden, 128 // esz, dt, 3)
    rb, r = _wide(rows, hidden, 48 // esz, dt, 4)
    g = torch.rand(hidden, dtype=torch.float64).add(0.5).to(TD[dt]).to(DEV)
    gs = torch.tensor([33.0], dtype=torch.float32, device=DEV)
    ob, out = _canvas(rows, hidden // 2 + 40, hidden // 2)
    kw = dict(global_scale=gs, block_size=block, scale_format=fmt, swizzled=swz)
    if resid:
        c_p, c_s, c_ro = rq.residual_rmsnorm_fp4quant(x.contiguous(), r.contiguous(), g, **kw)
        s_p, s_s, s_ro = rq.rmsnorm_fp4quant_strided(x, g, residual=r, out=out, **kw)
        assert torch.equal(s_ro, c_ro)
    else:
        c_p, c_s = rq.rmsnorm_fp4quant(x.contiguous(), g, **kw)
        s_p, s_s, _ = rq.rmsnorm_fp4quant_strided(x, g, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.equal(s_p, c_p)
    if swz:  # padding bytes of the swizzled buffer are unspecified: compare the scale positions
        n = hidden // block
        r_, c_ = np.meshgrid(np.arange(rows), np.arange(n), indexing="ij")
        import oracle
        idx = torch.as_tensor(oracle.swizzled_offset(r_, c_, n).ravel(), device=DEV)
        assert torch.equal(s_s[idx], c_s[idx])
    else:
        assert torch.equal(s_s, c_s)
    assert bool((ob[:, hidden // 2:] == CANARY).all()), "bytes outside the code view were written"


@pytest.mark.parametrize("fp4", [False, True])
def test_strided_in_place_residual(fp4):
    rows, hidden = 97, 1024
    say(f"[strided in place] fp4={fp4}")
    xb, x = _wide(rows, hidden, 64, "bf16", 5)
    rb, r = _wide(rows, hidden, 64, "bf16", 6)
    g = torch.rand(hidden, dtype=torch.float64).add(0.5).to(torch.bfloat16).to(DEV)
    want_sum = (x.float() + r.float()).to(torch.bfloat16)
    if fp4:
        want = rq.residual_rmsnorm_fp4quant(x.contiguous(), r.contiguous(), g, block_size=32)
        got = rq.rmsnorm_fp4quant_strided(x, g, residual=r, residual_out=x, block_size=32)
    else:
        want = rq.residual_rmsnorm_fp8(x.contiguous(), r.contiguous(), g)
        got = rq.rmsnorm_fp8_strided(x, g, residual=r, residual_out=x)
    torch.cuda.synchronize()
    assert torch.equal(x, want_sum)  # x now holds the sum, padding columns untouched
    assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])
