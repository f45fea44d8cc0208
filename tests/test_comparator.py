"""The comparator accepts the oracle's own output and rejects planted
mistakes (all planted on the CPU, in copies of the oracle's output)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_cap, compare_fp4, compare_fp8, near_midpoint


def _case(dt="bf16", rows=16, hidden=256, seed=0, resid=False, sdt="f32", fmt="e4m3fn"):
    rng = np.random.default_rng(seed)
    td = workloads.TORCH_DTYPES[dt]
    x = workloads.bits(torch.from_numpy(rng.standard_normal((rows, hidden))).to(td))
    r = workloads.bits(torch.from_numpy(rng.standard_normal((rows, hidden))).to(td)) if resid else None
    g = workloads.bits(torch.from_numpy(rng.uniform(0.5, 1.5, hidden)).to(td))
    kw = dict(in_dtype=dt, eps=1e-6, weight_offset=0.0)
    ref = oracle.rmsnorm_fp8(x, g, scale_ub=1200.0, out_fmt=fmt, scales_dtype=sdt, residual=r, **kw)
    y = oracle.rmsnorm_y(x, g, residual=r, **kw)["y"]
    return ref, y


def test_oracle_output_passes_exactly():
    ref, y = _case(resid=True)
    rep = compare_fp8(ref["codes"], ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32",
                      gpu_residual_out=ref["residual_out"])
    assert rep["codes_boundary"] == 0 and rep["scale_max_rel"] == 0


def test_code_flip_away_from_boundary_fails():
    ref, y = _case()
    codes = ref["codes"].copy()
    far = np.nonzero(~near_midpoint("e4m3fn", ref["q"]).ravel() & (codes.ravel() & 0x7F > 1))[0][0]
    codes.ravel()[far] += 1
    with pytest.raises(AssertionError, match="away from a rounding boundary"):
        compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32")


def _tie_rows(n_rows, hidden=8):
    # x = [3, 4, 3, 3, ...]: q = 336 for every 3, exactly halfway between 320 and 352
    x = np.full((n_rows, hidden), 3.0, np.float32)
    x[:, 1] = 4.0
    g = np.ones(hidden, np.float32)
    kw = dict(in_dtype="f32", eps=1e-6, weight_offset=0.0)
    ref = oracle.rmsnorm_fp8(x, g, scale_ub=1200.0, out_fmt="e4m3fn", scales_dtype="f32", **kw)
    y = oracle.rmsnorm_y(x, g, **kw)["y"]
    return ref, y


def test_one_step_across_a_midpoint_passes_but_wrong_direction_fails():
    ref, y = _tie_rows(2000)  # 16000 codes; 1 flip is within 0.01%
    i = (0, 0)
    assert ref["codes"][i] in (0x7A, 0x7B)
    other = 0x7B if ref["codes"][i] == 0x7A else 0x7A
    codes = ref["codes"].copy()
    codes[i] = other
    rep = compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32")
    assert rep["codes_boundary"] == 1
    codes[i] = ref["codes"][i] - 1 if other > ref["codes"][i] else ref["codes"][i] + 1  # wrong side
    with pytest.raises(AssertionError):
        compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32")
    codes[i] = other | 0x80  # sign flip
    with pytest.raises(AssertionError):
        compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32")


def test_every_boundary_flip_counts_against_the_cap_ties_included():
    # 4 rows x 6 exact ties: 24 flips in 32 codes, far above 0.01%
    ref, y = _tie_rows(4)
    codes = ref["codes"].copy()
    tie = (ref["codes"] == 0x7A) | (ref["codes"] == 0x7B)
    codes[tie] ^= 0x01  # 0x7A <-> 0x7B at exact ties
    with pytest.raises(AssertionError, match="exceed"):
        compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32")
    rep = compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32", cap=False)
    assert rep["codes_boundary"] == rep["codes_boundary_ties"] == int(tie.sum()) > 0
    # one tie flip in 2000 x 8 = 16000 codes is within the cap; two are not
    ref, y = _tie_rows(2000)
    codes = ref["codes"].copy()
    flip = lambda c: 0x7B if c == 0x7A else 0x7A  # noqa: E731
    codes[0, 0] = flip(codes[0, 0])
    assert compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32")["codes_boundary"] == 1
    codes[5, 2] = flip(codes[5, 2])
    with pytest.raises(AssertionError, match="exceed"):
        compare_fp8(codes, ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32")
    # q = 336 * (1 + 5e-7): inside the 1e-6 boundary band, not a tie; one
    # flip in 32 codes exceeds the cap
    x = np.full((4, 8), 3.0, np.float32)
    x[:, 0] = np.float32(3.0 * (1 + 5e-7))
    x[:, 1] = 4.0
    g = np.ones(8, np.float32)
    kw = dict(in_dtype="f32", eps=1e-6, weight_offset=0.0)
    ref2 = oracle.rmsnorm_fp8(x, g, scale_ub=1200.0, out_fmt="e4m3fn", scales_dtype="f32", **kw)
    y2 = oracle.rmsnorm_y(x, g, **kw)["y"]
    assert near_midpoint("e4m3fn", ref2["q"][:, 0]).all() and not near_midpoint("e4m3fn", ref2["q"][:, 0], 2.0**-22).any()
    c2 = ref2["codes"].copy()
    c2[0, 0] = 0x7A if c2[0, 0] == 0x7B else 0x7B
    with pytest.raises(AssertionError, match="exceed"):
        compare_fp8(c2, ref2["scales"], ref2, y2, out_fmt="e4m3fn", scales_dtype="f32")
    rep = compare_fp8(c2, ref2["scales"], ref2, y2, out_fmt="e4m3fn", scales_dtype="f32", cap=False)
    assert rep["codes_boundary"] == 1 and rep["codes_boundary_ties"] == 0
    with pytest.raises(AssertionError, match="exceed"):
        check_cap(rep["codes_boundary"], rep["codes_total"])
    check_cap(1, 10_000)


def test_scale_tolerance():
    ref, y = _case()
    s = ref["scales"].copy()
    s[3] = np.float32(s[3] * (1 + 5e-7))
    compare_fp8(ref["codes"], s, ref, y, out_fmt="e4m3fn", scales_dtype="f32")
    s[3] = np.float32(ref["scales"][3] * (1 + 3e-6))
    with pytest.raises(AssertionError, match="fp32 scale"):
        compare_fp8(ref["codes"], s, ref, y, out_fmt="e4m3fn", scales_dtype="f32")


def test_bf16_scale_off_by_one_away_from_boundary_fails():
    ref, y = _case(sdt="bf16")
    s = ref["scales"].copy()
    s[0] += 1
    with pytest.raises(AssertionError, match="away from a rounding boundary"):
        compare_fp8(ref["codes"], s, ref, y, out_fmt="e4m3fn", scales_dtype="bf16")


def test_residual_out_bit_flip_fails():
    ref, y = _case(resid=True)
    ro = ref["residual_out"].copy()
    ro[2, 5] ^= 1
    with pytest.raises(AssertionError, match="residual_out"):
        compare_fp8(ref["codes"], ref["scales"], ref, y, out_fmt="e4m3fn", scales_dtype="f32", gpu_residual_out=ro)


def test_fp4_planted_mistakes():
    rng = np.random.default_rng(5)
    x = workloads.bits(torch.from_numpy(rng.standard_t(3, (8, 256))).to(torch.bfloat16))
    g = workloads.bits(torch.from_numpy(rng.uniform(0.8, 1.2, 256)).to(torch.bfloat16))
    kw = dict(in_dtype="bf16", eps=1e-6, weight_offset=0.0)
    gs = float(np.float32(448 * 6 / oracle.absmax(x, g, **kw)))
    ref = oracle.rmsnorm_fp4(x, g, global_scale=gs, **kw)
    y = oracle.rmsnorm_y(x, g, **kw)["y"]
    rep = compare_fp4(ref["packed"], ref["block_scales"], ref, y, global_scale=gs)
    assert rep["codes_boundary"] == 0 and rep["block_scale_boundary"] == 0
    bs = ref["block_scales"].copy()
    bs[1, 3] += 1
    with pytest.raises(AssertionError, match="block scales"):
        compare_fp4(ref["packed"], bs, ref, y, global_scale=gs)
    p = ref["packed"].copy()
    p[4, 10] ^= 0x20  # high nibble changes by two steps
    with pytest.raises(AssertionError):
        compare_fp4(p, ref["block_scales"], ref, y, global_scale=gs)
    p = ref["packed"].copy()
    p[4, 10] = ((p[4, 10] & 0xF0) >> 4) | ((p[4, 10] & 0x0F) << 4)  # swapped nibbles
    if p[4, 10] != ref["packed"][4, 10]:
        with pytest.raises(AssertionError):
            compare_fp4(p, ref["block_scales"], ref, y, global_scale=gs)
