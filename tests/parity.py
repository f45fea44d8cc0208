"""Comparator for GPU output against the float64 oracle.

The rule (the tolerance the method's spec gives for this path):
  1. residual_out is bit-exact.
  2. A quantized code may differ from the oracle's only where the oracle's
     unrounded quantizer input q lies within 1e-6 relative of a rounding
     midpoint between two adjacent codes; such a code must be exactly one
     magnitude step away with the same sign, on the other side of that
     midpoint.  Every other code is bit-exact, and the boundary flips, all of
     them, are at most 0.01% of the codes of the tensor (for a tensor of
     fewer than 10^4 codes: none).  Flips whose q is within 2^-22 relative of
     the midpoint (exact ties of the exact-arithmetic ratio FMAX * t / max|t|,
     offset only by the fp32 rounding of the stored scale) are reported
     separately as `_ties`; they count against the cap like every other.
  3. Scales: fp32 per-row scales within 1e-6 relative (zero exactly);
     bf16/fp16 per-row scales and E4M3 block-scale codes bit-exact, except one
     step where the oracle's unrounded scale is within 1e-6 relative of a
     midpoint -- then that row's (block's) codes are re-derived by the oracle
     from the GPU's stored scale before rule 2 is applied.

Why 1e-6: the GPU forms q with a handful of fp32 roundings (relative error
below 4 * 2^-24 ~ 2.4e-7, plus the fp32 reduction error of mean(s^2), below
2e-7 for the rows used here), so a code can only flip when q is that close to
a midpoint; 1e-6 leaves margin and still makes flips rare (a random q lands in
the band with probability ~2e-5 for E4M3, ~4e-6 for E2M1).
"""
from __future__ import annotations

import numpy as np

import oracle

REL = 1e-6
TIE_REL = 2.0**-22
MAX_FRAC = 1e-4
MAXC = {"e4m3fn": 0x7E, "e4m3fnuz": 0x7F, "e2m1": 0x7}
SIGN = {"e4m3fn": 0x80, "e4m3fnuz": 0x80, "e2m1": 0x8}


def _midpoints(fmt):
    mags = oracle.decode(fmt, np.arange(MAXC[fmt] + 1))
    return (mags[:-1] + mags[1:]) / 2.0


def near_midpoint(fmt, q, rel=REL):
    """|q| within rel (relative) of a midpoint between adjacent codes of fmt."""
    mids = _midpoints(fmt)
    a = np.abs(np.asarray(q, np.float64))
    i = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    d = np.minimum(np.abs(a - mids[i - 1]), np.abs(a - mids[i]))
    m = np.where(np.abs(a - mids[i - 1]) <= np.abs(a - mids[i]), mids[i - 1], mids[i])
    return d <= rel * m


def _grid_midpoint_16bit(dtype, v):
    """v (float64) within REL of a rounding midpoint of the bf16/fp16 grid."""
    v = np.abs(np.asarray(v, np.float64))
    lo_bits = oracle.round_to(dtype, v)
    lo = oracle.value_of(dtype, lo_bits)
    # neighbours one step either side of the rounded value
    up = oracle.value_of(dtype, (lo_bits.astype(np.int64) + 1).astype(np.uint16))
    dn = oracle.value_of(dtype, np.maximum(lo_bits.astype(np.int64) - 1, 0).astype(np.uint16))
    mid_up, mid_dn = (lo + up) / 2, (lo + dn) / 2
    return (np.abs(v - mid_up) <= REL * mid_up) | (np.abs(v - mid_dn) <= REL * np.maximum(mid_dn, 1e-300))


class Report(dict):
    def __str__(self):
        return ", ".join(f"{k}={v}" for k, v in self.items() if k != "ok")


def _check_codes(fmt, gpu, expect, q, report, label, cap=True):
    gpu = np.asarray(gpu)
    expect = np.asarray(expect)
    diff = gpu != expect
    n = int(diff.sum())
    report[f"{label}_total"] = int(gpu.size)
    report[f"{label}_boundary"] = n
    if n == 0:
        return
    idx = np.nonzero(diff.ravel())[0]
    g = gpu.ravel()[idx].astype(np.int64)
    e = expect.ravel()[idx].astype(np.int64)
    qq = np.asarray(q).ravel()[idx]
    sign = SIGN[fmt]
    same_sign = (g & sign) == (e & sign)
    # the midpoint nearest |q| lies between magnitude codes i and i+1; the GPU
    # may give the one of those two that the oracle did not
    mids = _midpoints(fmt)
    a = np.abs(qq)
    i = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    i = np.where(np.abs(a - mids[i - 1]) <= np.abs(a - mids[i]), i - 1, i)
    gm, em = g & (sign - 1), e & (sign - 1)
    other_side = ((em == i) & (gm == i + 1)) | ((em == i + 1) & (gm == i))
    near = near_midpoint(fmt, qq)
    bad = ~(same_sign & other_side & near)
    if bad.any():
        j = np.nonzero(bad)[0][:8]
        raise AssertionError(f"{label}: {int(bad.sum())} codes differ away from a rounding boundary; "
                             f"flat index {idx[j]}, gpu {g[j]}, oracle {e[j]}, q {qq[j]}")
    report[f"{label}_boundary_ties"] = int(near_midpoint(fmt, qq, TIE_REL).sum())
    if cap:
        check_cap(n, gpu.size, label)


def check_cap(boundary: int, total: int, label: str = "codes") -> None:
    """Boundary flips (ties included) may be at most MAX_FRAC of the codes."""
    if boundary > MAX_FRAC * total:
        raise AssertionError(f"{label}: {boundary} boundary differences exceed {MAX_FRAC:.2%} of {total} codes "
                             f"({boundary / max(total, 1):.3g})")


def _y(y):
    return y() if callable(y) else y


def compare_fp8(gpu_codes, gpu_scales, ref, y, *, out_fmt, scales_dtype, gpu_residual_out=None, cap=True):
    """gpu_scales: numpy bits (float32 for f32, uint16 otherwise).  ref: oracle.rmsnorm_fp8 result
    (with q).  y: oracle float64 normalized values for the same rows, or a
    callable giving them (needed only where a 16-bit scale differs).
    cap=False leaves the 0.01% cap to the caller (check_cap over a whole
    tensor compared in row chunks)."""
    rep = Report()
    if ref["residual_out"] is not None:
        assert gpu_residual_out is not None
        diff = np.asarray(gpu_residual_out) != ref["residual_out"]
        if diff.any():
            i = np.nonzero(diff.ravel())[0][:8]
            raise AssertionError(f"residual_out differs at {diff.sum()} elements, e.g. flat {i}")
        rep["residual_out_exact"] = True
    expect = ref["codes"].copy()
    q = ref["q"].copy()
    if scales_dtype == "f32":
        o = ref["scales"].astype(np.float64)
        g = np.asarray(gpu_scales, np.float32).astype(np.float64)
        zero = o == 0
        if np.any(g[zero] != 0):
            raise AssertionError("GPU scale nonzero where the oracle's is zero")
        rel = np.abs(g - o)[~zero] / o[~zero]
        rep["scale_max_rel"] = float(rel.max()) if rel.size else 0.0
        if rel.size and rel.max() > REL:
            r = np.nonzero(~zero)[0][rel.argmax()]
            raise AssertionError(f"fp32 scale of row {r}: gpu {g[r]!r} oracle {o[r]!r} rel {rel.max():.3g}")
    else:
        gb = np.asarray(gpu_scales, np.uint16)
        ob = ref["scales"]
        d = gb != ob
        rep["scale_boundary_rows"] = int(d.sum())
        if d.any():
            rows = np.nonzero(d)[0]
            step1 = np.abs(gb[rows].astype(np.int64) - ob[rows].astype(np.int64)) == 1
            near = _grid_midpoint_16bit(scales_dtype, ref["sc"][rows].astype(np.float32).astype(np.float64))
            if not np.all(step1 & near):
                r = rows[~(step1 & near)][:4]
                raise AssertionError(f"{scales_dtype} scales differ away from a rounding boundary at rows {r}")
            # the oracle re-derives those rows' codes from the GPU's stored scale
            if cap:
                check_cap(rep["scale_boundary_rows"], gb.size, f"{scales_dtype} scales")
            gs = oracle.value_of(scales_dtype, gb[rows])[:, None]
            yv = _y(y)
            q[rows] = np.where(gs > 0, yv[rows] / gs, yv[rows] * 0.0)
            expect[rows] = oracle.encode(out_fmt, q[rows].astype(np.float32).astype(np.float64))
    _check_codes(out_fmt, gpu_codes, expect, q, rep, "codes", cap)
    rep["ok"] = True
    return rep


def unpack_e2m1(packed):
    p = np.asarray(packed, np.uint8)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)


def near_power_of_two(v, rel=REL):
    """v (> 0) within rel (relative) of a power of two: the decision points of
    a UE8M0 scale (the smallest power of two >= v)."""
    v = np.asarray(v, np.float64)
    with np.errstate(divide="ignore"):
        p = np.exp2(np.round(np.log2(np.where(v > 0, v, 1.0))))
    return (v > 0) & (np.abs(v - p) <= rel * p)


def compare_fp4(gpu_packed, gpu_block_scales, ref, y, *, global_scale, block_size=16, scale_format="e4m3",
                cap=True):
    """ref: oracle.rmsnorm_fp4 result (with q and sf) for the same block size and
    scale format; y: oracle float64 normalized values; gpu_block_scales
    row-major [rows, hidden/block_size].

    A block-scale code may differ by one where the oracle's unrounded scale
    is within 1e-6 of the format's decision point: an E4M3 rounding midpoint,
    or a power of two for UE8M0 (the scale is the smallest power of two >=
    amax/6).  That block's codes are then re-derived from the GPU's scale.
    Such block-scale flips are themselves scale codes on a boundary: they
    count against the same 0.01% cap, over the block scales.  y may be a
    callable (needed only where a block scale differs); cap=False leaves both
    caps to the caller."""
    rep = Report()
    gb = np.asarray(gpu_block_scales, np.uint8)
    ob = ref["block_scales"]
    q = ref["q"].copy()
    expect = unpack_e2m1(ref["packed"])
    d = gb != ob
    rep["block_scale_boundary"] = int(d.sum())
    if d.any():
        r, b = np.nonzero(d)
        step1 = np.abs(gb[r, b].astype(np.int64) - ob[r, b].astype(np.int64)) == 1
        sf32 = ref["sf"][r, b].astype(np.float32).astype(np.float64)
        near = near_power_of_two(sf32) if scale_format == "ue8m0" else near_midpoint("e4m3fn", sf32)
        if not np.all(step1 & near):
            k = np.nonzero(~(step1 & near))[0][:4]
            raise AssertionError(f"block scales differ away from a boundary at {list(zip(r[k], b[k]))}: "
                                 f"gpu {gb[r[k], b[k]]} oracle {ob[r[k], b[k]]} sf {ref['sf'][r[k], b[k]]}")
        gs = float(np.float32(global_scale))
        y = _y(y)
        for rr, bb in zip(r, b):
            sl = slice(block_size * bb, block_size * (bb + 1))
            if scale_format == "ue8m0":
                sg = int(gb[rr, bb])
                q[rr, sl] = y[rr, sl] * (np.ldexp(1.0, 127 - sg) if sg else 0.0)
            else:
                dg = oracle.decode("e4m3fn", [gb[rr, bb]])[0]
                q[rr, sl] = y[rr, sl] * gs / dg if dg > 0 else y[rr, sl] * 0.0
            expect[rr, sl] = oracle.encode("e2m1", q[rr, sl].astype(np.float32).astype(np.float64))
    rep["block_scale_total"] = int(gb.size)
    if cap:
        check_cap(rep["block_scale_boundary"], gb.size, "block scales")
    _check_codes("e2m1", unpack_e2m1(gpu_packed), expect, q, rep, "codes", cap)
    rep["ok"] = True
    return rep


def unswizzle_scales(buf, rows, sf_per_row):
    """Row-major [rows, sf_per_row] view of a swizzled scale buffer (the
    oracle's offsets), and a mask of the buffer bytes that hold no scale."""
    buf = np.asarray(buf, np.uint8)
    r, c = np.meshgrid(np.arange(rows), np.arange(sf_per_row), indexing="ij")
    off = oracle.swizzled_offset(r, c, sf_per_row)
    pad = np.ones(buf.size, bool)
    pad[off.ravel()] = False
    return buf[off], pad
