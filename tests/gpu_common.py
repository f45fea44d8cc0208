"""Helpers for the GPU tests: run the library through its binding (C ABI) on
seeded inputs and check the result against the oracle with the comparator."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp4_activation_quantization_amd as rq
import oracle
import workloads
from parity import check_cap, compare_fp4, compare_fp8, unswizzle_scales

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(t):
    return None if t is None else t.to(DEV)


def run_fp8(w, inp, *, rows_idx=None, ub=None, out_fmt=None, scales_dtype=None, weight_offset=None,
            in_place=None, stream=None):
    """Run the FP8 path on the GPU; returns host numpy (codes, scale bits, residual_out bits) for
    rows_idx (all rows if None) plus the torch outputs."""
    out_fmt = out_fmt or w.out_fmt
    sdt = scales_dtype or w.scales_dtype
    ub = w.scale_ub if ub is None else ub
    off = w.weight_offset if weight_offset is None else weight_offset
    x, g = to_dev(inp["x"]), to_dev(inp["gamma"])
    sc_t = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[sdt]
    if w.ninputs > 1:
        r = to_dev(inp["residual"])
        codes, scales, rout = rq.allreduce_residual_rmsnorm_fp8(
            [to_dev(t) for t in inp["inputs"]], r, g, eps=w.eps, weight_offset=off, scale_ub=ub, out_fp8=out_fmt,
            scales_dtype=sc_t, residual_out=r if in_place == "residual" else None, stream=stream)
    elif inp.get("residual") is not None:
        r = to_dev(inp["residual"])
        ro = None
        if in_place == "x":
            ro = x
        elif in_place == "residual":
            ro = r
        codes, scales, rout = rq.residual_rmsnorm_fp8(x, r, g, eps=w.eps, weight_offset=off, scale_ub=ub,
                                                      out_fp8=out_fmt, scales_dtype=sc_t, residual_out=ro,
                                                      stream=stream)
    else:
        codes, scales = rq.rmsnorm_fp8(x, g, eps=w.eps, weight_offset=off, scale_ub=ub, out_fp8=out_fmt,
                                       scales_dtype=sc_t, stream=stream)
        rout = None
    torch.cuda.synchronize()
    sel = slice(None) if rows_idx is None else torch.as_tensor(rows_idx, device=DEV)
    c = codes[sel].cpu().numpy()
    s = workloads.bits(scales[sel].cpu())
    ro = workloads.bits(rout[sel].cpu()) if rout is not None else None
    return c, s, ro


def oracle_fp8(w, inp, *, rows_idx=None, ub=None, out_fmt=None, scales_dtype=None, weight_offset=None):
    x = workloads.bits(inp["x"])
    r = workloads.bits(inp["residual"]) if inp.get("residual") is not None else None
    if rows_idx is not None:
        x = x[rows_idx]
        r = r[rows_idx] if r is not None else None
    g = workloads.bits(inp["gamma"])
    kw = dict(in_dtype=w.in_dtype, eps=w.eps, weight_offset=w.weight_offset if weight_offset is None else weight_offset)
    q = dict(scale_ub=w.scale_ub if ub is None else ub, out_fmt=out_fmt or w.out_fmt,
             scales_dtype=scales_dtype or w.scales_dtype)
    if w.ninputs > 1:
        ins = [workloads.bits(t) for t in inp["inputs"]]
        if rows_idx is not None:
            ins = [t[rows_idx] for t in ins]
        ref = oracle.allreduce_residual_rmsnorm_fp8(ins, r, g, **q, **kw)
        return ref, _lazy(lambda: oracle.rmsnorm_y(ref["residual_out"], g, **kw)["y"])
    ref = oracle.rmsnorm_fp8(x, g, residual=r, **q, **kw)
    return ref, _lazy(lambda: oracle.rmsnorm_y(x, g, residual=r, round_product=w.fp4_round_product, **kw)["y"])


def _lazy(fn):
    """The oracle's y for the same rows, computed on first use only (the
    comparator needs it where a 16-bit or block scale differs)."""
    memo = []

    def get():
        if not memo:
            memo.append(fn())
        return memo[0]
    return get


def check_fp8(w, inp, *, rows_idx=None, label="", **kw):
    c, s, ro = run_fp8(w, inp, rows_idx=rows_idx, **kw)
    kw.pop("in_place", None)
    kw.pop("stream", None)
    ref, y = oracle_fp8(w, inp, rows_idx=rows_idx, **kw)
    rep = compare_fp8(c, s, ref, y, out_fmt=kw.get("out_fmt") or w.out_fmt,
                      scales_dtype=kw.get("scales_dtype") or w.scales_dtype, gpu_residual_out=ro)
    say(f"  parity {label or w.name}: {rep}")
    return rep


CANARY = 0xA5  # fill of swizzled scale buffers: padding bytes must keep it


def run_fp4(w, inp, gs, *, rows_idx=None, weight_offset=None, stream=None):
    """Run the workload's FP4 variant; returns (packed, row-major block scales,
    residual_out or None) for the selected rows.  A swizzled buffer is checked
    to leave its padding untouched and is returned un-swizzled."""
    x, g = to_dev(inp["x"]), to_dev(inp["gamma"])
    gst = torch.tensor([gs], dtype=torch.float32, device=DEV) if gs is not None else None
    off = w.weight_offset if weight_offset is None else weight_offset
    rows, hidden = x.shape
    bs = None
    if w.fp4_swizzled:
        bs = torch.full((rq.fp4_scale_bytes(rows, hidden, w.fp4_block, True),), CANARY, dtype=torch.uint8,
                        device=DEV)
    kw = dict(eps=w.eps, weight_offset=off, global_scale=gst, block_size=w.fp4_block, scale_format=w.fp4_scale,
              swizzled=w.fp4_swizzled, block_scales=bs, stream=stream, round_product=w.fp4_round_product)
    ro = None
    if w.residual:
        packed, bs, ro = rq.residual_rmsnorm_fp4quant(x, to_dev(inp["residual"]), g, **kw)
    elif w.fp4_block == 16 and w.fp4_scale == "e4m3" and not w.fp4_swizzled and not w.fp4_round_product:
        packed, bs = rq.rmsnorm_fp4(x, g, eps=w.eps, weight_offset=off, global_scale=gst, stream=stream)
    else:
        packed, bs = rq.rmsnorm_fp4quant(x, g, **kw)
    torch.cuda.synchronize()
    bs = bs.cpu().numpy()
    if w.fp4_swizzled:
        raw = bs
        bs, pad = unswizzle_scales(raw, rows, hidden // w.fp4_block)
        assert np.all(raw[pad] == CANARY), "swizzled padding bytes were written"
    sel = slice(None) if rows_idx is None else np.asarray(rows_idx)
    ro = workloads.bits(ro.cpu())[sel] if ro is not None else None
    return packed.cpu().numpy()[sel], bs[sel], ro


def check_fp4(w, inp, gs, *, rows_idx=None, label="", weight_offset=None):
    p, bs, ro = run_fp4(w, inp, gs, rows_idx=rows_idx, weight_offset=weight_offset)
    x = workloads.bits(inp["x"])
    r = workloads.bits(inp["residual"]) if w.residual else None
    if rows_idx is not None:
        x = x[rows_idx]
        r = r[rows_idx] if r is not None else None
    g = workloads.bits(inp["gamma"])
    off = w.weight_offset if weight_offset is None else weight_offset
    kw = dict(in_dtype=w.in_dtype, eps=w.eps, weight_offset=off)
    gsv = 1.0 if gs is None else gs
    ref = oracle.rmsnorm_fp4(x, g, global_scale=gsv, block_size=w.fp4_block, scale_format=w.fp4_scale, residual=r,
                             round_product=w.fp4_round_product, **kw)
    if r is not None:
        assert np.array_equal(ro, ref["residual_out"]), "residual_out differs from the oracle's"
    y = _lazy(lambda: oracle.rmsnorm_y(x, g, residual=r, round_product=w.fp4_round_product, **kw)["y"])
    rep = compare_fp4(p, bs, ref, y, global_scale=gsv, block_size=w.fp4_block, scale_format=w.fp4_scale)
    say(f"  parity {label or w.name}: {rep}")
    return rep


_SUMMED = ("codes_total", "codes_boundary", "codes_boundary_ties", "block_scale_total", "block_scale_boundary",
           "scale_boundary_rows")


def check_whole(w, inp, gs=None, *, chunk_rows=2048, label=""):
    """Every row of a workload at its full size: one call of the library on
    the whole tensor (its automatic launch shape, the one the benchmark
    times), then the oracle over row chunks, every element compared.  The
    boundary flips of all chunks together must be at most 0.01% of the
    tensor's codes (and of its 16-bit or block scales)."""
    rows = w.rows
    if w.fp4:
        p_all, bs_all, ro_all = run_fp4(w, inp, gs)
    else:
        c_all, s_all, ro_all = run_fp8(w, inp)
    tot = {k: 0 for k in _SUMMED}
    scale_rel = 0.0
    g = workloads.bits(inp["gamma"])
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        sl = slice(r0, r1)
        if w.fp4:
            x = workloads.bits(inp["x"][sl])
            r = workloads.bits(inp["residual"][sl]) if w.residual else None
            kw = dict(in_dtype=w.in_dtype, eps=w.eps, weight_offset=w.weight_offset)
            ref = oracle.rmsnorm_fp4(x, g, global_scale=1.0 if gs is None else gs, block_size=w.fp4_block,
                                     scale_format=w.fp4_scale, residual=r, round_product=w.fp4_round_product, **kw)
            if r is not None:
                assert np.array_equal(ro_all[sl], ref["residual_out"]), f"residual_out differs in rows {r0}..{r1}"
            y = _lazy(lambda: oracle.rmsnorm_y(x, g, residual=r, round_product=w.fp4_round_product, **kw)["y"])
            rep = compare_fp4(p_all[sl], bs_all[sl], ref, y, global_scale=1.0 if gs is None else gs,
                              block_size=w.fp4_block, scale_format=w.fp4_scale, cap=False)
        else:
            part = dict(inp, x=inp["x"][sl])
            if inp.get("residual") is not None:
                part["residual"] = inp["residual"][sl]
            if w.ninputs > 1:
                part["inputs"] = [t[sl] for t in inp["inputs"]]
            ref, y = oracle_fp8(w, part)
            rep = compare_fp8(c_all[sl], s_all[sl], ref, y, out_fmt=w.out_fmt, scales_dtype=w.scales_dtype,
                              gpu_residual_out=ro_all[sl] if ro_all is not None else None, cap=False)
            scale_rel = max(scale_rel, rep.get("scale_max_rel", 0.0))
        for k in _SUMMED:
            tot[k] += rep.get(k, 0)
        say(f"  [{label or w.name}] rows {r0}..{r1}: codes_boundary {rep['codes_boundary']}")
    frac = tot["codes_boundary"] / max(tot["codes_total"], 1)
    say(f"  whole-tensor parity {label or w.name}: codes_boundary/codes_total = {tot['codes_boundary']}/"
        f"{tot['codes_total']} = {frac:.3g} (ties {tot['codes_boundary_ties']}), "
        f"block_scale_boundary {tot['block_scale_boundary']}/{tot['block_scale_total']}, "
        f"16-bit scale rows {tot['scale_boundary_rows']}, fp32 scale max rel {scale_rel:.3g}")
    check_cap(tot["codes_boundary"], tot["codes_total"], f"{label or w.name} codes")
    if w.fp4:
        check_cap(tot["block_scale_boundary"], tot["block_scale_total"], f"{label or w.name} block scales")
    else:
        check_cap(tot["scale_boundary_rows"], rows, f"{label or w.name} 16-bit scales")
    tot["fraction"] = frac
    return tot


def sample_rows(rows: int, k: int, seed: int, must=()):
    rng = np.random.default_rng(seed)
    pick = set(int(r) for r in must if 0 <= r < rows)
    pick.update([0, rows - 1])
    pick.update(int(v) for v in rng.choice(rows, size=min(k, rows), replace=False))
    return np.array(sorted(pick), np.int64)
