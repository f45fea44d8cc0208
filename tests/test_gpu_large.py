"""GPU: tensors past 4 GiB, on sampled rows against the oracle.

Row tensors of more than 2^32 bytes check that every byte offset is formed
in 64 bits (an offset wrapped at 2^31 or 2^32 would read or write another
row).  The inputs are built on the device from a seeded block of 61 host rows:
row i is block row i % 61 times 2^((i // 61) % 17 - 8) (exact in every input
type), with two elements replaced by the tags 1 + (i % 127) / 128 and
1 + ((i // 127) % 127) / 128.  Together with i % 61 the tags fix i modulo
61 * 127^2 = 983,869, more rows than any tensor here holds, so every row is
distinct and a row read in place of another shows in the result.  The host
rebuilds the sampled rows the same way, including the rows on either side of
each 2^31- and 2^32-byte boundary of every row tensor.
"""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import oracle
import workloads
from gpu_common import DEV, say
from parity import compare_fp4, compare_fp8

pytestmark = pytest.mark.gpu
TD = workloads.TORCH_DTYPES
BLOCK_ROWS = 61


class Tiled:
    """A [rows, hidden] tensor on the device built from a seeded block."""

    def __init__(self, rows, hidden, dt, seed, tag_cols):
        rng = np.random.default_rng(seed)
        self.block = torch.from_numpy(rng.standard_normal((BLOCK_ROWS, hidden))).to(TD[dt])
        self.rows, self.hidden, self.dt, self.tag_cols = rows, hidden, dt, tag_cols
        self.dev = torch.empty((rows, hidden), dtype=TD[dt], device=DEV)
        dblock = self.block.to(DEV)
        chunk = BLOCK_ROWS * 64
        reps = dblock.repeat(64, 1)
        for r0 in range(0, rows, chunk):
            n = min(chunk, rows - r0)
            i = torch.arange(r0, r0 + n, device=DEV)
            self.dev[r0:r0 + n] = reps[:n] * self._scale(i)[:, None]
        i = torch.arange(rows, device=DEV)
        for col, tag in zip(tag_cols, self._tags(i)):
            self.dev[:, col] = tag.to(TD[dt])

    @staticmethod
    def _scale(i):
        return torch.exp2(((i // BLOCK_ROWS) % 17 - 8).to(torch.float32))

    @staticmethod
    def _tags(i):
        return (1.0 + (i % 127).to(torch.float32) / 128.0, 1.0 + ((i // 127) % 127).to(torch.float32) / 128.0)

    def host_rows(self, idx):
        i = torch.as_tensor(idx, dtype=torch.int64)
        t = self.block[i % BLOCK_ROWS].to(torch.float32) * self._scale(i)[:, None]
        for col, tag in zip(self.tag_cols, self._tags(i)):
            t[:, col] = tag
        return t.to(TD[self.dt])


def boundary_rows(rows, row_bytes_list, seed, k=8):
    """Rows on either side of each 2^31 / 2^32 byte boundary of tensors with
    these row sizes, the first and last row, and k random rows."""
    pick = {0, rows - 1}
    for b in row_bytes_list:
        for edge in (1 << 31, 1 << 32):
            r = edge // b
            pick.update(v for v in (r - 1, r, r + 1) if 0 <= v < rows)
    pick.update(int(v) for v in np.random.default_rng(seed).choice(rows, k, replace=False))
    return np.array(sorted(pick), np.int64)


def rows_past_4gib(hidden, esz, extra):
    """Rows of hidden elements of esz bytes that take more than 2^32 bytes."""
    return (1 << 32) // (hidden * esz) + extra


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_residual_fp8_past_4gib():
    hidden = 8192
    rows = rows_past_4gib(hidden, 2, 1037)
    x = Tiled(rows, hidden, "bf16", 1, tag_cols=(5, 4000))
    r = Tiled(rows, hidden, "bf16", 2, tag_cols=(hidden - 3, 77))
    g = torch.from_numpy(np.random.default_rng(3).uniform(0.5, 1.5, hidden)).to(torch.bfloat16)
    say(f"[large] residual FP8 bf16 {rows}x{hidden} ({rows * hidden * 2 / 2**30:.2f} GiB per tensor)")
    codes, scales, ro = rq.residual_rmsnorm_fp8(x.dev, r.dev, g.to(DEV), eps=1e-6, scale_ub=1200.0)
    torch.cuda.synchronize()
    idx = boundary_rows(rows, [hidden * 2, hidden], seed=4)
    sel = torch.as_tensor(idx, device=DEV)
    hx, hr = workloads.bits(x.host_rows(idx)), workloads.bits(r.host_rows(idx))
    ref = oracle.rmsnorm_fp8(hx, workloads.bits(g), residual=hr, in_dtype="bf16", eps=1e-6, weight_offset=0.0,
                             scale_ub=1200.0, out_fmt="e4m3fn", scales_dtype="f32")
    y = oracle.rmsnorm_y(hx, workloads.bits(g), residual=hr, in_dtype="bf16", eps=1e-6, weight_offset=0.0)["y"]
    rep = compare_fp8(codes[sel].cpu().numpy(), workloads.bits(scales[sel].cpu()), ref, y, out_fmt="e4m3fn",
                      scales_dtype="f32", gpu_residual_out=workloads.bits(ro[sel].cpu()))
    say(f"  parity rows {idx.tolist()}: {rep}")
    del x, r, codes, scales, ro
    free()


@pytest.mark.parametrize("resid,hidden", [(False, 65536), (True, 65536), (True, 49152)],
                         ids=["registers", "lds", "registers-residual"])
def test_wide_fp8_past_4gib(resid, hidden):
    """Wide rows: 65536 (128 KiB each) held in registers without a residual
    and staged in LDS with one (8 vectors per lane); 49152 with a residual
    held in registers (6 vectors per lane)."""
    rows = rows_past_4gib(hidden, 2, 37)
    x = Tiled(rows, hidden, "bf16", 40, tag_cols=(3, hidden - 15536))  # column 50000 of a 65536 row
    r = Tiled(rows, hidden, "bf16", 41, tag_cols=(hidden - 1, 1234)) if resid else None
    g = torch.from_numpy(np.random.default_rng(42).uniform(0.5, 1.5, hidden)).to(torch.bfloat16)
    say(f"[large] wide FP8 bf16 {rows}x{hidden} residual={resid} ({rows * hidden * 2 / 2**30:.2f} GiB per tensor)")
    if resid:
        codes, scales, ro = rq.residual_rmsnorm_fp8(x.dev, r.dev, g.to(DEV), eps=1e-6, scale_ub=1200.0)
    else:
        codes, scales = rq.rmsnorm_fp8(x.dev, g.to(DEV), eps=1e-6, scale_ub=1200.0)
        ro = None
    torch.cuda.synchronize()
    idx = boundary_rows(rows, [hidden * 2, hidden], seed=43)
    sel = torch.as_tensor(idx, device=DEV)
    hx = workloads.bits(x.host_rows(idx))
    hr = workloads.bits(r.host_rows(idx)) if resid else None
    kw = dict(in_dtype="bf16", eps=1e-6, weight_offset=0.0)
    ref = oracle.rmsnorm_fp8(hx, workloads.bits(g), residual=hr, scale_ub=1200.0, out_fmt="e4m3fn",
                             scales_dtype="f32", **kw)
    y = oracle.rmsnorm_y(hx, workloads.bits(g), residual=hr, **kw)["y"]
    rep = compare_fp8(codes[sel].cpu().numpy(), workloads.bits(scales[sel].cpu()), ref, y, out_fmt="e4m3fn",
                      scales_dtype="f32", gpu_residual_out=workloads.bits(ro[sel].cpu()) if resid else None)
    say(f"  parity rows {idx.tolist()}: {rep}")
    del x, r, codes, scales, ro
    free()


def test_wide_fp4_past_4gib():
    """65536-wide rows without a residual (registers), FP4 with E4M3 scales."""
    hidden = 65536
    rows = rows_past_4gib(hidden, 2, 53)
    x = Tiled(rows, hidden, "bf16", 44, tag_cols=(11, 60000))
    g = torch.from_numpy(np.random.default_rng(45).uniform(0.5, 1.5, hidden)).to(torch.bfloat16)
    gst = torch.tensor([64.0], dtype=torch.float32, device=DEV)
    say(f"[large] wide FP4 bf16 {rows}x{hidden}")
    packed, bs = rq.rmsnorm_fp4quant(x.dev, g.to(DEV), eps=1e-6, global_scale=gst)
    torch.cuda.synchronize()
    idx = boundary_rows(rows, [hidden * 2, hidden // 2], seed=46)
    sel = torch.as_tensor(idx, device=DEV)
    hx = workloads.bits(x.host_rows(idx))
    kwo = dict(in_dtype="bf16", eps=1e-6, weight_offset=0.0)
    ref = oracle.rmsnorm_fp4(hx, workloads.bits(g), global_scale=64.0, **kwo)
    y = oracle.rmsnorm_y(hx, workloads.bits(g), **kwo)["y"]
    rep = compare_fp4(packed[sel].cpu().numpy(), bs[sel].cpu().numpy(), ref, y, global_scale=64.0)
    say(f"  parity rows {idx.tolist()}: {rep}")
    del x, packed, bs
    free()


def test_summed_inputs_fp8_past_4gib():
    hidden = 8192
    rows = rows_past_4gib(hidden, 2, 61)
    ins = [Tiled(rows, hidden, "bf16", 10 + k, tag_cols=(7 * k + 1, 5000 + k)) for k in range(2)]
    r = Tiled(rows, hidden, "bf16", 12, tag_cols=(100, 8000))
    g = torch.from_numpy(np.random.default_rng(13).uniform(0.5, 1.5, hidden)).to(torch.bfloat16)
    say(f"[large] 2 summed inputs + residual FP8 bf16 {rows}x{hidden}")
    codes, scales, ro = rq.allreduce_residual_rmsnorm_fp8([t.dev for t in ins], r.dev, g.to(DEV), eps=1e-6,
                                                          scale_ub=1200.0)
    torch.cuda.synchronize()
    idx = boundary_rows(rows, [hidden * 2, hidden], seed=14)
    sel = torch.as_tensor(idx, device=DEV)
    hins = [workloads.bits(t.host_rows(idx)) for t in ins]
    ref = oracle.allreduce_residual_rmsnorm_fp8(hins, workloads.bits(r.host_rows(idx)), workloads.bits(g),
                                                in_dtype="bf16", eps=1e-6, weight_offset=0.0, scale_ub=1200.0,
                                                out_fmt="e4m3fn", scales_dtype="f32")
    y = oracle.rmsnorm_y(ref["residual_out"], workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0.0)["y"]
    rep = compare_fp8(codes[sel].cpu().numpy(), workloads.bits(scales[sel].cpu()), ref, y, out_fmt="e4m3fn",
                      scales_dtype="f32", gpu_residual_out=workloads.bits(ro[sel].cpu()))
    say(f"  parity rows {idx.tolist()}: {rep}")
    del ins, r, codes, scales, ro
    free()


def test_phased_fp8_past_4gib():
    # 8191 elements per row: rows start at every 2-byte phase of the 16-byte
    # grid (the phased kernel)
    hidden = 8191
    rows = rows_past_4gib(hidden, 2, 300)
    x = Tiled(rows, hidden, "bf16", 20, tag_cols=(hidden - 1, 0))
    g = torch.from_numpy(np.random.default_rng(21).uniform(0.5, 1.5, hidden)).to(torch.bfloat16)
    say(f"[large] FP8 bf16 phased rows {rows}x{hidden}")
    codes, scales = rq.rmsnorm_fp8(x.dev, g.to(DEV), eps=1e-6, scale_ub=1200.0, out_fp8="e4m3fnuz",
                                   scales_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = boundary_rows(rows, [hidden * 2, hidden], seed=22)
    sel = torch.as_tensor(idx, device=DEV)
    hx = workloads.bits(x.host_rows(idx))
    ref = oracle.rmsnorm_fp8(hx, workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0.0, scale_ub=1200.0,
                             out_fmt="e4m3fnuz", scales_dtype="bf16")
    y = oracle.rmsnorm_y(hx, workloads.bits(g), in_dtype="bf16", eps=1e-6, weight_offset=0.0)["y"]
    rep = compare_fp8(codes[sel].cpu().numpy(), workloads.bits(scales[sel].cpu()), ref, y, out_fmt="e4m3fnuz",
                      scales_dtype="bf16")
    say(f"  parity rows {idx.tolist()}: {rep}")
    del x, codes, scales
    free()


def test_elementwise_fp8_past_4gib():
    # gamma one element off the 16-byte grid: the element-wise kernel
    hidden = 8192
    rows = rows_past_4gib(hidden, 2, 555)
    x = Tiled(rows, hidden, "bf16", 40, tag_cols=(3, 6000))
    r = Tiled(rows, hidden, "bf16", 41, tag_cols=(4, 6001))
    g = torch.from_numpy(np.random.default_rng(42).uniform(0.5, 1.5, hidden)).to(torch.bfloat16)
    gbuf = torch.empty(hidden + 8, dtype=torch.bfloat16, device=DEV)
    dg = gbuf[1:1 + hidden]
    dg.copy_(g.to(DEV))
    assert dg.data_ptr() % 16 == 2
    say(f"[large] residual FP8 bf16 element-wise {rows}x{hidden}")
    codes, scales, ro = rq.residual_rmsnorm_fp8(x.dev, r.dev, dg, eps=1e-6, scale_ub=1200.0, out_fp8="e4m3fnuz",
                                                scales_dtype=torch.float16)
    torch.cuda.synchronize()
    idx = boundary_rows(rows, [hidden * 2, hidden], seed=43)
    sel = torch.as_tensor(idx, device=DEV)
    hx, hr = workloads.bits(x.host_rows(idx)), workloads.bits(r.host_rows(idx))
    ref = oracle.rmsnorm_fp8(hx, workloads.bits(g), residual=hr, in_dtype="bf16", eps=1e-6, weight_offset=0.0,
                             scale_ub=1200.0, out_fmt="e4m3fnuz", scales_dtype="f16")
    y = oracle.rmsnorm_y(hx, workloads.bits(g), residual=hr, in_dtype="bf16", eps=1e-6, weight_offset=0.0)["y"]
    rep = compare_fp8(codes[sel].cpu().numpy(), workloads.bits(scales[sel].cpu()), ref, y, out_fmt="e4m3fnuz",
                      scales_dtype="f16", gpu_residual_out=workloads.bits(ro[sel].cpu()))
    say(f"  parity rows {idx.tolist()}: {rep}")
    del x, r, codes, scales, ro
    free()


@pytest.mark.parametrize("swizzled,resid,block,fmt", [(True, False, 16, "e4m3"), (False, True, 32, "ue8m0")],
                         ids=["swizzled-e4m3-16", "residual-ue8m0-32"])
def test_fp4_past_4gib(swizzled, resid, block, fmt):
    hidden = 7168 if swizzled else 4096
    rows = rows_past_4gib(hidden, 2, 173)
    x = Tiled(rows, hidden, "bf16", 30, tag_cols=(9, 2222))
    r = Tiled(rows, hidden, "bf16", 31, tag_cols=(40, 3333)) if resid else None
    g = torch.from_numpy(np.random.default_rng(32).uniform(0.5, 1.5, hidden)).to(torch.bfloat16)
    gs = 64.0 if fmt == "e4m3" else None
    gst = torch.tensor([gs], dtype=torch.float32, device=DEV) if gs is not None else None
    say(f"[large] FP4 bf16 {rows}x{hidden} swizzled={swizzled} residual={resid} block={block} {fmt}")
    kw = dict(eps=1e-6, global_scale=gst, block_size=block, scale_format=fmt, swizzled=swizzled)
    if resid:
        packed, bs, ro = rq.residual_rmsnorm_fp4quant(x.dev, r.dev, g.to(DEV), **kw)
    else:
        packed, bs = rq.rmsnorm_fp4quant(x.dev, g.to(DEV), **kw)
        ro = None
    torch.cuda.synchronize()
    idx = boundary_rows(rows, [hidden * 2, hidden // 2], seed=33)
    sel = torch.as_tensor(idx, device=DEV)
    nsf = hidden // block
    if swizzled:
        off = oracle.swizzled_offset(idx[:, None], np.arange(nsf)[None, :], nsf)
        gb = bs.cpu().numpy()[off]
    else:
        gb = bs[sel].cpu().numpy()
    hx = workloads.bits(x.host_rows(idx))
    hr = workloads.bits(r.host_rows(idx)) if resid else None
    kwo = dict(in_dtype="bf16", eps=1e-6, weight_offset=0.0)
    ref = oracle.rmsnorm_fp4(hx, workloads.bits(g), global_scale=1.0 if gs is None else gs, block_size=block,
                             scale_format=fmt, residual=hr, **kwo)
    if resid:
        assert np.array_equal(workloads.bits(ro[sel].cpu()), ref["residual_out"])
    y = oracle.rmsnorm_y(hx, workloads.bits(g), residual=hr, **kwo)["y"]
    rep = compare_fp4(packed[sel].cpu().numpy(), gb, ref, y, global_scale=1.0 if gs is None else gs,
                      block_size=block, scale_format=fmt)
    say(f"  parity rows {idx.tolist()}: {rep}")
    del x, r, packed, bs, ro
    free()
