"""GPU: allreduce_residual_rmsnorm_fp8 -- the sum of several input buffers
plus the residual, then RMSNorm + FP8 (Mojo allreduce_residual_rmsnorm_fp8,
on buffers this GPU can read) -- against the oracle (residual_out bit-exact,
codes and scales by the comparator), and the hand rows' sums bit-exact."""
import json
import os

import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
import oracle
import workloads
from gpu_common import DEV, say
from parity import compare_fp8

pytestmark = pytest.mark.gpu
TD = workloads.TORCH_DTYPES
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_rows.json")))
SC = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(autouse=True)
def automatic_shapes():
    rq.set_tuning(0, 0, 0)
    yield
    rq.set_tuning(0, 0, 0)


def _inputs(n, rows, hidden, dt, seed):
    rng = np.random.default_rng(seed)
    mk = lambda: torch.from_numpy(rng.standard_normal((rows, hidden))).to(TD[dt])  # noqa: E731
    ins = [mk() for _ in range(n)]
    return ins, mk(), torch.from_numpy(rng.uniform(0.5, 1.5, hidden)).to(TD[dt])


def run_and_check(ins, r, g, dt, label, out_fmt="e4m3fn", sdt="f32", off=0.0, in_place=False, dev_inputs=None):
    kw = dict(eps=1e-6, weight_offset=off, scale_ub=1200.0)
    dins = dev_inputs if dev_inputs is not None else [t.to(DEV) for t in ins]
    dr = r.to(DEV)
    codes, scales, ro = rq.allreduce_residual_rmsnorm_fp8(dins, dr, g.to(DEV), out_fp8=out_fmt, scales_dtype=SC[sdt],
                                                          residual_out=dr if in_place else None, **kw)
    torch.cuda.synchronize()
    ref = oracle.allreduce_residual_rmsnorm_fp8([workloads.bits(t) for t in ins], workloads.bits(r),
                                                workloads.bits(g), in_dtype=dt, out_fmt=out_fmt, scales_dtype=sdt,
                                                **kw)
    y = oracle.rmsnorm_y(ref["residual_out"], workloads.bits(g), in_dtype=dt, eps=1e-6, weight_offset=off)["y"]
    rep = compare_fp8(codes.cpu().numpy(), workloads.bits(scales.cpu()), ref, y, out_fmt=out_fmt, scales_dtype=sdt,
                      gpu_residual_out=workloads.bits(ro.cpu()))
    say(f"  parity {label}: {rep}")
    return codes, scales, ro


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_inputs_sum_matches_oracle(dt, n):
    # (37, 512): four rows per block at one vector per lane, the last block
    # partly filled; (260, 4096): the large-batch shape, one vector per lane
    for rows, hidden in ((1, 512), (37, 512), (67, 4096), (260, 4096), (300, 1032)):
        ins, r, g = _inputs(n, rows, hidden, dt, seed=n * 100 + rows)
        say(f"[allreduce] {dt} n={n} {rows}x{hidden}")
        run_and_check(ins, r, g, dt, f"{dt} n={n} {rows}x{hidden}")


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_formats_scale_types_offset(fmt, sdt):
    ins, r, g = _inputs(4, 70, 2048, "bf16", seed=9)
    say(f"[allreduce matrix] {fmt} {sdt}")
    run_and_check(ins, r, g, "bf16", f"{fmt} {sdt}", out_fmt=fmt, sdt=sdt, off=0.5)


def test_in_place_and_shared_inputs():
    ins, r, g = _inputs(3, 130, 4096, "bf16", seed=11)
    say("[allreduce] in place over residual")
    run_and_check(ins, r, g, "bf16", "in place", in_place=True)
    # the same buffer passed twice, and the residual passed as an input
    d0, dr = ins[0].to(DEV), r.to(DEV)
    say("[allreduce] shared inputs")
    run_and_check([ins[0], ins[0], r], r, g, "bf16", "shared inputs", dev_inputs=[d0, d0, dr])


def test_one_input_equals_the_residual_path():
    ins, r, g = _inputs(1, 301, 4096, "bf16", seed=13)
    x, dr, dg = ins[0].to(DEV), r.to(DEV), g.to(DEV)
    say("[allreduce] one input vs residual_rmsnorm_fp8")
    c1, s1, ro1 = rq.allreduce_residual_rmsnorm_fp8([x], dr, dg, eps=1e-6, scale_ub=1200.0)
    c2, s2, ro2 = rq.residual_rmsnorm_fp8(x, dr, dg, eps=1e-6, scale_ub=1200.0)
    torch.cuda.synchronize()
    assert torch.equal(ro1, ro2)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


@pytest.mark.parametrize("waves,vpt,blocks", [(2, 4, 0), (4, 2, 0), (4, 4, 0), (8, 1, 0), (16, 1, 0), (4, 2, 7)])
def test_forced_shapes(waves, vpt, blocks):
    ins, r, g = _inputs(3, 203, 4096, "f16", seed=17)
    rq.set_tuning(waves, vpt, blocks)
    say(f"[allreduce shape] {waves}x{vpt} blocks={blocks}")
    run_and_check(ins, r, g, "f16", f"shape {waves}x{vpt}/{blocks}")


@pytest.mark.parametrize("row", GOLDEN["allreduce_rows"], ids=lambda r: r["id"])
def test_hand_rows_bit_exact(row):
    dt = row["in_dtype"]
    epv = 4 if dt == "f32" else 8
    n = len(row["residual"])
    pad = (-n) % epv  # whole 16-byte vectors: pad the row with zeros
    mk = lambda v: torch.tensor([list(v) + [0.0] * pad], dtype=torch.float64).to(TD[dt]).to(DEV)  # noqa: E731
    ins = [mk(v) for v in row["inputs"]]
    r = mk(row["residual"])
    g = torch.ones(n + pad, dtype=TD[dt], device=DEV)
    say(f"[allreduce hand row] {row['id']}")
    _, _, ro = rq.allreduce_residual_rmsnorm_fp8(ins, r, g, eps=1e-6, scale_ub=1200.0)
    torch.cuda.synchronize()
    got = workloads.bits(ro.cpu())[0][:n]
    width = 8 if dt == "f32" else 4
    assert [f"0x{int(b):0{width}X}" for b in np.ravel(got).view(np.uint32 if dt == "f32" else np.uint16)] == \
        row["expect_residual_out_bits"]
