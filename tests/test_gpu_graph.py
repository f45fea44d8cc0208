"""GPU: the entry points captured in a HIP graph (as a decode loop would run
them) give, on every replay, the results of an eager call on the same
inputs.  The inputs are rewritten in place between replays, with eager
library calls and synchronizations in between, and each replay is checked.
The FP4 global scale is a device tensor (FlashInfer rmsnorm_fp4quant.py keeps
it on the device so that a captured graph reads the value current at replay
time): it changes between replays too.  The kernels clear no memory, so no
memset node enters a graph."""
import numpy as np
import pytest
import torch

import fp4_activation_quantization_amd as rq
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu
REPLAYS = 3


def _rand(shape, dt, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * (1 + seed % 3)).to(dt).to(DEV)


def _check_replays(name, inputs, make_inputs, run, outputs):
    """inputs: static device tensors the graph reads; make_inputs(i) -> new
    values for them; run(outs) enqueues the call writing into outs (a list of
    tensors like `outputs`)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(outputs)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(outputs)
    eager = [torch.empty_like(t) for t in outputs]
    for i in range(REPLAYS):
        for t, v in zip(inputs, make_inputs(i)):
            t.copy_(v)
        run(eager)
        torch.cuda.synchronize()
        for t in outputs:
            t.fill_(0x5A if t.dtype == torch.uint8 else 7)
        graph.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(outputs, eager)):
            assert torch.equal(got, want), f"{name}: replay {i}, output {k} differs from the eager call"
    say(f"[graph] {name}: {REPLAYS} replays equal the eager calls")
    del graph


@pytest.mark.parametrize("rows,hidden", [(1, 8192), (64, 8192), (300, 4095)], ids=["1x8192", "64x8192", "300x4095"])
def test_rmsnorm_fp8(rows, hidden):
    x = _rand((rows, hidden), torch.float16, 1)
    g = _rand((hidden,), torch.float16, 2)
    out = torch.empty((rows, hidden), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows,), dtype=torch.bfloat16, device=DEV)

    def run(o):
        rq.rmsnorm_fp8(x, g, weight_offset=1.0, scale_ub=1e4, out_fp8="e4m3fnuz", out=o[0], scales=o[1],
                       scales_dtype=torch.bfloat16)

    _check_replays(f"rmsnorm_fp8 {rows}x{hidden}", [x], lambda i: [_rand((rows, hidden), torch.float16, 10 + i)],
                   run, [out, sc])


def test_residual_rmsnorm_fp8():
    rows, hidden = 64, 4096
    x = _rand((rows, hidden), torch.bfloat16, 3)
    r = _rand((rows, hidden), torch.bfloat16, 4)
    g = _rand((hidden,), torch.bfloat16, 5)
    out = torch.empty((rows, hidden), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows,), dtype=torch.float32, device=DEV)
    ro = torch.empty_like(r)

    def run(o):
        rq.residual_rmsnorm_fp8(x, r, g, scale_ub=1200.0, out=o[0], scales=o[1], residual_out=o[2])

    _check_replays("residual_rmsnorm_fp8", [x, r],
                   lambda i: [_rand((rows, hidden), torch.bfloat16, 20 + i), _rand((rows, hidden), torch.bfloat16, 30 + i)],
                   run, [out, sc, ro])


@pytest.mark.parametrize("swizzled", [False, True], ids=["rowmajor", "swizzled"])
def test_rmsnorm_fp4quant_device_global_scale(swizzled):
    rows, hidden = 128, 7168  # whole 128 x 4 scale tiles: no padding bytes to compare
    x = _rand((rows, hidden), torch.bfloat16, 6)
    g = _rand((hidden,), torch.bfloat16, 7)
    gs = torch.tensor([100.0], dtype=torch.float32, device=DEV)
    out = torch.empty((rows, hidden // 2), dtype=torch.uint8, device=DEV)
    nbs = rq.fp4_scale_bytes(rows, hidden, 16, swizzled)
    bs = torch.zeros((nbs,) if swizzled else (rows, hidden // 16), dtype=torch.uint8, device=DEV)

    def run(o):
        rq.rmsnorm_fp4quant(x, g, global_scale=gs, block_size=16, scale_format="e4m3", swizzled=swizzled,
                            out=o[0], block_scales=o[1])

    def inputs(i):
        return [_rand((rows, hidden), torch.bfloat16, 40 + i), torch.tensor([50.0 * (i + 1)], device=DEV)]

    _check_replays(f"rmsnorm_fp4quant swizzled={swizzled}", [x, gs], inputs, run, [out, bs])


def test_residual_fp4_and_summed_inputs():
    rows, hidden = 48, 2048
    x = _rand((rows, hidden), torch.bfloat16, 8)
    r = _rand((rows, hidden), torch.bfloat16, 9)
    g = _rand((hidden,), torch.bfloat16, 11)
    outs = [torch.empty((rows, hidden // 2), dtype=torch.uint8, device=DEV),
            torch.empty((rows, hidden // 32), dtype=torch.uint8, device=DEV), torch.empty_like(r)]

    def run_fp4(o):
        rq.residual_rmsnorm_fp4quant(x, r, g, block_size=32, scale_format="ue8m0", out=o[0], block_scales=o[1],
                                     residual_out=o[2])

    _check_replays("residual_rmsnorm_fp4quant", [x, r],
                   lambda i: [_rand((rows, hidden), torch.bfloat16, 50 + i), _rand((rows, hidden), torch.bfloat16, 60 + i)],
                   run_fp4, outs)

    ins = [_rand((rows, hidden), torch.bfloat16, 70 + k) for k in range(4)]
    outs8 = [torch.empty((rows, hidden), dtype=torch.uint8, device=DEV),
             torch.empty((rows,), dtype=torch.float32, device=DEV), torch.empty_like(r)]

    def run_sum(o):
        rq.allreduce_residual_rmsnorm_fp8(ins, r, g, scale_ub=1200.0, out=o[0], scales=o[1], residual_out=o[2])

    _check_replays("allreduce_residual_rmsnorm_fp8", ins + [r],
                   lambda i: [_rand((rows, hidden), torch.bfloat16, 80 + 10 * i + k) for k in range(5)],
                   run_sum, outs8)


@pytest.mark.parametrize("resid,hidden", [(False, 65536), (True, 65536), (True, 49152)],
                         ids=["registers", "lds", "registers-residual"])
def test_wide_rows(resid, hidden):
    """Rows above 4096 vectors: held in registers with gamma in LDS (65536
    without a residual, 49152 with one) or staged in LDS (65536 with a
    residual); every launch raises the kernel's dynamic-LDS limit and queries
    occupancy, host calls made during capture."""
    rows = 40
    x = _rand((rows, hidden), torch.bfloat16, 13)
    r = _rand((rows, hidden), torch.bfloat16, 14) if resid else None
    g = _rand((hidden,), torch.bfloat16, 15)
    outs8 = [torch.empty((rows, hidden), dtype=torch.uint8, device=DEV),
             torch.empty((rows,), dtype=torch.float32, device=DEV)] + ([torch.empty_like(x)] if resid else [])
    gs = torch.tensor([30.0], dtype=torch.float32, device=DEV)
    outs4 = [torch.empty((rows, hidden // 2), dtype=torch.uint8, device=DEV),
             torch.empty((rows, hidden // 16), dtype=torch.uint8, device=DEV)] + ([torch.empty_like(x)] if resid else [])

    def run8(o):
        if resid:
            rq.residual_rmsnorm_fp8(x, r, g, scale_ub=1200.0, out=o[0], scales=o[1], residual_out=o[2])
        else:
            rq.rmsnorm_fp8(x, g, scale_ub=1200.0, out=o[0], scales=o[1])

    def run4(o):
        if resid:
            rq.residual_rmsnorm_fp4quant(x, r, g, global_scale=gs, out=o[0], block_scales=o[1], residual_out=o[2])
        else:
            rq.rmsnorm_fp4quant(x, g, global_scale=gs, out=o[0], block_scales=o[1])

    ins = [x] + ([r] if resid else [])

    def inputs(i):
        return [_rand((rows, hidden), torch.bfloat16, 90 + 10 * i + k) for k in range(len(ins))]

    _check_replays(f"wide rmsnorm_fp8 resid={resid}", ins, inputs, run8, outs8)
    _check_replays(f"wide rmsnorm_fp4quant resid={resid}", ins, inputs, run4, outs4)


def test_replays_follow_the_global_scale():
    """The stored E4M3 block scales of a replay track the device global scale
    written after capture: doubling gs doubles every unsaturated stored scale
    (or leaves it saturated at 448 = 0x7E)."""
    rows, hidden = 8, 1024
    x = _rand((rows, hidden), torch.bfloat16, 12)
    g = torch.ones(hidden, dtype=torch.bfloat16, device=DEV)
    gs = torch.tensor([1.0], dtype=torch.float32, device=DEV)
    out = torch.empty((rows, hidden // 2), dtype=torch.uint8, device=DEV)
    bs = torch.empty((rows, hidden // 16), dtype=torch.uint8, device=DEV)
    rq.rmsnorm_fp4quant(x, g, global_scale=gs, out=out, block_scales=bs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rq.rmsnorm_fp4quant(x, g, global_scale=gs, out=out, block_scales=bs)
    graph.replay()
    torch.cuda.synchronize()
    s1 = bs.cpu().numpy().copy()
    gs.fill_(2.0)
    graph.replay()
    torch.cuda.synchronize()
    s2 = bs.cpu().numpy()
    # E4M3FN codes of normal values: doubling adds 8 to the code (one exponent step)
    normal = (s1 >= 0x08) & (s1 + 8 <= 0x7E)
    assert normal.any()
    assert np.array_equal(s2[normal], s1[normal] + 8)
    del graph
