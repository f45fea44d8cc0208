"""GPU: calls on different streams, and from different host threads, run
concurrently without affecting each other's results (include/rmsq.h: calls
are reentrant; concurrent calls on different streams are safe when their
outputs do not overlap).  Each concurrent result must equal the same call
made alone on the default stream."""
import threading

import pytest
import torch

import fp4_activation_quantization_amd as rq
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu


def _rand(shape, dt, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dt).to(DEV)


def _jobs():
    """(name, run(stream) -> outputs) for a mix of entry points and shapes."""
    jobs = []
    # (96, 65536): wide rows, staged in LDS with a residual, in registers without
    for i, (rows, hidden) in enumerate([(512, 4096), (64, 8192), (300, 4095), (1024, 7168), (96, 65536)]):
        x, r = _rand((rows, hidden), torch.bfloat16, 10 * i), _rand((rows, hidden), torch.bfloat16, 10 * i + 1)
        g = _rand((hidden,), torch.bfloat16, 10 * i + 2)
        jobs.append((f"residual_fp8 {rows}x{hidden}",
                     lambda s, x=x, r=r, g=g: rq.residual_rmsnorm_fp8(x, r, g, scale_ub=1200.0, stream=s)))
        if hidden > 32768:
            jobs.append((f"fp8 {rows}x{hidden}", lambda s, x=x, g=g: rq.rmsnorm_fp8(x, g, scale_ub=1200.0, stream=s)))
        if hidden % 16 == 0:
            gs = torch.tensor([64.0], device=DEV)
            nbs = rq.fp4_scale_bytes(rows, hidden, 16, True)

            # a zeroed scale buffer (filled on the call's stream): the tiles'
            # padding bytes are never written and must compare equal
            def fp4_swz(s, x=x, g=g, gs=gs, nbs=nbs):
                bs = torch.zeros((nbs,), dtype=torch.uint8, device=DEV)
                return rq.rmsnorm_fp4quant(x, g, global_scale=gs, swizzled=True, block_scales=bs, stream=s)

            jobs.append((f"fp4 swizzled {rows}x{hidden}", fp4_swz))
            jobs.append((f"residual mxfp4 {rows}x{hidden}",
                         lambda s, x=x, r=r, g=g: rq.residual_rmsnorm_fp4quant(x, r, g, block_size=32, stream=s)))
    return jobs


def _same(a, b):
    return all(torch.equal(u, v) for u, v in zip(a, b))


def test_streams():
    jobs = _jobs()
    want = [run(None) for _, run in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [None] * len(jobs)
    for rep in range(3):
        for k, (_, run) in enumerate(jobs):  # round robin over the streams, all in flight together
            s = streams[(k + rep) % len(streams)]
            with torch.cuda.stream(s):
                got[k] = run(s)
        torch.cuda.synchronize()
        for (name, _), a, b in zip(jobs, got, want):
            assert _same(a, b), f"{name} differs on a side stream (pass {rep})"
    say(f"[streams] {len(jobs)} calls x 3 passes over {len(streams)} streams equal the default-stream results")


def test_host_threads():
    jobs = _jobs()
    want = [run(None) for _, run in jobs]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rep in range(5):
                    outs = [run(s) for _, run in jobs]
                    s.synchronize()
                    for (name, _), a, b in zip(jobs, outs, want):
                        if not _same(a, b):
                            errors.append(f"thread {t}: {name} differs (pass {rep})")
        except Exception as e:  # surfaced below
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors[:5]
    say(f"[threads] 4 host threads x 5 passes of {len(jobs)} calls equal the single-thread results")
