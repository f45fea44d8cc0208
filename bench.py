"""Benchmark of the fused (residual +) RMSNorm + FP8 / FP4 quantization path on one MI355X.

One step = one call of the fused kernel over one batch of seeded synthetic
activations already resident in HBM.  The headline workload is the residual
path at the large-batch 70B-class shape (32768 rows x 8192, bf16 in,
e4m3fn out, fp32 scales, bf16 residual_out); the metric is algorithmic HBM
bytes per second.

Timing of the headline: untimed launches until the GPU has run at least
--settle-ms of them (its clocks settle: a cold start runs the first
milliseconds of launches slower), W untimed warm-up steps, then K
back-to-back steps between two HIP events recorded on the stream the kernel
runs on, bracketed by device synchronizations.  A step is one kernel launch,
so the average step time is the kernel's average launch duration (including
the ~1 us dispatch gap between launches); per-launch event pairs are not
used because they add several microseconds to every launch.  Buffers rotate
through enough independent copies (>= 1 GiB in total) that the 256 MB
Infinity Cache cannot serve a step from a previous one.  Every other
workload is timed after the same settling as the median of --windows
windows of back-to-back launches, each at least --window-ms of GPU time.

Printed: one JSON line.  Other workloads are reported in its "workloads"
object; --workloads selects them (the headline leads when it is selected).
The CPU baseline is the float64 oracle timed on each workload (the whole
tensor or its first rows, bounded), on the CPU share the GPU job has.
--copy-calibration runs only reference kernels of known traffic (the
streaming probe, then a device copy), the references that rocprofv3's
FETCH_SIZE / WRITE_SIZE readings are scaled by.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp4_activation_quantization_amd as rq  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
CACHE_DEFEAT_BYTES = 1 << 30
STREAM_MIN_BYTES = 16 << 20  # smaller workloads are latency-bound: no bandwidth reference
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "fp4_activation_quantization_amd", "csrc")
SC_T = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def kernel_source_hash() -> str:
    """Hash of every source the library is built from (csrc/ and the public
    headers): counter summaries taken on other sources are stale."""
    h = hashlib.sha256()
    inc = os.path.join(ROOT, "include")
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)) + sorted(os.path.join(inc, f)
                                                                             for f in os.listdir(inc))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def algorithmic_split(w: workloads.Workload) -> tuple[int, int]:
    """(bytes read, bytes written): one read of every input element (gamma and
    the global scale once), one write of every output."""
    esz = {"bf16": 2, "f16": 2, "f32": 4}[w.in_dtype]
    n = w.rows * w.hidden
    if w.fp4:
        # the global scale is read only with E4M3 scales; padding of the
        # swizzled scale tiles is not written
        reads = n * esz + w.hidden * esz + (4 if w.fp4_scale == "e4m3" else 0)
        writes = n // 2 + n // w.fp4_block
        if w.residual:
            reads += n * esz   # residual
            writes += n * esz  # residual_out
        return reads, writes
    ssz = {"f32": 4, "bf16": 2, "f16": 2}[w.scales_dtype]
    reads, writes = w.ninputs * n * esz + w.hidden * esz, n + w.rows * ssz
    if w.residual:
        reads += n * esz   # residual
        writes += n * esz  # residual_out
    return reads, writes


def algorithmic_bytes(w: workloads.Workload) -> int:
    """One read of every input element, one write of every output, gamma once."""
    return sum(algorithmic_split(w))


class Case:
    """Device buffers (rotated copies) and pre-marshalled C-ABI arguments for one workload."""

    def __init__(self, w: workloads.Workload, copies: int, gs: float | None):
        inp = workloads.make(w)
        dev = "cuda:0"
        self.w = w
        self.inp = inp  # host tensors (the CPU baseline runs the oracle on them)
        self.gs = gs
        x0 = inp["x"].to(dev)
        g = inp["gamma"].to(dev)
        r0 = inp["residual"].to(dev) if inp["residual"] is not None else None
        self.keep = [g]
        self.outs = []  # tensors the calls write
        self.calls = []
        L = rq.lib()
        dt = {"bf16": rq.BF16, "f16": rq.F16, "f32": rq.F32}[w.in_dtype]
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        ins0 = [t.to(dev) for t in inp["inputs"]] if w.ninputs > 1 else None
        for i in range(copies):
            x = x0 if i == 0 else x0.clone()
            if w.fp4:
                out = torch.empty((w.rows, w.hidden // 2), dtype=torch.uint8, device=dev)
                bs = torch.empty((rq.fp4_scale_bytes(w.rows, w.hidden, w.fp4_block, w.fp4_swizzled),),
                                 dtype=torch.uint8, device=dev)
                gst = torch.tensor([gs], dtype=torch.float32, device=dev)
                self.keep += [x, out, bs, gst]
                self.outs += [out, bs]
                sfmt = rq.SF_UE8M0 if w.fp4_scale == "ue8m0" else rq.SF_E4M3
                layout = rq.SF_SWIZZLED if w.fp4_swizzled else rq.SF_ROW_MAJOR
                if w.residual:
                    r = r0 if i == 0 else r0.clone()
                    ro = torch.empty_like(x)
                    self.keep += [r, ro]
                    self.outs.append(ro)
                    args = (w.rows, w.hidden, dt, P(x), P(r), P(ro), P(g), w.eps, w.weight_offset, P(gst), w.fp4_block,
                            sfmt, layout, 0, P(out), P(bs), stream)
                    self.calls.append((L.residual_rmsnorm_fp4quant, args))
                else:
                    args = (w.rows, w.hidden, dt, P(x), P(g), w.eps, w.weight_offset, P(gst), w.fp4_block, sfmt,
                            layout, 0, P(out), P(bs), stream)
                    self.calls.append((L.rmsnorm_fp4quant, args))
                continue
            out = torch.empty((w.rows, w.hidden), dtype=torch.uint8, device=dev)
            sc = torch.empty((w.rows,), dtype=SC_T[w.scales_dtype], device=dev)
            fmt = {"e4m3fn": rq.E4M3FN, "e4m3fnuz": rq.E4M3FNUZ}[w.out_fmt]
            sdt = {"f32": rq.F32, "bf16": rq.BF16, "f16": rq.F16}[w.scales_dtype]
            if w.ninputs > 1:
                ins = ins0 if i == 0 else [t.clone() for t in ins0]
                r = r0 if i == 0 else r0.clone()
                ro = torch.empty_like(r)
                ptrs = (ctypes.c_void_p * len(ins))(*[P(t) for t in ins])
                self.keep += ins + [r, ro, out, sc, ptrs]
                self.outs += [ro, out, sc]
                args = (w.rows, w.hidden, dt, len(ins), ptrs, P(r), P(ro), P(g), w.eps, w.weight_offset, w.scale_ub,
                        fmt, P(out), sdt, P(sc), stream)
                self.calls.append((L.allreduce_residual_rmsnorm_fp8, args))
            elif w.residual:
                r = r0 if i == 0 else r0.clone()
                ro = torch.empty_like(x)
                self.keep += [x, r, ro, out, sc]
                self.outs += [ro, out, sc]
                args = (w.rows, w.hidden, dt, P(x), P(r), P(ro), P(g), w.eps, w.weight_offset, w.scale_ub, fmt,
                        P(out), sdt, P(sc), stream)
                self.calls.append((L.residual_rmsnorm_fp8, args))
            else:
                self.keep += [x, out, sc]
                self.outs += [out, sc]
                args = (w.rows, w.hidden, dt, P(x), P(g), w.eps, w.weight_offset, w.scale_ub, fmt, P(out), sdt,
                        P(sc), stream)
                self.calls.append((L.rmsnorm_fp8, args))

    def step(self, i: int, stream: ctypes.c_void_p | None = None) -> None:
        fn, args = self.calls[i % len(self.calls)]
        if stream is not None:  # every entry point takes the stream last
            args = args[:-1] + (stream,)
        rc = fn(*args)
        if rc != 0:
            raise rq.RmsqError(fn.__name__, rc, rq.lib().rmsq_last_hip_error())

    def outputs(self) -> list:
        """The device tensors the calls write (for replay checks)."""
        return self.outs


def time_case(case: Case, steps: int, warmup: int) -> dict:
    """W untimed steps, then K back-to-back steps between two HIP events recorded
    on the kernel's stream, bracketed by device synchronizations.  The average
    launch duration is the elapsed time over K: it includes the dispatch gap
    between consecutive kernels (about a microsecond), so it is an upper bound
    on the kernel's own duration."""
    for i in range(warmup):
        case.step(i)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    t0.record()
    for i in range(steps):
        case.step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = t0.elapsed_time(t1)
    per_us = total_ms * 1e3 / steps
    b = algorithmic_bytes(case.w)
    return {"steps": steps, "ms_per_step": total_ms / steps, "wall_s": wall, "launch_us": per_us, "bytes": b,
            "gbps": b / (per_us * 1e-6) / 1e9, "rows_per_s": case.w.rows / (per_us * 1e-6)}


def settle(case: Case, min_ms: float) -> int:
    """Untimed launches until at least min_ms of GPU time has elapsed (in
    chunks timed by events): the GPU's clocks settle before measuring."""
    done, elapsed, chunk = 0, 0.0, 8
    while elapsed < min_ms:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(chunk):
            case.step(done + i)
        t1.record()
        torch.cuda.synchronize()
        elapsed += t0.elapsed_time(t1)
        done += chunk
        chunk = min(chunk * 2, 4096)
    return done


def time_windows(case: Case, window_ms: float, windows: int) -> dict:
    """Median over `windows` windows of back-to-back launches, each at least
    window_ms of GPU time, timed like time_case."""
    probe = time_case(case, 8, 0)["launch_us"]
    n = max(8, int(math.ceil(window_ms * 1e3 / max(probe, 1e-3))))
    per = sorted(time_case(case, n, 0)["launch_us"] for _ in range(windows))
    med = per[len(per) // 2]
    b = algorithmic_bytes(case.w)
    return {"steps": n * windows, "window_launches": n, "windows": windows, "launch_us": med,
            "launch_us_min": per[0], "launch_us_max": per[-1], "ms_per_step": med * 1e-3, "bytes": b,
            "gbps": b / (med * 1e-6) / 1e9, "rows_per_s": case.w.rows / (med * 1e-6)}


def time_graph(case: Case, calls: int, replays: int) -> dict:
    """Per-call GPU time of latency-sized launches without host launch
    overhead: `calls` back-to-back calls captured into one HIP graph (on the
    capture stream), replayed `replays` times between two events.  Each
    replay's outputs are checked against an eager run first."""
    eager = None
    torch.cuda.synchronize()
    for i in range(calls):
        case.step(i)
    torch.cuda.synchronize()
    eager = [t.clone() for t in case.outputs()]
    for t in case.outputs():
        t.fill_(0)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(calls):
                case.step(i, sp)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):  # several replays, each checked against the eager run
        for t in case.outputs():
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(case.outputs(), eager):
            if not torch.equal(t, e):
                raise RuntimeError(f"{case.w.name}: graph replay differs from the eager run")
    # one event per replay boundary: the mean over all replays, and the median
    # of the replays' per-call times (p50)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record()
    for k in range(replays):
        g.replay()
        ev[k + 1].record()
    torch.cuda.synchronize()
    per_us = ev[0].elapsed_time(ev[-1]) * 1e3 / (replays * calls)
    each = sorted(ev[k].elapsed_time(ev[k + 1]) * 1e3 / calls for k in range(replays))
    del g
    return {"graph_us": per_us, "graph_us_p50": each[len(each) // 2], "graph_calls": calls,
            "graph_replays": replays}


def probe_layout(w: workloads.Workload) -> tuple[int, int, list[int]]:
    """The fused kernel's row tensors: (inputs per row, bytes of each input
    row, bytes of each output row).  A per-row scale narrower than 4 bytes
    counts as 4 (the probe's smallest store)."""
    esz = {"bf16": 2, "f16": 2, "f32": 4}[w.in_dtype]
    row = w.hidden * esz
    nin = (w.ninputs if w.ninputs > 1 else 1) + (1 if w.residual else 0)
    outs = [row] if w.residual else []
    if w.fp4:
        outs += [w.hidden // 2, w.hidden // w.fp4_block]
    else:
        outs += [w.hidden, max(4, {"f32": 4, "bf16": 2, "f16": 2}[w.scales_dtype])]
    return nin, row, outs


class _ProbeCase:
    """A streaming reference launch (librmsq_probe) over a workload's bytes,
    in the shape time_case / time_windows expect (rotated buffer sets)."""

    def __init__(self, w: workloads.Workload, copies: int, cfg: dict):
        from fp4_activation_quantization_amd import probe

        self.w, self.cfg, self.keep, self.launches = w, cfg, [], []
        dev = "cuda:0"
        if cfg["kind"] == "rows":
            nin, row, outs = probe_layout(w)
            self.nbytes = w.rows * (nin * row + sum(outs))
            for _ in range(copies):
                ins = [torch.ones(w.rows * row, dtype=torch.uint8, device=dev) for _ in range(nin)]
                ous = [torch.empty(w.rows * b, dtype=torch.uint8, device=dev) for b in outs]
                self.keep += ins + ous
                self.launches.append(probe.Rows(w.rows, ins, row, ous, outs, block=cfg["block"], vpt=cfg["vpt"],
                                                grid=cfg.get("grid", 0), phased=cfg.get("phased", False),
                                                mapped=cfg.get("mapped", False), lds_bytes=cfg.get("lds", 0)))
        else:
            rb, wb = (-(-b // 16) * 16 for b in algorithmic_split(w))
            self.nbytes = rb + wb
            for _ in range(copies):
                src = torch.ones(rb, dtype=torch.uint8, device=dev)
                dst = torch.empty(wb, dtype=torch.uint8, device=dev)
                self.keep += [src, dst]
                self.launches.append(probe.Chunks(src, rb, dst, wb, rv=cfg["rv"], wv=cfg["wv"], block=cfg["block"],
                                                  loads_in_flight=cfg["nl"], blocks_per_cu=cfg.get("per_cu", 0),
                                                  interleave=cfg.get("interleave", False)))

    def step(self, i: int) -> None:
        self.launches[i % len(self.launches)]()


def _unit_ratio(rb: int, wb: int, limit: int = 64) -> tuple[int, int]:
    """Smallest rv, wv (each <= limit) whose ratio is within 2% of rb : wb."""
    want = rb / wb
    for tot in range(2, 2 * limit + 1):
        for r in range(1, tot):
            wv = tot - r
            if r <= limit and wv <= limit and abs(r / wv - want) <= 0.02 * want:
                return r, wv
    return (limit, 1) if want > 1 else (1, limit)


def probe_candidates(w: workloads.Workload, full: bool = False) -> list[dict]:
    """Streaming reference configurations for a workload: the row layout of
    the fused kernel (one block per row, every load of the row in flight) at
    block sizes whose lanes hold the row, and the two-stream chunk form at the
    byte ratio; `full` widens the set to the sweep (loads in flight,
    persistent grids, interleaved writes)."""
    nin, row, outs = probe_layout(w)
    nvec = row // 16
    cands = []
    for block in ((64, 128, 256, 512, 1024) if full else (256, 512, 1024)):
        for vpt in (1, 2, 4, 8):
            if block * vpt >= nvec:
                break
        else:
            continue
        if nin * vpt > 16 or row % 16 or any(b % 16 and (b % 4 or b > 4 * block) for b in outs) or \
                any(b % 16 == 0 and b > row for b in outs):
            continue
        for grid in ((0, 256, 1024, 2048) if full else (0,)):
            cands.append({"kind": "rows", "block": block, "vpt": vpt, "grid": grid})
        # the fused kernels' own order (first output, a barrier, the others)
        # and store pieces (codes by the lane holding their input vector),
        # with 4, 3 or 2 blocks per CU at most (unused LDS)
        if len(outs) > 1:
            for lds in (0, 40960, 54272, 65536):
                cands.append({"kind": "rows", "block": block, "vpt": vpt, "grid": 0, "phased": True, "mapped": True,
                              "lds": lds})
    rb, wb = algorithmic_split(w)
    base = _unit_ratio(rb, wb)
    # the default set: the configurations that won the full sweep on the
    # named workloads (MI355X)
    ratios = [base] + ([(2 * base[0], 2 * base[1])] if 2 * max(base) <= 64 else [])
    for rv, wv in ratios:
        for block in ((256, 512, 1024) if full else (256, 1024)):
            for nl in ((4, 8, 16) if full else (16,)):
                for per_cu in ((0, 4) if full else (0,)):
                    for inter in (False, True):
                        cands.append({"kind": "chunks", "rv": rv, "wv": wv, "block": block, "nl": nl,
                                      "per_cu": per_cu, "interleave": inter})
    return cands


def stream_ceiling(w: workloads.Workload, copies: int, settle_ms: float, window_ms: float, windows: int,
                   full: bool = False, log=None, retime: tuple | None = None) -> dict:
    """The streaming ceiling for this workload's traffic: every candidate
    streaming reference configuration (probe_candidates) timed like the
    workloads (settled, median window, the same number of rotated buffer
    sets); the fastest, in GB/s of the bytes it moves, with its
    configuration, and all of them.  retime = (settle_ms, window_ms,
    windows) times the fastest once more that way."""
    results = []
    for cfg in probe_candidates(w, full):
        c = _ProbeCase(w, copies, cfg)
        settle(c, settle_ms)
        us = time_windows(c, window_ms, windows)["launch_us"]
        results.append({"gbps": round(c.nbytes / (us * 1e-6) / 1e9, 1), "launch_us": round(us, 3), **cfg})
        if log:
            log(f"  {results[-1]}")
        del c
        torch.cuda.empty_cache()
    results.sort(key=lambda r: -r["gbps"])
    best = dict(results[0])
    if retime:
        # the fastest configuration again under the fused kernels' own
        # protocol (their settling and windows)
        c = _ProbeCase(w, copies, {k: v for k, v in best.items() if k not in ("gbps", "launch_us")})
        settle(c, retime[0])
        us = time_windows(c, retime[1], retime[2])["launch_us"]
        best.update(gbps=round(c.nbytes / (us * 1e-6) / 1e9, 1), launch_us=round(us, 3))
        del c
        torch.cuda.empty_cache()
    return {"gbps": best["gbps"], "config": best, "all": results}


def fp4_global_scale(name: str) -> float:
    """The stored calibration of an FP4 workload (1.0 where its scales do not use one)."""
    p = os.path.join(ROOT, "tests", "golden", "fp4_global_scale.json")
    entry = json.load(open(p))["workloads"].get(name)
    return entry["global_scale"] if entry else 1.0


def copies_for(w: workloads.Workload) -> int:
    b = algorithmic_bytes(w)
    if b < (16 << 20):
        return 1  # latency-sized: reported warm (served from cache)
    return max(1, -(-CACHE_DEFEAT_BYTES // b))


def traffic_from_profiles(name: str) -> float | None:
    """HBM bytes per launch measured by rocprofv3 counters for this workload, if they
    were taken on the current kernel sources (else None)."""
    p = os.path.join(PROFILES, f"traffic_{name}.md")
    if not os.path.exists(p):
        return None
    for line in open(p):
        if line.startswith("traffic_json:"):
            d = json.loads(line.split(":", 1)[1])
            if d.get("kernel_source_hash") == kernel_source_hash():
                return d.get("hbm_bytes_per_launch")
    return None


def cpu_threads() -> int:
    """Oracle threads: the 16-CPU share one GPU's job is allotted on a
    shared MI355X host, or fewer where the machine has fewer cores."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_rate(case: Case, max_rows: int, threads: int, min_seconds: float) -> dict:
    """The float64 oracle over the workload's first max_rows rows (all of
    them if fewer) on `threads` threads, repeated until min_seconds have
    elapsed (median pass), and on one thread over a 64-row sample; rows/s and
    GB/s with the workload's algorithmic bytes per row."""
    import oracle

    w, inp = case.w, case.inp
    n = min(w.rows, max_rows)
    x = workloads.bits(inp["x"][:n])
    r = workloads.bits(inp["residual"][:n]) if inp.get("residual") is not None else None
    g = workloads.bits(inp["gamma"])
    kw = dict(in_dtype=w.in_dtype, eps=w.eps, weight_offset=w.weight_offset, want_q=False)

    def run(rows, th):
        if w.fp4:
            oracle.rmsnorm_fp4(x[:rows], g, global_scale=case.gs or 1.0, block_size=w.fp4_block,
                               scale_format=w.fp4_scale, residual=r[:rows] if r is not None else None,
                               round_product=w.fp4_round_product, threads=th, **kw)
        elif w.ninputs > 1:
            ins = [workloads.bits(t[:rows]) for t in inp["inputs"]]
            oracle.allreduce_residual_rmsnorm_fp8(ins, r[:rows], g, scale_ub=w.scale_ub, out_fmt=w.out_fmt,
                                                  scales_dtype=w.scales_dtype, threads=th, **kw)
        else:
            oracle.rmsnorm_fp8(x[:rows], g, scale_ub=w.scale_ub, out_fmt=w.out_fmt, scales_dtype=w.scales_dtype,
                               residual=r[:rows] if r is not None else None, threads=th, **kw)

    oracle.lib()
    times, t_all = [], time.perf_counter()
    while True:
        t0 = time.perf_counter()
        run(n, threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all >= min_seconds or len(times) >= 3:
            break
    per_pass = sorted(times)[len(times) // 2]
    n1 = min(n, 64)
    t0 = time.perf_counter()
    run(n1, 1)
    d1 = time.perf_counter() - t0
    row_bytes = algorithmic_bytes(w) / w.rows
    return {"rows_per_s": round(n / per_pass, 1), "gbps": round(row_bytes * n / per_pass / 1e9, 6),
            "rows": n, "passes": len(times), "threads": threads,
            "single_thread_rows_per_s": round(n1 / d1, 1)}


def cpu_baseline(results: dict, lead: str) -> dict:
    """The headline's oracle rate in the contract's form, with every timed
    workload's beside it."""
    threads = cpu_threads()
    per = {n: r["cpu"] for n, r in results.items() if r.get("cpu")}
    h = per.get(lead)
    if h is None:
        return {}
    try:
        quota = open("/sys/fs/cgroup/cpu.max").read().split()
        cg = None if quota[0] == "max" else round(int(quota[0]) / int(quota[1]), 2)
    except (OSError, ValueError, IndexError):
        cg = None
    return {"value": h["gbps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {h['rows']} rows of {lead} (of {workload_of(lead).rows}), median of "
                      f"{h['passes']} pass(es), float64 C oracle split by rows over {threads} threads",
            "rows_per_s": h["rows_per_s"], "single_thread_rows_per_s": h["single_thread_rows_per_s"],
            "host_logical_cpus": os.cpu_count(), "cgroup_cpu_quota": cg,
            "threads_note": "a one-GPU job is allotted a 16-CPU share of the host; the oracle runs one thread "
                            "per CPU of it (host_logical_cpus counts what the process sees)",
            "per_workload": per}


def copy_calibration(nbytes: int, steps: int) -> None:
    """Reference kernels of known traffic for scaling rocprofv3's FETCH_SIZE /
    WRITE_SIZE counters: the streaming probe (the fused kernels' non-temporal
    16-byte loads and stores) reading nbytes and writing nbytes / 4, then
    torch's device copy of nbytes (ordinary loads and stores)."""
    from fp4_activation_quantization_amd import probe

    nbytes -= nbytes % 64
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    f = probe.Chunks(src, nbytes, dst, nbytes // 4, rv=4, wv=1, block=256, loads_in_flight=16)
    for _ in range(steps):
        f()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe_read_bytes": nbytes, "probe_write_bytes": nbytes // 4, "copy_bytes": nbytes,
                      "steps": steps}), flush=True)


def placement_sweep(w: workloads.Workload, log) -> None:
    """How a residual FP8 workload's rate depends on where its row tensors
    sit: (1) five fresh allocations of the workload's buffers in this process,
    a growing spacer allocation held between them; (2) x, residual and
    residual_out carved from one allocation at chosen offsets, with the
    row-form streaming reference on the same views.  Each time is the median
    of 3 windows of 50 ms after 30 ms of settling."""
    from fp4_activation_quantization_amd import probe

    assert w.residual and not w.fp4 and w.ninputs == 1, "a residual FP8 workload"
    spacers = []
    for t in range(5):
        c = Case(w, 1, None)
        settle(c, 30)
        r = time_windows(c, 50, 3)
        log(f"| fresh allocation {t} | {r['launch_us']:.2f} | | x at {c.keep[1].data_ptr():#x} |")
        del c
        torch.cuda.empty_cache()
        spacers.append(torch.empty((t + 1) * (256 << 20), dtype=torch.uint8, device="cuda:0"))
    spacers.clear()
    torch.cuda.empty_cache()
    inp = workloads.make(w)
    esz = {"bf16": 2, "f16": 2, "f32": 4}[w.in_dtype]
    td = workloads.TORCH_DTYPES[w.in_dtype]
    tb = w.rows * w.hidden * esz
    MB = 1 << 20
    big = torch.empty(3 * tb + 64 * MB, dtype=torch.uint8, device="cuda:0")
    g = inp["gamma"].to("cuda:0")
    out = torch.empty(w.rows * w.hidden, dtype=torch.uint8, device="cuda:0")
    sc = torch.empty(w.rows, dtype=torch.float32, device="cuda:0")
    row = w.hidden * esz

    class _Timed:
        def __init__(self, fn):
            self.w, self.step = w, (lambda i: fn())

    for d1, d2 in [(0, 0), (4096, 8192), (65536, 131072), (MB, 2 * MB), (2 * MB + 4096, 4 * MB + 8192),
                   (8 * MB, 16 * MB), (16 * MB + 65536, 32 * MB + 131072), (3 * MB, 7 * MB)]:
        views = [big[o:o + tb].view(td).view(w.rows, w.hidden) for o in (0, tb + d1, 2 * tb + d2)]
        x, r, ro = views
        x.copy_(inp["x"])
        r.copy_(inp["residual"])
        fused = _Timed(lambda: rq.residual_rmsnorm_fp8(x, r, g, eps=w.eps, scale_ub=w.scale_ub, out=out, scales=sc,
                                                       residual_out=ro))
        settle(fused, 30)
        tf = time_windows(fused, 50, 3)["launch_us"]
        u8 = [v.view(torch.uint8).view(-1) for v in views]
        f = probe.Rows(w.rows, u8[:2], row, [u8[2], out, sc.view(torch.uint8)], [row, w.hidden, 4], block=256,
                       vpt=max(1, min(8, row // 4096)))
        ref = _Timed(f)
        settle(ref, 30)
        tp = time_windows(ref, 50, 3)["launch_us"]
        log(f"| residual at +{d1 // 1024} KiB, residual_out at +{d2 // 1024} KiB | {tf:.2f} | {tp:.2f} | |")


def workload_of(name: str) -> workloads.Workload:
    """A named workload, or an ad-hoc shape 'op:ROWSxHIDDEN:dtype' (for example
    rmsnorm_fp8:1024x65536:bf16, op as in workloads.Workload) with seeded
    normal activations, eps 1e-6 and the Workload defaults otherwise."""
    if name in workloads.WORKLOADS:
        return workloads.WORKLOADS[name]
    try:
        op, shape, dt = name.split(":")
        rows, hidden = (int(v) for v in shape.split("x"))
    except ValueError:
        raise SystemExit(f"unknown workload {name!r}: a name from workloads.py or op:ROWSxHIDDEN:dtype")
    return workloads.Workload(name, op, rows, hidden, dt, 95, eps=1e-6)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workloads", default="all",
                    help="'all', 'headline' or comma-separated workload names or shapes op:ROWSxHIDDEN:dtype")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed GPU time before each workload's warm-up (clock settling)")
    ap.add_argument("--window-ms", type=float, default=100.0, help="GPU time per timing window (other workloads)")
    ap.add_argument("--windows", type=int, default=5, help="timing windows per workload other than the headline")
    ap.add_argument("--cpu-seconds", type=float, default=1.0, help="minimum oracle time per workload")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of each workload the oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true", help="skip the streaming reference kernels")
    ap.add_argument("--probe-window-ms", type=float, default=30.0, help="GPU time per timing window of each "
                    "streaming reference configuration")
    ap.add_argument("--probe-windows", type=int, default=3, help="timing windows per streaming reference "
                    "configuration")
    ap.add_argument("--probe-sweep", action="store_true", help="only sweep the streaming reference kernels over "
                    "their full configuration set for the selected workloads, print a table and exit")
    ap.add_argument("--placement-sweep", action="store_true", help="only time the selected residual FP8 workloads "
                    "on several buffer placements, print a table and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run the counter-scaling references (the streaming probe reading BYTES and writing "
                    "BYTES/4, then a device copy of BYTES) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (rows shard across GPUs "
              "without communication; see the design notes). Run with --gpus 1.", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return 0
    rq.lib()

    if args.workloads == "all":
        names = list(workloads.WORKLOADS)
    elif args.workloads == "headline":
        names = [workloads.HEADLINE]
    else:
        names = args.workloads.split(",")
    lead = workloads.HEADLINE if workloads.HEADLINE in names else names[0]
    # the lead workload runs first, on a GPU whose memory no other workload
    # has used yet (later runs of the same kernel measured up to 2% slower)
    names = [lead] + [n for n in names if n != lead]

    if args.placement_sweep:
        for name in names:
            print(f"## {name}\n\n| placement | fused us | row-form streaming reference us | |\n|---|---|---|---|",
                  flush=True)
            placement_sweep(workload_of(name), lambda m: print(m, flush=True))
        return 0

    if args.probe_sweep:
        for name in names:
            w = workload_of(name)
            sc = stream_ceiling(w, copies_for(w), 20.0, args.probe_window_ms, args.probe_windows, full=True,
                                log=lambda m: print(m, file=sys.stderr, flush=True))
            print(f"## {name} ({len(sc['all'])} configurations, {copies_for(w)} buffer set(s))", flush=True)
            print("| GB/s | us | kind | config |\n|---|---|---|---|", flush=True)
            for r in sc["all"]:
                cfg = {k: v for k, v in r.items() if k not in ("gbps", "launch_us", "kind")}
                print(f"| {r['gbps']:.0f} | {r['launch_us']:.2f} | {r['kind']} | {cfg} |", flush=True)
        return 0

    results = {}
    for name in names:
        w = workload_of(name)
        k = copies_for(w)
        # ad-hoc FP4 shapes take a global scale of 64 (named ones their stored value)
        gs = (fp4_global_scale(name) if name in workloads.WORKLOADS else 64.0) if w.fp4 else None
        case = Case(w, k, gs)
        settled = settle(case, args.settle_ms)
        if name == lead:
            res = time_case(case, args.steps, args.warmup)  # exactly K timed steps
        else:
            res = time_windows(case, args.window_ms, args.windows)
        res["settle_launches"] = settled
        res["buffer_sets"] = k
        res["launch"] = rq.query_shape(w.rows, w.hidden, workloads.TORCH_DTYPES[w.in_dtype], w.fp4, w.residual,
                                       summed=w.ninputs > 1)
        # latency-sized calls: also their GPU time inside a graph (decode steps run graphed)
        res.update(time_graph(case, 100, max(5, args.steps // 100)) if algorithmic_bytes(w) < STREAM_MIN_BYTES else {})
        # the oracle on this workload's host inputs, after the GPU timing
        res["cpu"] = None if args.no_cpu_baseline else oracle_rate(case, args.cpu_rows, cpu_threads(), args.cpu_seconds)
        results[name] = res
        del case
        torch.cuda.empty_cache()
        # the achievable ceiling for this traffic mix (bandwidth-sized workloads only)
        sc = (stream_ceiling(w, k, 20.0, args.probe_window_ms, args.probe_windows,
                             retime=(args.settle_ms, args.window_ms, args.windows))
              if algorithmic_bytes(w) >= STREAM_MIN_BYTES and not args.no_stream_ceiling else None)
        res["stream_gbps"] = sc["gbps"] if sc else None
        res["stream_config"] = {k_: v for k_, v in sc["config"].items() if k_ != "gbps"} if sc else None
        ceil = f", streaming ceiling {res['stream_gbps']:.0f} GB/s ({res['stream_config']})" if sc else ""
        if "graph_us" in res:
            ceil += f", {res['graph_us']:.2f} us per call in a graph (p50 over replays {res['graph_us_p50']:.2f})"
        cpu = f", oracle {res['cpu']['rows_per_s']:.0f} rows/s" if res["cpu"] else ""
        print(f"# {name}: {res['launch_us']:.2f} us/launch, {res['gbps']:.0f} GB/s{ceil}{cpu}, {k} buffer set(s), "
              f"launch {res['launch']}", file=sys.stderr, flush=True)

    h = results[lead]
    w = workload_of(lead)
    line = {
        "metric": "GB/s and % of HBM peak (rows/s) for fused residual+RMSNorm+FP8 quant, 1 GPU"
                  if lead == workloads.HEADLINE else f"GB/s (algorithmic HBM bytes) for {w.op}, 1 GPU",
        "value": round(h["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded PCG64 activations; see workloads.py)",
        "config": {"workload": w.name, "rows": w.rows, "hidden": w.hidden, "in_dtype": w.in_dtype,
                   "op": w.op, "global_batch": w.rows, "buffer_sets": h["buffer_sets"], "launch": h["launch"],
                   "settle_launches": h["settle_launches"]},
        "rows_per_s": round(h["rows_per_s"], 1),
        "pct_hbm_peak": round(100.0 * h["gbps"] / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(h["gbps"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(h["gbps"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles(w.name),
                     "stream_reference": round(h["stream_gbps"], 1) if h["stream_gbps"] else None,
                     "launch_us": round(h["launch_us"], 3), "bytes_per_launch": h["bytes"]},
        "workloads": {n: {"launch_us": round(r["launch_us"], 3), "gbps": round(r["gbps"], 1),
                          "timing": "exactly K steps" if n == lead else
                          f"median of {r['windows']} windows of {r['window_launches']} launches",
                          "launch_us_min": round(r.get("launch_us_min", r["launch_us"]), 3),
                          "launch_us_max": round(r.get("launch_us_max", r["launch_us"]), 3),
                          "frac_hbm": round(r["gbps"] / HBM_PEAK_GBS, 4), "rows_per_s": round(r["rows_per_s"], 1),
                          "bytes": r["bytes"], "buffer_sets": r["buffer_sets"], "launch": r["launch"],
                          "graph_us": round(r["graph_us"], 3) if "graph_us" in r else None,
                          "graph_us_p50": round(r["graph_us_p50"], 3) if "graph_us_p50" in r else None,
                          "stream_reference_gbps": round(r["stream_gbps"], 1) if r["stream_gbps"] else None,
                          "stream_reference_config": r["stream_config"],
                          "frac_of_stream_reference": round(r["gbps"] / r["stream_gbps"], 4)
                          if r["stream_gbps"] else None}
                      for n, r in results.items()},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(results, lead)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
