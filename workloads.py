"""Seeded synthetic activations for the fused RMSNorm + FP8/FP4 quantization path.

This module draws inputs only: it holds none of the method's arithmetic and
is shared by the oracle tests, the GPU parity tests and the benchmark.  Every
tensor comes from ``numpy.random.Generator(PCG64)`` seeded with
``SeedSequence([seed, workload_id])`` spawned into four streams
(x, residual, gamma, selection), drawn in float32/float64 and cast to the
input dtype with torch's round-to-nearest-even.

The workloads reproduce the shapes and value structure of the activations
these kernels see in LLM inference: a small smoke shape, a Llama-3-8B hidden
size with a few hot outlier channels, single-token decode batches with a
Gemma-style (1 + gamma) weight, a 70B-class prefill batch with heavy-tailed
(Laplace) activations and a few hot rows, and a 7168-wide FP4 tensor whose
1% heavy channels follow Student-t(3) (quantized three ways: 16-element E4M3
scales row-major or swizzled, and 32-element UE8M0 scales; and once more
behind a residual add).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    op: str  # "rmsnorm_fp8" | "residual_rmsnorm_fp8" | "rmsnorm_fp4" | "residual_rmsnorm_fp4"
    rows: int
    hidden: int
    in_dtype: str           # "bf16" | "f16" | "f32"
    workload_id: int
    eps: float
    weight_offset: float = 0.0
    scale_ub: float = 1200.0
    out_fmt: str = "e4m3fn"  # FP8 only
    scales_dtype: str = "f32"  # FP8 only
    x_dist: str = "normal"    # "normal" | "laplace"
    x_std: float = 1.0
    gamma_dist: str = "uniform"
    gamma_lo: float = 0.5
    gamma_hi: float = 1.5
    gamma_std: float = 0.0
    outlier_channels: int = 0     # columns scaled by outlier_scale (x and residual)
    outlier_scale: float = 1.0
    outlier_row_frac: float = 0.0  # fraction of rows scaled by outlier_scale
    heavy_channel_frac: float = 0.0  # fraction of columns drawn from Student-t(3)
    widen_from: str | None = None    # f32 workload holding another workload's bf16 values
    fp4_block: int = 16              # FP4 only: elements per block scale (16 or 32)
    fp4_scale: str = "e4m3"          # FP4 only: "e4m3" or "ue8m0" block scales
    fp4_swizzled: bool = False       # FP4 only: 128 x 4-tile scale layout
    fp4_round_product: bool = False  # FP4 only: the page's 16-bit x * w numerics
    ninputs: int = 1                 # FP8 summed inputs (allreduce op): input buffers summed with the residual

    @property
    def residual(self) -> bool:
        return self.op.startswith("residual_") or self.op.startswith("allreduce_residual_")

    @property
    def fp4(self) -> bool:
        return self.op.endswith("_fp4")

    def with_rows(self, rows: int) -> "Workload":
        return dataclasses.replace(self, rows=rows)


WORKLOADS = {w.name: w for w in [
    Workload("rmsnorm_fp8_bf16_16x512", "rmsnorm_fp8", 16, 512, "bf16", 0, eps=1e-6,
             gamma_lo=0.5, gamma_hi=1.5),
    Workload("residual_rmsnorm_fp8_bf16_8192x4096", "residual_rmsnorm_fp8", 8192, 4096, "bf16", 1,
             eps=1e-5, gamma_lo=0.8, gamma_hi=1.2, outlier_channels=8, outlier_scale=50.0),
    Workload("rmsnorm_fp8_f16_decode_1x8192", "rmsnorm_fp8", 1, 8192, "f16", 2, eps=1e-6,
             weight_offset=1.0, scale_ub=1e4, out_fmt="e4m3fnuz", scales_dtype="bf16",
             x_std=math.sqrt(2.0), gamma_dist="normal", gamma_std=math.sqrt(0.02)),
    Workload("rmsnorm_fp8_f16_decode_8x8192", "rmsnorm_fp8", 8, 8192, "f16", 2, eps=1e-6,
             weight_offset=1.0, scale_ub=1e4, out_fmt="e4m3fnuz", scales_dtype="bf16",
             x_std=math.sqrt(2.0), gamma_dist="normal", gamma_std=math.sqrt(0.02)),
    Workload("rmsnorm_fp8_f16_decode_64x8192", "rmsnorm_fp8", 64, 8192, "f16", 2, eps=1e-6,
             weight_offset=1.0, scale_ub=1e4, out_fmt="e4m3fnuz", scales_dtype="bf16",
             x_std=math.sqrt(2.0), gamma_dist="normal", gamma_std=math.sqrt(0.02)),
    Workload("residual_rmsnorm_fp8_bf16_32768x8192", "residual_rmsnorm_fp8", 32768, 8192, "bf16", 3,
             eps=1e-5, x_dist="laplace", gamma_lo=0.5, gamma_hi=1.5, outlier_row_frac=0.01,
             outlier_scale=100.0),
    Workload("residual_rmsnorm_fp8_f32_32768x8192", "residual_rmsnorm_fp8", 32768, 8192, "f32", 3,
             eps=1e-5, x_dist="laplace", gamma_lo=0.5, gamma_hi=1.5, outlier_row_frac=0.01,
             outlier_scale=100.0, widen_from="bf16"),
    Workload("rmsnorm_fp4_bf16_16384x7168", "rmsnorm_fp4", 16384, 7168, "bf16", 4, eps=1e-6,
             gamma_lo=0.8, gamma_hi=1.2, heavy_channel_frac=0.01),
    # the same tensor (same workload id, so the same draws) quantized as MXFP4
    # (32-element blocks, UE8M0 scales), and as NVFP4 with swizzled scales
    Workload("rmsnorm_mxfp4_bf16_16384x7168", "rmsnorm_fp4", 16384, 7168, "bf16", 4, eps=1e-6,
             gamma_lo=0.8, gamma_hi=1.2, heavy_channel_frac=0.01, fp4_block=32, fp4_scale="ue8m0"),
    Workload("rmsnorm_fp4_swizzled_bf16_16384x7168", "rmsnorm_fp4", 16384, 7168, "bf16", 4, eps=1e-6,
             gamma_lo=0.8, gamma_hi=1.2, heavy_channel_frac=0.01, fp4_swizzled=True),
    # a residual stream in front of the FP4 quantizer (x and residual drawn alike)
    Workload("residual_rmsnorm_fp4_bf16_16384x7168", "residual_rmsnorm_fp4", 16384, 7168, "bf16", 5, eps=1e-6,
             gamma_lo=0.8, gamma_hi=1.2, heavy_channel_frac=0.01),
    # the headline's rows as 8 per-GPU partial buffers summed with the residual
    # (each buffer drawn like the headline's x, same outlier channels)
    Workload("allreduce_residual_rmsnorm_fp8_bf16_8x8192x4096", "allreduce_residual_rmsnorm_fp8", 8192, 4096, "bf16",
             6, eps=1e-5, gamma_lo=0.8, gamma_hi=1.2, outlier_channels=8, outlier_scale=50.0, ninputs=8),
]}

# The workload the headline throughput is quoted on: the large-batch
# residual FP8 shape (70B-class, 32768 x 8192 bf16), the largest one-GPU
# configuration of the fused residual + RMSNorm + FP8 metric.
HEADLINE = "residual_rmsnorm_fp8_bf16_32768x8192"


def _streams(w: Workload, seed: int):
    ss = np.random.SeedSequence([seed, w.workload_id])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def _draw_activations(rng, w: Workload, sel: dict) -> np.ndarray:
    shape = (w.rows, w.hidden)
    if w.x_dist == "laplace":
        # Laplace(0, 1) as the difference of two independent Exp(1) draws
        a = rng.standard_exponential(shape, dtype=np.float32)
        a -= rng.standard_exponential(shape, dtype=np.float32)
    else:
        a = rng.standard_normal(shape, dtype=np.float32)
        if w.x_std != 1.0:
            a *= np.float32(w.x_std)
    if sel["heavy_cols"] is not None:
        heavy = rng.standard_t(3.0, size=(w.rows, sel["heavy_cols"].size)).astype(np.float32)
        a[:, sel["heavy_cols"]] = heavy
    if sel["outlier_cols"] is not None:
        a[:, sel["outlier_cols"]] *= np.float32(w.outlier_scale)
    if sel["outlier_rows"] is not None:
        a[sel["outlier_rows"], :] *= np.float32(w.outlier_scale)
    return a


def _selection(rng, w: Workload) -> dict:
    sel = {"outlier_cols": None, "outlier_rows": None, "heavy_cols": None}
    if w.outlier_channels:
        sel["outlier_cols"] = np.sort(rng.choice(w.hidden, size=w.outlier_channels, replace=False))
    if w.outlier_row_frac > 0.0 and w.rows > 0:
        k = max(1, int(math.ceil(w.outlier_row_frac * w.rows)))
        sel["outlier_rows"] = np.sort(rng.choice(w.rows, size=k, replace=False))
    if w.heavy_channel_frac > 0.0:
        k = max(1, int(math.ceil(w.heavy_channel_frac * w.hidden)))
        sel["heavy_cols"] = np.sort(rng.choice(w.hidden, size=k, replace=False))
    return sel


def _to(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(a).to(TORCH_DTYPES[dtype])


def make(w: Workload | str, seed: int = 0, rows: int | None = None) -> dict:
    """Host (CPU) input tensors for a workload: x, residual (or None), gamma.

    rows overrides the row count (same distributions, same column choices).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if rows is not None:
        w = w.with_rows(rows)
    if w.widen_from is not None:
        base = make(dataclasses.replace(w, in_dtype=w.widen_from, widen_from=None), seed)
        out = {k: (v.to(torch.float32) if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
        out["workload"] = w
        return out
    rx, rr, rg, rs = _streams(w, seed)
    sel = _selection(rs, w)
    x = _to(_draw_activations(rx, w, sel), w.in_dtype)
    # further input buffers continue x's stream
    inputs = [x] + [_to(_draw_activations(rx, w, sel), w.in_dtype) for _ in range(w.ninputs - 1)]
    res = _to(_draw_activations(rr, w, sel), w.in_dtype) if w.residual else None
    if w.gamma_dist == "normal":
        g = rg.normal(0.0, w.gamma_std, size=w.hidden)
    else:
        g = rg.uniform(w.gamma_lo, w.gamma_hi, size=w.hidden)
    gamma = _to(g.astype(np.float32), w.in_dtype)
    out = {"x": x, "residual": res, "gamma": gamma, "workload": w, "selection": sel}
    if w.ninputs > 1:
        out["inputs"] = inputs
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a CPU tensor as numpy (float32, or uint16 for 16-bit types)."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of bits(): a CPU tensor of dtype holding these bits."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(TORCH_DTYPES[dtype])
