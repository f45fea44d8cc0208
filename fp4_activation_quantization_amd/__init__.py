"""Python binding of librmsq (fused RMSNorm + FP8 / FP4 quantization on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of librmsq.so, reached through the C ABI declared in include/rmsq.h.
torch provides device memory and the current stream.  There is no fallback:
if the library is missing or a call fails, an exception is raised.

Functions mirror the C entry points:
  rmsnorm_fp8(x, gamma, ...)                   -> (codes, scales)
  residual_rmsnorm_fp8(x, residual, gamma, ...) -> (codes, scales, residual_out)
  rmsnorm_fp4(x, gamma, ...)                   -> (packed_codes, block_scales)
  convert(kind, src, dst)
Tensors may have any number of leading dimensions; the last one is hidden.
Outputs are allocated (uint8 / scale dtype) when not given.  Every tensor
must live on x's GPU, and given buffers must have the sizes the kernels
write (checked here, since the C ABI receives bare pointers); the call runs
with x's GPU current.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librmsq.so")

# enums of include/rmsq.h
F32, F16, BF16 = 0, 1, 2
E4M3FN, E4M3FNUZ = 0, 1
SF_E4M3, SF_UE8M0 = 0, 1            # FP4 block-scale formats
SF_ROW_MAJOR, SF_SWIZZLED = 0, 1    # FP4 block-scale layouts
FP4_ROUND_PRODUCT = 1               # FP4 flag: the page's 16-bit x * w
CVT_F32_TO_E4M3FN, CVT_F32_TO_E4M3FNUZ, CVT_F32_TO_E2M1, CVT_F32_TO_BF16, CVT_F32_TO_F16, CVT_E4M3FN_TO_F32 = range(6)
STATUS = {0: "RMSQ_OK", -1: "RMSQ_ERR_NULL", -2: "RMSQ_ERR_DTYPE", -3: "RMSQ_ERR_SHAPE", -4: "RMSQ_ERR_ALIGN",
          -5: "RMSQ_ERR_VALUE", -6: "RMSQ_ERR_ALIAS", -7: "RMSQ_ERR_UNSUPPORTED", -8: "RMSQ_ERR_LAUNCH"}

_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_FMT = {"e4m3fn": E4M3FN, "e4m3fnuz": E4M3FNUZ}

_lib = None


class RmsqError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn} failed: {STATUS.get(status, status)}"
        if status == -8:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """The loaded librmsq.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp4_activation_quantization_amd.build` "
                           "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.rmsnorm_fp8.argtypes = [I64, I64, I, P, P, F, F, F, I, P, I, P, P]
    L.residual_rmsnorm_fp8.argtypes = [I64, I64, I, P, P, P, P, F, F, F, I, P, I, P, P]
    L.gated_rmsnorm_fp8.argtypes = [I64, I64, I, P, P, P, F, F, F, I, P, I, P, P]
    L.rmsnorm_fp4.argtypes = [I64, I64, I, P, P, F, F, P, P, P, P]
    L.allreduce_residual_rmsnorm_fp8.argtypes = [I64, I64, I, I, ctypes.POINTER(P), P, P, P, F, F, F, I, P, I, P, P]
    L.rmsnorm_fp4quant.argtypes = [I64, I64, I, P, P, F, F, P, I, I, I, I, P, P, P]
    L.rmsnorm_fp8_strided.argtypes = [I64, I64, I, P, I64, P, I64, P, I64, P, F, F, F, I, P, I64, I, P, P]
    L.rmsnorm_fp4quant_strided.argtypes = [I64, I64, I, P, I64, P, I64, P, I64, P, F, F, P, I, I, I, I, P, I64, P, P]
    L.residual_rmsnorm_fp4quant.argtypes = [I64, I64, I, P, P, P, P, F, F, P, I, I, I, I, P, P, P]
    L.rmsq_fp4_scale_bytes.argtypes = [I64, I64, I, I]
    L.rmsq_fp4_scale_bytes.restype = I64
    L.rmsq_convert.argtypes = [I, P, P, I64, P]
    L.rmsq_set_tuning.argtypes = [I, I, I]
    L.rmsq_query_shape.argtypes = [I64, I64, I, I, ctypes.POINTER(I), ctypes.POINTER(I), ctypes.POINTER(I)]
    L.rmsq_status_string.argtypes = [I]
    L.rmsq_status_string.restype = ctypes.c_char_p
    for fn in ("rmsnorm_fp8", "residual_rmsnorm_fp8", "allreduce_residual_rmsnorm_fp8", "gated_rmsnorm_fp8",
               "rmsnorm_fp4",
               "rmsnorm_fp4quant", "residual_rmsnorm_fp4quant", "rmsnorm_fp8_strided", "rmsnorm_fp4quant_strided", "rmsq_convert",
               "rmsq_set_tuning",
               "rmsq_query_shape", "rmsq_abi_version", "rmsq_last_hip_error"):
        getattr(L, fn).restype = I
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise RmsqError(fn, status, lib().rmsq_last_hip_error() if status == -8 else 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# one-byte element types accepted for code outputs (written as raw bytes)
_BYTE = tuple(t for t in (torch.uint8, torch.int8, getattr(torch, "float8_e4m3fn", None),
                          getattr(torch, "float8_e4m3fnuz", None)) if t is not None)


def _gpu(name: str, t, dev: torch.device) -> None:
    """t (if given) must live on GPU `dev`: the kernels receive raw device
    pointers, and a host pointer, or another GPU's, would fault there."""
    if t is not None and (not t.is_cuda or t.device != dev):
        raise ValueError(f"{name} must be a tensor on {dev if dev.type == 'cuda' else 'a GPU'}, got {t.device}")


def _buf(name: str, t, dev: torch.device, numel: int, dtypes) -> None:
    """An output or input buffer the kernel walks as numel dense elements."""
    _gpu(name, t, dev)
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not one of {dtypes}")
    if t.numel() != numel or not t.is_contiguous():
        raise ValueError(f"{name}: expected {numel} contiguous elements, got {t.numel()} "
                         f"({'contiguous' if t.is_contiguous() else 'not contiguous'})")


def _device(x: torch.Tensor):
    """x's GPU made current for the call (a no-op when it already is)."""
    _gpu("x", x, x.device)
    if x.device.index is None or x.device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(x.device)


def _check_gamma(gamma, x: torch.Tensor, hidden: int) -> None:
    _buf("gamma", gamma, x.device, hidden, (x.dtype,))


def _check_global_scale(global_scale, dev: torch.device) -> None:
    if global_scale is not None:
        _gpu("global_scale", global_scale, dev)
        if global_scale.dtype != torch.float32 or global_scale.numel() != 1:
            raise ValueError("global_scale must be a one-element float32 tensor")


def _rows_hidden(x: torch.Tensor):
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    hidden = x.shape[-1] if x.dim() else 0
    rows = x.numel() // hidden if hidden else 0
    return rows, hidden


def _u8(t: torch.Tensor) -> torch.Tensor:
    return t if t.dtype == torch.uint8 else t.view(torch.uint8)


def rmsnorm_fp8(x, gamma, eps=1e-6, weight_offset=0.0, scale_ub=float("inf"), out_fp8="e4m3fn",
                out=None, scales=None, scales_dtype=torch.float32, stream=None):
    """RMSNorm + per-row dynamic FP8 (C: rmsnorm_fp8).  Returns (codes uint8 [..., H], scales [...])."""
    rows, hidden = _rows_hidden(x)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=scales_dtype, device=x.device)
    ctx = _device(x)
    _check_gamma(gamma, x, hidden)
    _buf("out", out, x.device, rows * hidden, _BYTE)
    _buf("scales", scales, x.device, rows, tuple(_DT))
    with ctx:
        _check("rmsnorm_fp8", lib().rmsnorm_fp8(rows, hidden, _DT[x.dtype], _ptr(x), _ptr(gamma), eps, weight_offset,
                                                scale_ub, _FMT[out_fp8], _ptr(_u8(out)), _DT[scales.dtype],
                                                _ptr(scales), _stream(x, stream)))
    return out, scales


def gated_rmsnorm_fp8(a, b, gamma, eps=1e-6, weight_offset=0.0, scale_ub=float("inf"), out_fp8="e4m3fn",
                      out=None, scales=None, scales_dtype=torch.float32, stream=None):
    """RMSNorm + per-row dynamic FP8 of x = a * b (rounded to a.dtype), formed
    as the kernel loads a and b (C: gated_rmsnorm_fp8).  Returns (codes, scales)."""
    rows, hidden = _rows_hidden(a)
    if b.dtype != a.dtype or b.shape != a.shape:
        raise ValueError("b must match a in dtype and shape")
    if out is None:
        out = torch.empty(a.shape, dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty(a.shape[:-1], dtype=scales_dtype, device=a.device)
    ctx = _device(a)
    _check_gamma(gamma, a, hidden)
    _buf("b", b, a.device, rows * hidden, (a.dtype,))
    _buf("out", out, a.device, rows * hidden, _BYTE)
    _buf("scales", scales, a.device, rows, tuple(_DT))
    with ctx:
        _check("gated_rmsnorm_fp8",
               lib().gated_rmsnorm_fp8(rows, hidden, _DT[a.dtype], _ptr(a), _ptr(b), _ptr(gamma), eps, weight_offset,
                                       scale_ub, _FMT[out_fp8], _ptr(_u8(out)), _DT[scales.dtype], _ptr(scales),
                                       _stream(a, stream)))
    return out, scales


def residual_rmsnorm_fp8(x, residual, gamma, eps=1e-6, weight_offset=0.0, scale_ub=float("inf"),
                         out_fp8="e4m3fn", out=None, scales=None, residual_out=None,
                         scales_dtype=torch.float32, stream=None):
    """residual_out = x + residual (rounded to x.dtype), then RMSNorm + per-row FP8
    (C: residual_rmsnorm_fp8).  Returns (codes, scales, residual_out)."""
    rows, hidden = _rows_hidden(x)
    if residual.dtype != x.dtype or residual.shape != x.shape:
        raise ValueError("residual must match x in dtype and shape")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=scales_dtype, device=x.device)
    if residual_out is None:
        residual_out = torch.empty_like(x)
    ctx = _device(x)
    _check_gamma(gamma, x, hidden)
    _buf("residual", residual, x.device, rows * hidden, (x.dtype,))
    _buf("residual_out", residual_out, x.device, rows * hidden, (x.dtype,))
    _buf("out", out, x.device, rows * hidden, _BYTE)
    _buf("scales", scales, x.device, rows, tuple(_DT))
    with ctx:
        _check("residual_rmsnorm_fp8",
               lib().residual_rmsnorm_fp8(rows, hidden, _DT[x.dtype], _ptr(x), _ptr(residual), _ptr(residual_out),
                                          _ptr(gamma), eps, weight_offset, scale_ub, _FMT[out_fp8], _ptr(_u8(out)),
                                          _DT[scales.dtype], _ptr(scales), _stream(x, stream)))
    return out, scales, residual_out


def allreduce_residual_rmsnorm_fp8(inputs, residual, gamma, eps=1e-6, weight_offset=0.0, scale_ub=float("inf"),
                                   out_fp8="e4m3fn", out=None, scales=None, residual_out=None,
                                   scales_dtype=torch.float32, stream=None):
    """residual_out = residual + sum(inputs) (the exact sum rounded once to
    residual.dtype), then RMSNorm + per-row FP8 (C: allreduce_residual_rmsnorm_fp8;
    the inputs are tensors this GPU can read, no communication).  Returns
    (codes, scales, residual_out)."""
    rows, hidden = _rows_hidden(residual)
    inputs = list(inputs)
    for t in inputs:
        if t.dtype != residual.dtype or t.shape != residual.shape or not t.is_contiguous():
            raise ValueError("every input must be contiguous with residual's shape and dtype")
    if out is None:
        out = torch.empty(residual.shape, dtype=torch.uint8, device=residual.device)
    if scales is None:
        scales = torch.empty(residual.shape[:-1], dtype=scales_dtype, device=residual.device)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    ctx = _device(residual)
    for k, t in enumerate(inputs):
        _gpu(f"inputs[{k}]", t, residual.device)
    _check_gamma(gamma, residual, hidden)
    _buf("residual_out", residual_out, residual.device, rows * hidden, (residual.dtype,))
    _buf("out", out, residual.device, rows * hidden, _BYTE)
    _buf("scales", scales, residual.device, rows, tuple(_DT))
    ptrs = (ctypes.c_void_p * max(1, len(inputs)))(*[_ptr(t) for t in inputs])
    with ctx:
        _check("allreduce_residual_rmsnorm_fp8",
               lib().allreduce_residual_rmsnorm_fp8(rows, hidden, _DT[residual.dtype], len(inputs), ptrs,
                                                    _ptr(residual), _ptr(residual_out), _ptr(gamma), eps,
                                                    weight_offset, scale_ub, _FMT[out_fp8], _ptr(_u8(out)),
                                                    _DT[scales.dtype], _ptr(scales), _stream(residual, stream)))
    return out, scales, residual_out


def rmsnorm_fp4(x, gamma, eps=1e-6, weight_offset=0.0, global_scale=None, out=None, block_scales=None,
                stream=None):
    """RMSNorm + FP4 E2M1 with one E4M3 scale per 16 elements (C: rmsnorm_fp4).

    global_scale: a float32 device tensor of one element, or None (1.0).
    Returns (packed uint8 [..., H/2], block_scales uint8 [..., H/16]).
    """
    rows, hidden = _rows_hidden(x)
    if out is None:
        out = torch.empty((*x.shape[:-1], hidden // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        block_scales = torch.empty((*x.shape[:-1], hidden // 16), dtype=torch.uint8, device=x.device)
    ctx = _device(x)
    _check_global_scale(global_scale, x.device)
    _check_gamma(gamma, x, hidden)
    _buf("out", out, x.device, rows * (hidden // 2), _BYTE)
    _buf("block_scales", block_scales, x.device, rows * (hidden // 16), _BYTE)
    with ctx:
        _check("rmsnorm_fp4", lib().rmsnorm_fp4(rows, hidden, _DT[x.dtype], _ptr(x), _ptr(gamma), eps, weight_offset,
                                                _ptr(global_scale), _ptr(_u8(out)), _ptr(_u8(block_scales)),
                                                _stream(x, stream)))
    return out, block_scales


def fp4_scale_bytes(rows: int, hidden: int, block_size: int = 16, swizzled: bool = False) -> int:
    """Bytes of the block-scale buffer (C: rmsq_fp4_scale_bytes)."""
    n = lib().rmsq_fp4_scale_bytes(rows, hidden, block_size, SF_SWIZZLED if swizzled else SF_ROW_MAJOR)
    if n < 0:
        _check("rmsq_fp4_scale_bytes", int(n))
    return int(n)


def _check_fp4_outputs(x, rows, hidden, block_size, swizzled, out, block_scales, global_scale) -> None:
    """Packed codes: rows * hidden/2 dense bytes; block scales: a dense
    buffer of at least rows * hidden/block bytes (row-major) or
    fp4_scale_bytes() bytes (swizzled)."""
    _buf("out", out, x.device, rows * (hidden // 2), _BYTE)
    _gpu("block_scales", block_scales, x.device)
    if block_scales.dtype not in _BYTE or not block_scales.is_contiguous():
        raise ValueError("block_scales must be a contiguous one-byte tensor")
    if swizzled:
        if block_scales.numel() < fp4_scale_bytes(rows, hidden, block_size, True):
            raise ValueError("block_scales is smaller than fp4_scale_bytes()")
    elif block_scales.numel() < rows * (hidden // block_size):
        raise ValueError(f"block_scales: {block_scales.numel()} bytes, fewer than rows * hidden / block_size")
    _check_global_scale(global_scale, x.device)


def rmsnorm_fp4quant(x, gamma, eps=1e-6, weight_offset=0.0, global_scale=None, block_size=16,
                     scale_format=None, swizzled=False, out=None, block_scales=None, stream=None,
                     round_product=False):
    """RMSNorm + FP4 E2M1 with one scale per block_size (16 or 32) elements
    (C: rmsnorm_fp4quant).

    scale_format: "e4m3" or "ue8m0"; None picks "e4m3" for 16-element and
    "ue8m0" for 32-element blocks.  global_scale (a one-element float32
    device tensor, or None for 1.0) is used by E4M3 scales only.
    swizzled: 128 x 4-tile scale layout (a flat uint8 buffer of
    fp4_scale_bytes() bytes) instead of [..., H/block_size] row-major.
    round_product: the FP4 page's numerics (x * w rounded to the input type
    before the rstd scaling); exact products otherwise.
    Returns (packed uint8 [..., H/2], block_scales uint8).
    """
    rows, hidden = _rows_hidden(x)
    if scale_format is None:
        scale_format = "ue8m0" if block_size == 32 else "e4m3"
    sfmt = {"e4m3": SF_E4M3, "ue8m0": SF_UE8M0}[scale_format]
    if out is None:
        out = torch.empty((*x.shape[:-1], hidden // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        if swizzled:
            block_scales = torch.empty((fp4_scale_bytes(rows, hidden, block_size, True),), dtype=torch.uint8,
                                       device=x.device)
        else:
            block_scales = torch.empty((*x.shape[:-1], hidden // block_size), dtype=torch.uint8, device=x.device)
    ctx = _device(x)
    _check_fp4_outputs(x, rows, hidden, block_size, swizzled, out, block_scales, global_scale)
    _check_gamma(gamma, x, hidden)
    with ctx:
        _check("rmsnorm_fp4quant", lib().rmsnorm_fp4quant(
            rows, hidden, _DT[x.dtype], _ptr(x), _ptr(gamma), eps, weight_offset, _ptr(global_scale), block_size,
            sfmt, SF_SWIZZLED if swizzled else SF_ROW_MAJOR, FP4_ROUND_PRODUCT if round_product else 0,
            _ptr(_u8(out)), _ptr(_u8(block_scales)), _stream(x, stream)))
    return out, block_scales


def residual_rmsnorm_fp4quant(x, residual, gamma, eps=1e-6, weight_offset=0.0, global_scale=None, block_size=16,
                              scale_format=None, swizzled=False, out=None, block_scales=None, residual_out=None,
                              stream=None, round_product=False):
    """residual_out = x + residual (rounded once to x's dtype), then
    rmsnorm_fp4quant of residual_out (C: residual_rmsnorm_fp4quant).
    residual_out may be x or residual itself (in-place update).
    Returns (packed, block_scales, residual_out)."""
    rows, hidden = _rows_hidden(x)
    if residual.shape != x.shape or residual.dtype != x.dtype or not residual.is_contiguous():
        raise ValueError("residual must be contiguous with x's shape and dtype")
    if scale_format is None:
        scale_format = "ue8m0" if block_size == 32 else "e4m3"
    sfmt = {"e4m3": SF_E4M3, "ue8m0": SF_UE8M0}[scale_format]
    if residual_out is None:
        residual_out = torch.empty_like(x)
    if out is None:
        out = torch.empty((*x.shape[:-1], hidden // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        if swizzled:
            block_scales = torch.empty((fp4_scale_bytes(rows, hidden, block_size, True),), dtype=torch.uint8,
                                       device=x.device)
        else:
            block_scales = torch.empty((*x.shape[:-1], hidden // block_size), dtype=torch.uint8, device=x.device)
    ctx = _device(x)
    _check_fp4_outputs(x, rows, hidden, block_size, swizzled, out, block_scales, global_scale)
    _check_gamma(gamma, x, hidden)
    _buf("residual", residual, x.device, rows * hidden, (x.dtype,))
    _buf("residual_out", residual_out, x.device, rows * hidden, (x.dtype,))
    with ctx:
        _check("residual_rmsnorm_fp4quant", lib().residual_rmsnorm_fp4quant(
            rows, hidden, _DT[x.dtype], _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(gamma), eps,
            weight_offset, _ptr(global_scale), block_size, sfmt, SF_SWIZZLED if swizzled else SF_ROW_MAJOR,
            FP4_ROUND_PRODUCT if round_product else 0, _ptr(_u8(out)), _ptr(_u8(block_scales)),
            _stream(x, stream)))
    return out, block_scales, residual_out


def _row_view(t: torch.Tensor, name: str):
    """(rows, row stride in elements) of a tensor whose last dim is
    contiguous and whose leading dims collapse to one row stride."""
    if t.dim() == 0 or t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    try:
        v = t.view(-1, t.shape[-1])
    except RuntimeError as e:
        raise ValueError(f"{name}: leading dimensions must collapse to one row stride") from e
    return v.shape[0], (v.stride(0) if v.shape[0] > 1 else t.shape[-1])


def _check_views(x, *, residual, residual_out, out, out_width=None) -> None:
    """Row views of the strided entry points: on x's GPU, x's row count, the
    row width the kernel writes (codes: hidden, or hidden/2 packed FP4)."""
    lead = tuple(x.shape[:-1])
    for name, t, width, dtypes in (("residual", residual, x.shape[-1], (x.dtype,)),
                                   ("residual_out", residual_out, x.shape[-1], (x.dtype,)),
                                   ("out", out, x.shape[-1] if out_width is None else out_width, _BYTE)):
        if t is None:
            continue
        _gpu(name, t, x.device)
        if t.dtype not in dtypes or tuple(t.shape) != lead + (width,):
            raise ValueError(f"{name}: expected shape {lead + (width,)} of {dtypes}, got {tuple(t.shape)} {t.dtype}")


def rmsnorm_fp8_strided(x, gamma, residual=None, eps=1e-6, weight_offset=0.0, scale_ub=float("inf"),
                        out_fp8="e4m3fn", out=None, scales=None, residual_out=None, scales_dtype=torch.float32,
                        stream=None):
    """rmsnorm_fp8 / residual_rmsnorm_fp8 on row-strided tensors (C:
    rmsnorm_fp8_strided): x, residual, residual_out and out may be views
    whose rows are not adjacent (e.g. x = buf[:, :hidden]).  Outputs are
    allocated contiguous when not given.  Returns (codes, scales,
    residual_out or None)."""
    rows, xs = _row_view(x, "x")
    hidden = x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=scales_dtype, device=x.device)
    rs = ros = hidden
    if residual is not None:
        if residual.dtype != x.dtype or residual.shape != x.shape:
            raise ValueError("residual must match x in dtype and shape")
        if residual_out is None:
            residual_out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
        _, rs = _row_view(residual, "residual")
        _, ros = _row_view(residual_out, "residual_out")
    _, os_ = _row_view(_u8(out), "out")
    ctx = _device(x)
    _check_views(x, residual=residual, residual_out=residual_out, out=out)
    _check_gamma(gamma, x, hidden)
    _buf("scales", scales, x.device, rows, tuple(_DT))
    with ctx:
        _check("rmsnorm_fp8_strided", lib().rmsnorm_fp8_strided(
            rows, hidden, _DT[x.dtype], _ptr(x), xs, _ptr(residual), rs, _ptr(residual_out), ros, _ptr(gamma), eps,
            weight_offset, scale_ub, _FMT[out_fp8], _ptr(_u8(out)), os_, _DT[scales.dtype], _ptr(scales),
            _stream(x, stream)))
    return out, scales, residual_out


def rmsnorm_fp4quant_strided(x, gamma, residual=None, eps=1e-6, weight_offset=0.0, global_scale=None,
                             block_size=16, scale_format=None, swizzled=False, round_product=False, out=None,
                             block_scales=None, residual_out=None, stream=None):
    """rmsnorm_fp4quant / residual_rmsnorm_fp4quant on row-strided tensors
    (C: rmsnorm_fp4quant_strided).  Returns (packed, block_scales,
    residual_out or None)."""
    rows, xs = _row_view(x, "x")
    hidden = x.shape[-1]
    if scale_format is None:
        scale_format = "ue8m0" if block_size == 32 else "e4m3"
    sfmt = {"e4m3": SF_E4M3, "ue8m0": SF_UE8M0}[scale_format]
    if out is None:
        out = torch.empty((*x.shape[:-1], hidden // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        block_scales = (torch.empty((fp4_scale_bytes(rows, hidden, block_size, True),), dtype=torch.uint8,
                                    device=x.device) if swizzled else
                        torch.empty((*x.shape[:-1], hidden // block_size), dtype=torch.uint8, device=x.device))
    elif not block_scales.is_contiguous() or \
            block_scales.numel() * block_scales.element_size() < fp4_scale_bytes(rows, hidden, block_size, swizzled):
        raise ValueError("block_scales must be contiguous and hold fp4_scale_bytes() bytes")
    rs = ros = hidden
    if residual is not None:
        if residual.dtype != x.dtype or residual.shape != x.shape:
            raise ValueError("residual must match x in dtype and shape")
        if residual_out is None:
            residual_out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
        _, rs = _row_view(residual, "residual")
        _, ros = _row_view(residual_out, "residual_out")
    _, os_ = _row_view(_u8(out), "out")
    ctx = _device(x)
    _check_views(x, residual=residual, residual_out=residual_out, out=out, out_width=hidden // 2)
    _check_gamma(gamma, x, hidden)
    _gpu("block_scales", block_scales, x.device)
    _check_global_scale(global_scale, x.device)
    with ctx:
        _check("rmsnorm_fp4quant_strided", lib().rmsnorm_fp4quant_strided(
            rows, hidden, _DT[x.dtype], _ptr(x), xs, _ptr(residual), rs, _ptr(residual_out), ros, _ptr(gamma), eps,
            weight_offset, _ptr(global_scale), block_size, sfmt, SF_SWIZZLED if swizzled else SF_ROW_MAJOR,
            FP4_ROUND_PRODUCT if round_product else 0, _ptr(_u8(out)), os_, _ptr(_u8(block_scales)),
            _stream(x, stream)))
    return out, block_scales, residual_out


def convert(kind: int, src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """Elementwise device conversion (C: rmsq_convert); n = src.numel()."""
    n = src.numel()
    need = {CVT_F32_TO_E4M3FN: n, CVT_F32_TO_E4M3FNUZ: n, CVT_F32_TO_E2M1: (n + 1) // 2, CVT_F32_TO_BF16: 2 * n,
            CVT_F32_TO_F16: 2 * n, CVT_E4M3FN_TO_F32: 4 * n}.get(kind)
    src_esz = 1 if kind == CVT_E4M3FN_TO_F32 else 4
    ctx = _device(src)
    _gpu("dst", dst, src.device)
    if need is not None and (src.element_size() != src_esz or not src.is_contiguous() or not dst.is_contiguous()
                             or dst.numel() * dst.element_size() < need):
        raise ValueError("convert: src must be dense with the kind's input width, dst dense and large enough")
    with ctx:
        _check("rmsq_convert", lib().rmsq_convert(kind, _ptr(src), _ptr(dst), n, _stream(src, stream)))
    return dst


def set_tuning(waves_per_row: int = 0, vectors_per_lane: int = 0, grid_blocks: int = 0) -> None:
    """Process-wide launch-shape override (0 = automatic)."""
    _check("rmsq_set_tuning", lib().rmsq_set_tuning(waves_per_row, vectors_per_lane, grid_blocks))


def query_shape(rows: int, hidden: int, dtype: torch.dtype, fp4: bool = False, residual: bool = False,
                elementwise: bool = False, summed: bool = False) -> dict:
    """Launch shape of the FP8 (fp4=False) or FP4 path with or without a
    residual; for FP8 (any hidden) the vector / phased kernels' shape, with
    elementwise the element-wise kernel's (vectors_per_lane is then elements
    per lane; it does not depend on the residual), with summed
    allreduce_residual_rmsnorm_fp8's."""
    w, v, r = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    path = (2 if residual else 1) if fp4 else (6 if summed else 3 if elementwise else 5 if residual else 0)
    _check("rmsq_query_shape", lib().rmsq_query_shape(rows, hidden, _DT[dtype], path, ctypes.byref(w),
                                                      ctypes.byref(v), ctypes.byref(r)))
    return {"waves_per_row": w.value, "vectors_per_lane": v.value, "rows_per_block": r.value}
