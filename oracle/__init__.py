"""Float64 CPU reference for fused (residual +) RMSNorm + FP8 / FP4 quantization.

TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the CPU
baseline leg of the benchmark may use this package; the library and its
Python binding never do.  It shares no code with the GPU path: the C source
next to this file rebuilds every format from its bit-level definition.

The arithmetic lives in ``rmsq_oracle.c`` (plain float64 C, one rounding per
operation as written); this module only marshals numpy arrays through ctypes
and splits rows across threads (rows are independent, so the split does not
change any result).

Definitions follow the Mojo API pages ``rms_norm_fused_fp8`` (argument list:
epsilon, weight_offset, scale_ub, per-row scales) and
``allreduce_residual_rmsnorm_fp8`` (residual and the pre-norm sum output), and
FlashInfer ``rmsnorm_fp4quant.py`` (sections "Constants", "FP8 E4M3
Intrinsics", "E2M1 Conversion", kernel phases 2 and 3).
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

# identifiers private to the oracle (the C file uses the same numbers)
F32, F16, BF16 = 0, 1, 2
E4M3FN, E4M3FNUZ, E2M1, UE8M0 = 0, 1, 2, 3
SF_E4M3, SF_UE8M0 = 0, 1  # FP4 block-scale formats

DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
FORMATS = {"e4m3fn": E4M3FN, "e4m3fnuz": E4M3FNUZ, "e2m1": E2M1, "ue8m0": UE8M0}
SCALE_FORMATS = {"e4m3": SF_E4M3, "ue8m0": SF_UE8M0}

_lib = None


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it with gcc if it is not there yet."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    L.oracle_rmsnorm_fp8.argtypes = [I64, I64, I, P, P, P, P, D, D, D, I, P, I, P, P, P]
    L.oracle_rmsnorm_fp8.restype = I
    L.oracle_rmsnorm_fp4.argtypes = [I64, I64, I, P, P, D, D, D, P, P, P, P]
    L.oracle_rmsnorm_fp4.restype = I
    L.oracle_rmsnorm_fp4q.argtypes = [I64, I64, I, P, P, P, P, D, D, D, I, I, I, P, P, P, P]
    L.oracle_rmsnorm_fp4q.restype = I
    L.oracle_rmsnorm_y.argtypes = [I64, I64, I, P, P, P, P, D, D, I, P, P]
    L.oracle_rmsnorm_y.restype = I
    L.oracle_rmsnorm_absmax.argtypes = [I64, I64, I, P, P, D, D]
    L.oracle_rmsnorm_absmax.restype = D
    L.oracle_sum_round.argtypes = [I, I, ctypes.POINTER(P), P, I64, P]
    L.oracle_encode_array.argtypes = [I, P, I64, P]
    L.oracle_decode_array.argtypes = [I, P, I64, P]
    L.oracle_round_array.argtypes = [I, P, I64, P]
    L.oracle_value_array.argtypes = [I, P, I64, P]
    L.oracle_encode.argtypes = [I, D]
    L.oracle_encode.restype = I
    L.oracle_decode.argtypes = [I, I]
    L.oracle_decode.restype = D
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bits_array(a, in_dtype: str) -> np.ndarray:
    """Raw element bits: float32 for f32, uint16 for f16/bf16."""
    want = np.float32 if in_dtype == "f32" else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"{in_dtype} data must be passed as {np.dtype(want).name} bits, got {a.dtype}")
    return a


def _default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _row_chunks(rows: int, threads: int):
    threads = max(1, min(threads, rows))
    step = (rows + threads - 1) // threads
    return [(r0, min(rows, r0 + step)) for r0 in range(0, rows, step)]


def rmsnorm_fp8(x, gamma, *, in_dtype: str, eps: float, weight_offset: float, scale_ub: float,
                out_fmt: str, scales_dtype: str, residual=None, threads: int | None = None,
                want_q: bool = True) -> dict:
    """Reference FP8 per-row path.  x/residual: [rows, hidden] bits; gamma: [hidden] bits.

    eps, weight_offset and scale_ub are taken as the fp32 values the GPU
    receives, widened to float64.  Returns codes [rows, hidden] (uint8),
    scales [rows] (bits in scales_dtype), residual_out bits (or None),
    q [rows, hidden] float64 (unrounded quantizer input) and sc [rows]
    float64 (unrounded scale after the clamp).
    """
    L = lib()
    x = _bits_array(x, in_dtype)
    g = _bits_array(gamma, in_dtype)
    rows, hidden = x.shape
    assert g.shape == (hidden,)
    res = _bits_array(residual, in_dtype) if residual is not None else None
    rout = np.empty_like(x) if res is not None else None
    codes = np.empty((rows, hidden), np.uint8)
    sc_np = np.float32 if scales_dtype == "f32" else np.uint16
    scales = np.empty((rows,), sc_np)
    q = np.empty((rows, hidden), np.float64) if want_q else None
    sc = np.empty((rows,), np.float64)
    e, o, u = (float(np.float32(v)) for v in (eps, weight_offset, scale_ub))

    def work(r0, r1):
        n = r1 - r0
        if n <= 0:
            return 0
        return L.oracle_rmsnorm_fp8(
            n, hidden, DTYPES[in_dtype], _ptr(x[r0:r1]),
            _ptr(res[r0:r1]) if res is not None else None,
            _ptr(rout[r0:r1]) if rout is not None else None,
            _ptr(g), e, o, u, FORMATS[out_fmt], _ptr(codes[r0:r1]), DTYPES[scales_dtype],
            _ptr(scales[r0:r1]), _ptr(q[r0:r1]) if q is not None else None, _ptr(sc[r0:r1]))

    _run(work, rows, threads)
    return {"codes": codes, "scales": scales, "residual_out": rout, "q": q, "sc": sc}


def sum_round(inputs, residual, *, in_dtype: str) -> np.ndarray:
    """round_to_in_dtype(residual + sum of inputs), the exact float64 sum
    rounded once (bits of in_dtype, residual's shape)."""
    res = _bits_array(residual, in_dtype)
    ins = [_bits_array(t, in_dtype) for t in inputs]
    assert ins and all(t.shape == res.shape for t in ins)
    out = np.empty_like(res)
    ptrs = (ctypes.c_void_p * len(ins))(*[t.ctypes.data for t in ins])
    lib().oracle_sum_round(DTYPES[in_dtype], len(ins), ptrs, _ptr(res), res.size, _ptr(out))
    return out


def allreduce_residual_rmsnorm_fp8(inputs, residual, gamma, *, in_dtype: str, eps: float, weight_offset: float,
                                   scale_ub: float, out_fmt: str, scales_dtype: str,
                                   threads: int | None = None, want_q: bool = True) -> dict:
    """Reference for the pre-norm sum over several input buffers: s =
    round(residual + sum of inputs) (sum_round), then the FP8 path on s
    (Mojo allreduce_residual_rmsnorm_fp8: residual_output is the pre-norm
    sum, which is what is normalized).  Returns rmsnorm_fp8's dict with
    residual_out = s."""
    s = sum_round(inputs, residual, in_dtype=in_dtype)
    ref = rmsnorm_fp8(s, gamma, in_dtype=in_dtype, eps=eps, weight_offset=weight_offset, scale_ub=scale_ub,
                      out_fmt=out_fmt, scales_dtype=scales_dtype, threads=threads, want_q=want_q)
    ref["residual_out"] = s
    return ref


def rmsnorm_fp4(x, gamma, *, in_dtype: str, eps: float, weight_offset: float, global_scale: float,
                threads: int | None = None, want_q: bool = True, block_size: int = 16,
                scale_format: str = "e4m3", residual=None, round_product: bool = False) -> dict:
    """Reference FP4 (E2M1) path with one scale per block of block_size (16 or
    32) elements: E4M3 scales (gs * amax / 6 clamped to 448) or UE8M0 scales
    (power of two >= amax / 6, no global scale).

    Returns packed [rows, hidden/2] (element 2k in the low nibble),
    block_scales [rows, hidden/block_size] (scale codes, row-major), q
    [rows, hidden] float64 and sf [rows, hidden/block_size] float64 (the
    unrounded block scale: after the clamp for E4M3, amax / 6 for UE8M0).
    With a residual, the row is s = round(x + residual) (also returned as
    residual_out bits) and the quantizer runs on it.  round_product: the FP4
    page's numerics, y = round_to_in_dtype(s * g') * rstd.
    """
    L = lib()
    x = _bits_array(x, in_dtype)
    g = _bits_array(gamma, in_dtype)
    rows, hidden = x.shape
    if block_size not in (16, 32) or scale_format not in SCALE_FORMATS:
        raise ValueError("block_size must be 16 or 32 and scale_format e4m3 or ue8m0")
    if hidden % block_size:
        raise ValueError(f"hidden must be a multiple of {block_size}")
    nblk = hidden // block_size
    packed = np.empty((rows, hidden // 2), np.uint8)
    bs = np.empty((rows, nblk), np.uint8)
    q = np.empty((rows, hidden), np.float64) if want_q else None
    sf = np.empty((rows, nblk), np.float64)
    e, o, gs = (float(np.float32(v)) for v in (eps, weight_offset, global_scale))
    sfmt = SCALE_FORMATS[scale_format]
    res = _bits_array(residual, in_dtype) if residual is not None else None
    rout = np.empty_like(x) if res is not None else None

    def work(r0, r1):
        n = r1 - r0
        if n <= 0:
            return 0
        return L.oracle_rmsnorm_fp4q(n, hidden, DTYPES[in_dtype], _ptr(x[r0:r1]),
                                     _ptr(res[r0:r1]) if res is not None else None,
                                     _ptr(rout[r0:r1]) if rout is not None else None, _ptr(g), e, o, gs,
                                     block_size, sfmt, int(round_product), _ptr(packed[r0:r1]), _ptr(bs[r0:r1]),
                                     _ptr(q[r0:r1]) if q is not None else None, _ptr(sf[r0:r1]))

    _run(work, rows, threads)
    return {"packed": packed, "block_scales": bs, "q": q, "sf": sf, "residual_out": rout}


# ---- swizzled scale layout ---------------------------------------------------
# FlashInfer "rmsnorm_fp4quant.py", the kernel's scale store and the API
# docstring: 128 x 4 tiles, flat offset
#   m_tile * (k_tiles * 512) + k_tile * 512 + outer_m * 16 + inner_m * 4 + inner_k
# with m_tile = row // 128, inner_m = (row % 128) // 32, outer_m = row % 32,
# k_tile = sf // 4, inner_k = sf % 4, k_tiles = ceil(sf_per_row / 4); the
# buffer holds ceil(rows / 128) * k_tiles * 512 bytes.  Positions of rows or
# scale columns past the ends (the tiles' padding) are not written.

def swizzled_size(rows: int, sf_per_row: int) -> int:
    return -(-rows // 128) * -(-sf_per_row // 4) * 512


def swizzled_offset(row, sf, sf_per_row: int):
    row = np.asarray(row, dtype=np.int64)
    sf = np.asarray(sf, dtype=np.int64)
    k_tiles = -(-sf_per_row // 4)
    return ((row // 128) * (k_tiles * 512) + (sf // 4) * 512 + (row % 32) * 16 + ((row % 128) // 32) * 4
            + sf % 4)


def swizzle_scales(block_scales: np.ndarray, out: np.ndarray | None = None, fill: int = 0) -> np.ndarray:
    """Place a row-major [rows, sf_per_row] scale matrix at its swizzled
    offsets; padding positions keep `out`'s bytes (or `fill`)."""
    rows, nsf = block_scales.shape
    if out is None:
        out = np.full(swizzled_size(rows, nsf), fill, np.uint8)
    r, c = np.meshgrid(np.arange(rows), np.arange(nsf), indexing="ij")
    out[swizzled_offset(r, c, nsf)] = block_scales
    return out


def rmsnorm_y(x, gamma, *, in_dtype: str, eps: float, weight_offset: float, residual=None,
              threads: int | None = None, round_product: bool = False) -> dict:
    """Normalized values y (float64), rstd per row and residual_out bits
    (round_product: the FP4 page-compatible y, see rmsnorm_fp4)."""
    L = lib()
    x = _bits_array(x, in_dtype)
    g = _bits_array(gamma, in_dtype)
    rows, hidden = x.shape
    res = _bits_array(residual, in_dtype) if residual is not None else None
    rout = np.empty_like(x) if res is not None else None
    y = np.empty((rows, hidden), np.float64)
    rstd = np.empty((rows,), np.float64)
    e, o = (float(np.float32(v)) for v in (eps, weight_offset))

    def work(r0, r1):
        n = r1 - r0
        if n <= 0:
            return 0
        return L.oracle_rmsnorm_y(n, hidden, DTYPES[in_dtype], _ptr(x[r0:r1]),
                                  _ptr(res[r0:r1]) if res is not None else None,
                                  _ptr(rout[r0:r1]) if rout is not None else None,
                                  _ptr(g), e, o, int(round_product), _ptr(y[r0:r1]), _ptr(rstd[r0:r1]))

    _run(work, rows, threads)
    return {"y": y, "rstd": rstd, "residual_out": rout}


def absmax(x, gamma, *, in_dtype: str, eps: float, weight_offset: float, threads: int | None = None) -> float:
    """max |y| over the whole tensor (no residual)."""
    L = lib()
    x = _bits_array(x, in_dtype)
    g = _bits_array(gamma, in_dtype)
    rows, hidden = x.shape
    e, o = (float(np.float32(v)) for v in (eps, weight_offset))
    chunks = _row_chunks(rows, threads or _default_threads())
    with ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(lambda c: L.oracle_rmsnorm_absmax(c[1] - c[0], hidden, DTYPES[in_dtype],
                                                              _ptr(x[c[0]:c[1]]), _ptr(g), e, o), chunks))
    return max(parts) if parts else 0.0


def _run(work, rows: int, threads: int | None):
    if rows == 0:
        return
    chunks = _row_chunks(rows, threads or _default_threads())
    if len(chunks) == 1:
        rc = [work(*chunks[0])]
    else:
        with ThreadPoolExecutor(len(chunks)) as ex:
            rc = list(ex.map(lambda c: work(*c), chunks))
    if any(rc):
        raise RuntimeError(f"oracle failed with status {rc}")


# ---- producers (rms_norm_fused_fp8's input_fn) ----------------------------

def gated_product(a, b, *, in_dtype: str) -> np.ndarray:
    """x = a * b element by element, rounded once to in_dtype (RNE); returns
    x's stored bits.  This is the producer gated_rmsnorm_fp8 puts in front of
    the normalization, in the place of the input_fn parameter of Mojo docs
    "rms_norm_fused_fp8" (the function that loads input values).  The float64
    product of two values of in_dtype is exact (at most 2 x 24 significant
    bits, and float64's exponent range holds it), so the one rounding is
    round_to's."""
    return round_to(in_dtype, value_of(in_dtype, a) * value_of(in_dtype, b))


# ---- codecs ---------------------------------------------------------------

def encode(fmt: str, values) -> np.ndarray:
    """Saturating round-to-nearest-even encode of float64 values to fmt codes."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_encode_array(FORMATS[fmt], _ptr(v), v.size, _ptr(out))
    return out


def decode(fmt: str, codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_decode_array(FORMATS[fmt], _ptr(c), c.size, _ptr(out))
    return out


def round_to(dtype: str, values) -> np.ndarray:
    """Round float64 values to dtype (RNE); returns the stored bits."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.float32 if dtype == "f32" else np.uint16)
    lib().oracle_round_array(DTYPES[dtype], _ptr(v), v.size, _ptr(out))
    return out


def value_of(dtype: str, bits) -> np.ndarray:
    """Exact float64 value of stored bits of dtype."""
    b = _bits_array(bits, dtype)
    out = np.empty(b.shape, np.float64)
    lib().oracle_value_array(DTYPES[dtype], _ptr(b), b.size, _ptr(out))
    return out


def format_max(fmt: str) -> float:
    return {"e4m3fn": 448.0, "e4m3fnuz": 240.0, "e2m1": 6.0}[fmt]
