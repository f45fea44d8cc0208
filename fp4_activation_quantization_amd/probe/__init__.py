"""ctypes binding of librmsq_probe.so: the streaming reference kernels the
benchmark times beside the fused kernels (declared in rmsq_probe.h).  They
compute nothing; their rate is the streaming ceiling for a traffic pattern."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librmsq_probe.so")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with fp4_activation_quantization_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.rmsq_probe_chunks.argtypes = [P, I64, P, I64, I, I, I, I, I, I, P]
        L.rmsq_probe_chunks.restype = I
        L.rmsq_probe_rows.argtypes = [I64, I, ctypes.POINTER(P), I64, I, ctypes.POINTER(P), ctypes.POINTER(I64), I, I,
                                      I, I, I, P]
        L.rmsq_probe_rows.restype = I
        _lib = L
    return _lib


def _bytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _on_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("probe buffers must be contiguous GPU tensors")


class Chunks:
    """A chunk-probe launch with its arguments marshalled once."""

    def __init__(self, src: torch.Tensor, read_bytes: int, dst: torch.Tensor, write_bytes: int, *, rv: int, wv: int,
                 block: int = 256, loads_in_flight: int = 16, blocks_per_cu: int = 0, interleave: bool = False,
                 stream=None):
        _on_gpu(src, dst)
        if _bytes(src) < read_bytes or _bytes(dst) < write_bytes:
            raise ValueError("probe buffer smaller than its byte count")
        s = stream if stream is not None else torch.cuda.current_stream(src.device).cuda_stream
        self.args = (ctypes.c_void_p(src.data_ptr()), read_bytes, ctypes.c_void_p(dst.data_ptr()), write_bytes, rv, wv,
                     block, loads_in_flight, blocks_per_cu, int(interleave), ctypes.c_void_p(s))

    def __call__(self) -> None:
        rc = lib().rmsq_probe_chunks(*self.args)
        if rc != 0:
            raise RuntimeError(f"rmsq_probe_chunks returned {rc}")


class Rows:
    """A row-probe launch (the tensor layout of a fused row kernel) with its
    arguments marshalled once."""

    def __init__(self, rows: int, inputs: list[torch.Tensor], in_row_bytes: int, outputs: list[torch.Tensor],
                 out_row_bytes: list[int], *, block: int, vpt: int, grid: int = 0, phased: bool = False,
                 mapped: bool = False, lds_bytes: int = 0, stream=None):
        _on_gpu(*inputs, *outputs)
        if any(_bytes(t) < rows * in_row_bytes for t in inputs) or \
                any(_bytes(t) < rows * b for t, b in zip(outputs, out_row_bytes)) or len(outputs) != len(out_row_bytes):
            raise ValueError("probe buffer smaller than rows x its row bytes")
        P = ctypes.c_void_p
        self._ins = (P * len(inputs))(*[t.data_ptr() for t in inputs])
        self._outs = (P * len(outputs))(*[t.data_ptr() for t in outputs])
        self._ob = (ctypes.c_int64 * len(outputs))(*out_row_bytes)
        s = stream if stream is not None else torch.cuda.current_stream(inputs[0].device).cuda_stream
        self.args = (rows, len(inputs), self._ins, in_row_bytes, len(outputs), self._outs, self._ob, block, vpt, grid,
                     int(phased) | (2 if mapped else 0), lds_bytes, P(s))

    def __call__(self) -> None:
        rc = lib().rmsq_probe_rows(*self.args)
        if rc != 0:
            raise RuntimeError(f"rmsq_probe_rows returned {rc}")
