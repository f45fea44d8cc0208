"""The C ABI without a GPU: the library loads, exports every function that
include/rmsq.h declares, and rejects each invalid argument with its status
code before making any HIP call (so these run on a CPU-only machine).

Fake device pointers below are never dereferenced.  A module-wide fixture
forces a launch shape (one wave, one vector per lane) that cannot hold the
rows used here (hidden >= 1024), so a call that passes every argument check
stops with RMSQ_ERR_UNSUPPORTED instead of launching: that is how the tests
show a check was passed.
"""
import ctypes
import math
import os
import re

import pytest

import fp4_activation_quantization_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsq.h")

OK, NULL, DTYPE, SHAPE, ALIGN, VALUE, ALIAS, UNSUP = 0, -1, -2, -3, -4, -5, -6, -7
BASE = 1 << 32  # fake, 16-byte aligned addresses far apart
MB = 1 << 28


@pytest.fixture(autouse=True)
def no_launch_possible():
    rq.set_tuning(1, 1, 0)
    yield
    rq.set_tuning(0, 0, 0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int64_t|int|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for f in ("rmsnorm_fp8", "residual_rmsnorm_fp8", "allreduce_residual_rmsnorm_fp8", "gated_rmsnorm_fp8",
              "rmsnorm_fp4", "rmsnorm_fp4quant", "residual_rmsnorm_fp4quant",
              "rmsnorm_fp8_strided", "rmsnorm_fp4quant_strided", "rmsq_fp4_scale_bytes",
              "rmsq_convert",
              "rmsq_set_tuning", "rmsq_query_shape", "rmsq_status_string", "rmsq_abi_version",
              "rmsq_last_hip_error"):
        assert f in fns, f


def test_library_exports_every_declared_symbol():
    L = rq.lib()
    for f in declared_functions():
        assert hasattr(L, f), f"{f} declared in rmsq.h but not exported"


def test_abi_version_and_status_strings():
    L = rq.lib()
    assert L.rmsq_abi_version() == 1
    for code in range(-8, 1):
        assert L.rmsq_status_string(code) not in (None, b"", b"unknown status")
    assert L.rmsq_status_string(42) == b"unknown status"
    assert L.rmsq_last_hip_error() == 0


def P(i):
    return ctypes.c_void_p(BASE + i * MB)


def fp8(rows=4, hidden=4096, dt=rq.BF16, x=None, g=None, eps=1e-6, off=0.0, ub=1200.0, fmt=rq.E4M3FN, out=None,
        sdt=rq.F32, sc=None):
    x = P(0) if x is None else x
    g = P(1) if g is None else g
    out = P(2) if out is None else out
    sc = P(3) if sc is None else sc
    return rq.lib().rmsnorm_fp8(rows, hidden, dt, x, g, eps, off, ub, fmt, out, sdt, sc, None)


def rfp8(rows=4, hidden=4096, dt=rq.BF16, x=None, r=None, ro=None, g=None, out=None, sc=None, eps=1e-6):
    x = P(0) if x is None else x
    r = P(4) if r is None else r
    ro = P(5) if ro is None else ro
    g = P(1) if g is None else g
    out = P(2) if out is None else out
    sc = P(3) if sc is None else sc
    return rq.lib().residual_rmsnorm_fp8(rows, hidden, dt, x, r, ro, g, eps, 0.0, 1200.0, rq.E4M3FN, out, rq.F32,
                                         sc, None)


def fp4(rows=4, hidden=4096, dt=rq.BF16, x=None, g=None, gs=None, out=None, bs=None, eps=1e-6, off=0.0):
    x = P(0) if x is None else x
    g = P(1) if g is None else g
    out = P(2) if out is None else out
    bs = P(3) if bs is None else bs
    return rq.lib().rmsnorm_fp4(rows, hidden, dt, x, g, eps, off, gs, out, bs, None)


def gfp8(rows=4, hidden=4096, dt=rq.BF16, a=None, b=None, g=None, eps=1e-6, off=0.0, ub=1200.0, fmt=rq.E4M3FN,
         out=None, sdt=rq.F32, sc=None):
    a = P(0) if a is None else a
    b = P(4) if b is None else b
    g = P(1) if g is None else g
    out = P(2) if out is None else out
    sc = P(3) if sc is None else sc
    return rq.lib().gated_rmsnorm_fp8(rows, hidden, dt, a, b, g, eps, off, ub, fmt, out, sdt, sc, None)


def test_gated_argument_errors():
    """gated_rmsnorm_fp8 rejects before any launch (the forced one-wave shape
    cannot hold a valid call's row either: UNSUPPORTED, still no launch)."""
    assert gfp8(dt=9) == DTYPE and gfp8(sdt=5) == DTYPE and gfp8(fmt=3) == DTYPE
    assert gfp8(rows=-1) == SHAPE and gfp8(hidden=0) == SHAPE and gfp8(hidden=4100) == SHAPE
    assert gfp8(hidden=4102, dt=rq.F32) == SHAPE and gfp8(rows=1 << 62, hidden=1 << 20) == SHAPE
    assert gfp8(eps=-1.0) == VALUE and gfp8(ub=0.0) == VALUE and gfp8(off=math.nan) == VALUE
    assert gfp8(hidden=8 * 4096 + 8) == UNSUP and gfp8(hidden=4 * 4096 + 4, dt=rq.F32) == UNSUP
    assert gfp8(rows=0, a=ctypes.c_void_p(0)) == OK  # nothing to do
    z = ctypes.c_void_p(0)
    assert gfp8(a=z) == NULL and gfp8(b=z) == NULL and gfp8(g=z) == NULL and gfp8(out=z) == NULL
    assert gfp8(sc=z) == NULL
    odd = lambda i: ctypes.c_void_p(BASE + i * MB + 8)  # noqa: E731
    assert gfp8(a=odd(0)) == ALIGN and gfp8(b=odd(4)) == ALIGN and gfp8(g=odd(1)) == ALIGN
    assert gfp8(out=odd(2)) == ALIGN and gfp8(sc=ctypes.c_void_p(BASE + 3 * MB + 2)) == ALIGN
    assert gfp8(out=P(0)) == ALIAS and gfp8(sc=P(4)) == ALIAS and gfp8(out=P(1)) == ALIAS
    assert gfp8(sc=P(2)) == ALIAS
    assert gfp8(b=P(0)) == UNSUP  # a and b may be the same tensor
    assert gfp8() == UNSUP


def test_fp8_dtype_errors():
    assert fp8(dt=7) == DTYPE
    assert fp8(sdt=-1) == DTYPE
    assert fp8(fmt=2) == DTYPE


def test_fp8_shape_errors():
    assert fp8(rows=-1) == SHAPE
    assert fp8(hidden=0) == SHAPE
    assert fp8(hidden=-8) == SHAPE
    assert fp8(rows=1 << 62, hidden=1 << 20) == SHAPE
    # any width passes: rows that are not whole 16-byte vectors go to the
    # phased or element-wise kernel (which the forced one-wave shape cannot
    # hold either)
    assert fp8(hidden=4100) == UNSUP
    assert fp8(hidden=4102, dt=rq.F32) == UNSUP


def test_fp8_value_errors():
    for eps in (-1e-6, math.inf, math.nan):
        assert fp8(eps=eps) == VALUE
    for ub in (0.0, -1.0, math.nan):
        assert fp8(ub=ub) == VALUE
    for off in (math.inf, math.nan):
        assert fp8(off=off) == VALUE


def test_fp8_unsupported_width():
    assert fp8(hidden=8 * 4096 + 8) == UNSUP
    assert fp8(hidden=4 * 4096 + 4, dt=rq.F32) == UNSUP
    rq.set_tuning(0, 0, 0)  # automatic shapes: only the width limits remain
    try:
        assert fp8(hidden=32770) == UNSUP                   # contiguous: beyond the phased kernel
        off = ctypes.c_void_p(BASE + 2)                     # x off out's phase: the element-wise kernel
        assert fp8(hidden=16386, x=off) == UNSUP and fp8(hidden=16392, x=off) == UNSUP
    finally:
        rq.set_tuning(1, 1, 0)


def test_zero_rows_is_a_noop_even_with_null_pointers():
    z = ctypes.c_void_p(0)
    assert rq.lib().rmsnorm_fp8(0, 64, rq.BF16, z, z, 1e-6, 0.0, 1.0, rq.E4M3FN, z, rq.F32, z, None) == OK
    assert rq.lib().residual_rmsnorm_fp8(0, 64, rq.BF16, z, z, z, z, 1e-6, 0.0, 1.0, rq.E4M3FN, z, rq.F32, z,
                                         None) == OK
    assert rq.lib().rmsnorm_fp4(0, 64, rq.BF16, z, z, 1e-6, 0.0, z, z, z, None) == OK
    assert rq.lib().rmsq_convert(rq.CVT_F32_TO_E4M3FN, z, z, 0, None) == OK


def test_fp8_null_errors():
    z = ctypes.c_void_p(0)
    assert fp8(x=z) == NULL
    assert fp8(g=z) == NULL
    assert fp8(out=z) == NULL
    assert fp8(sc=z) == NULL
    assert rfp8(r=z) == NULL
    assert rfp8(ro=z) == NULL


def test_fp8_alignment_errors():
    # FP8 tensors need only element alignment (rows off 16-byte boundaries
    # take the element-wise kernel); codes have none
    odd = lambda i, k: ctypes.c_void_p(BASE + i * MB + k)
    assert fp8(x=odd(0, 1)) == ALIGN and fp8(x=odd(0, 2)) == UNSUP and fp8(x=odd(0, 8)) == UNSUP
    assert fp8(x=odd(0, 2), dt=rq.F32) == ALIGN and fp8(x=odd(0, 4), dt=rq.F32) == UNSUP
    assert fp8(g=odd(1, 1)) == ALIGN and fp8(g=odd(1, 2)) == UNSUP
    assert fp8(out=odd(2, 1)) == UNSUP
    assert fp8(sc=odd(3, 2)) == ALIGN                  # fp32 scales need 4 bytes
    assert fp8(sc=odd(3, 2), sdt=rq.BF16) == UNSUP     # bf16 scales need 2: all checks pass
    assert rfp8(r=odd(4, 1)) == ALIGN and rfp8(r=odd(4, 4)) == UNSUP
    assert rfp8(ro=odd(5, 3)) == ALIGN and rfp8(ro=odd(5, 4)) == UNSUP


def test_fp8_alias_errors():
    near = lambda i, k: ctypes.c_void_p(BASE + i * MB + k)
    assert fp8(out=near(0, 64)) == ALIAS     # codes inside x
    assert fp8(sc=near(2, 16)) == ALIAS      # scales inside codes
    assert fp8(out=near(1, 0)) == ALIAS      # codes over gamma
    assert rfp8(ro=near(0, 16)) == ALIAS     # partial overlap of residual_out and x
    assert rfp8(ro=near(4, 32)) == ALIAS     # partial overlap of residual_out and residual
    assert rfp8(ro=near(2, 0)) == ALIAS      # residual_out over the codes
    assert rfp8(ro=near(1, 0)) == ALIAS      # residual_out over gamma
    # exact in-place residual updates pass every check
    assert rfp8(ro=P(0)) == UNSUP
    assert rfp8(ro=P(4)) == UNSUP
    assert rfp8(x=P(4), r=P(4), ro=P(4)) == UNSUP
    assert fp8() == UNSUP and rfp8() == UNSUP and fp4() == UNSUP
    # in place over x while residual partially overlaps x
    assert rfp8(ro=P(0), r=near(0, 32)) == ALIAS


def test_fp4_errors():
    assert fp4(dt=rq.F32) == UNSUP   # fp32 input passes every check
    assert fp4(dt=9) == DTYPE
    assert fp4(hidden=24) == SHAPE
    assert fp4(hidden=0) == SHAPE
    assert fp4(rows=-2) == SHAPE
    assert fp4(eps=-1.0) == VALUE
    assert fp4(off=math.nan) == VALUE
    assert fp4(hidden=16 * 2048 + 16) == UNSUP
    z = ctypes.c_void_p(0)
    assert fp4(x=z) == NULL and fp4(bs=z) == NULL and fp4(out=z) == NULL and fp4(g=z) == NULL
    assert fp4(x=ctypes.c_void_p(BASE + 8)) == ALIGN
    assert fp4(gs=ctypes.c_void_p(BASE + 9 * MB + 2)) == ALIGN
    assert fp4(bs=ctypes.c_void_p(BASE + 2 * MB + 16)) == ALIAS
    assert fp4(gs=ctypes.c_void_p(BASE + 3 * MB)) == ALIAS


def fp4q(rows=4, hidden=4096, block=16, sfmt=None, layout=None, gs=None, out=None, bs=None, flags=0):
    sfmt = rq.SF_E4M3 if sfmt is None else sfmt
    layout = rq.SF_ROW_MAJOR if layout is None else layout
    out = P(2) if out is None else out
    bs = P(3) if bs is None else bs
    return rq.lib().rmsnorm_fp4quant(rows, hidden, rq.BF16, P(0), P(1), 1e-6, 0.0, gs, block, sfmt, layout, flags,
                                     out, bs, None)


def test_fp4quant_errors():
    assert fp4q(block=8) == VALUE
    assert fp4q(block=64) == VALUE
    assert fp4q(sfmt=2) == DTYPE
    assert fp4q(layout=2) == DTYPE
    assert fp4q(hidden=48, block=32) == SHAPE
    assert fp4q(flags=2) == VALUE and fp4q(flags=-1) == VALUE
    assert fp4q(flags=rq.FP4_ROUND_PRODUCT) == UNSUP
    for block in (16, 32):
        for sfmt in (rq.SF_E4M3, rq.SF_UE8M0):
            for layout in (rq.SF_ROW_MAJOR, rq.SF_SWIZZLED):
                assert fp4q(block=block, sfmt=sfmt, layout=layout) == UNSUP
    # UE8M0 scales never read the global scale: a misaligned one is not an error
    bad_gs = ctypes.c_void_p(BASE + 9 * MB + 2)
    assert fp4q(sfmt=rq.SF_E4M3, gs=bad_gs) == ALIGN
    assert fp4q(sfmt=rq.SF_UE8M0, gs=bad_gs) == UNSUP
    # the swizzled buffer covers whole 128 x 4 tiles: 32768 bytes here, against
    # 1024 row-major, so a buffer just below the codes overlaps only when swizzled
    below = ctypes.c_void_p(BASE + 2 * MB - 2048)
    assert fp4q(bs=below) == UNSUP
    assert fp4q(bs=below, layout=rq.SF_SWIZZLED) == ALIAS


def rfp4q(x=None, r=None, ro=None, g=None, out=None, bs=None, dt=rq.BF16, hidden=4096, gs=None):
    x = P(0) if x is None else x
    r = P(4) if r is None else r
    ro = P(5) if ro is None else ro
    g = P(1) if g is None else g
    out = P(2) if out is None else out
    bs = P(3) if bs is None else bs
    return rq.lib().residual_rmsnorm_fp4quant(4, hidden, dt, x, r, ro, g, 1e-6, 0.0, gs, 16, rq.SF_E4M3,
                                              rq.SF_ROW_MAJOR, 0, out, bs, None)


def test_residual_fp4quant_errors():
    z = ctypes.c_void_p(0)
    near = lambda i, k: ctypes.c_void_p(BASE + i * MB + k)
    assert rfp4q() == UNSUP and rfp4q(dt=rq.F32) == UNSUP
    assert rfp4q(r=z) == NULL and rfp4q(ro=z) == NULL
    assert rfp4q(r=near(4, 4)) == ALIGN and rfp4q(ro=near(5, 8)) == ALIGN
    assert rfp4q(ro=near(0, 16)) == ALIAS      # partial overlap with x
    assert rfp4q(ro=near(4, 32)) == ALIAS      # partial overlap with residual
    assert rfp4q(ro=P(2)) == ALIAS             # over the codes
    assert rfp4q(ro=P(3)) == ALIAS             # over the scales
    assert rfp4q(ro=P(1)) == ALIAS             # over gamma
    assert rfp4q(r=P(2)) == ALIAS              # residual under the codes
    assert rfp4q(gs=P(5)) == ALIAS             # global scale inside residual_out
    # exact in-place updates pass every check
    assert rfp4q(ro=P(0)) == UNSUP and rfp4q(ro=P(4)) == UNSUP
    L = rq.lib()
    q = lambda path: L.rmsq_query_shape(16384, 512, rq.BF16, path, None, None, None)  # fits the forced shape
    assert q(0) == OK and q(1) == OK and q(2) == OK and q(3) == OK and q(5) == OK and q(6) == OK
    assert q(4) == VALUE and q(7) == VALUE
    # FP8 takes any width: 513 elements need 65 vectors' lanes, one more than forced
    assert L.rmsq_query_shape(16384, 513, rq.BF16, 0, None, None, None) == UNSUP
    assert L.rmsq_query_shape(16384, 513, rq.BF16, 1, None, None, None) == SHAPE


def s8(x_stride=4096, r=None, r_stride=4096, ro=None, ro_stride=4096, out_stride=4096, dt=rq.BF16, x=None,
       out=None, hidden=4096):
    x = P(0) if x is None else x
    out = P(2) if out is None else out
    return rq.lib().rmsnorm_fp8_strided(4, hidden, dt, x, x_stride, r, r_stride, ro, ro_stride, P(1), 1e-6, 0.0,
                                        1200.0, rq.E4M3FN, out, out_stride, rq.F32, P(3), None)


def s4(x_stride=4096, out_stride=2048, r=None, r_stride=4096, ro=None, ro_stride=4096, dt=rq.BF16, out=None):
    out = P(2) if out is None else out
    return rq.lib().rmsnorm_fp4quant_strided(4, 4096, dt, P(0), x_stride, r, r_stride, ro, ro_stride, P(1), 1e-6,
                                             0.0, None, 16, rq.SF_E4M3, rq.SF_ROW_MAJOR, 0, out, out_stride, P(3),
                                             None)


def test_strided_argument_checks():
    assert s8() == UNSUP and s4() == UNSUP                      # contiguous strides pass
    assert s8(x_stride=8192, out_stride=8192) == UNSUP          # wider rows pass
    assert s8(x_stride=4095) == SHAPE                           # shorter than the row
    assert s8(x_stride=4100) == UNSUP                           # 8200 bytes: the element-wise kernel
    assert s8(out_stride=4095) == SHAPE and s8(out_stride=4100) == UNSUP
    assert s8(out_stride=4100, dt=rq.F32, hidden=4096, x_stride=4100) == UNSUP
    assert s8(r=P(4), r_stride=4100, ro=P(5)) == UNSUP
    assert s8(r=P(4), r_stride=4095, ro=P(5)) == SHAPE and s8(r=P(4), ro=P(5), ro_stride=4095) == SHAPE
    assert s4(out_stride=2047) == SHAPE and s4(out_stride=2052) == SHAPE and s4(out_stride=2056) == UNSUP
    # extents grow with the stride: 4 contiguous bf16 rows of 4096 span 32 KiB,
    # with rows 8192 elements apart they span 3 * 16 KiB + 8 KiB = 56 KiB
    after_x = ctypes.c_void_p(BASE + 32768)
    assert s8(out=after_x) == UNSUP
    assert s8(out=after_x, x_stride=8192) == ALIAS
    # residual_out over x is in place only with the same row stride
    assert s8(r=P(4), ro=P(0)) == UNSUP
    assert s8(r=P(4), ro=P(0), ro_stride=8192) == ALIAS
    assert s4(r=P(4), ro=P(4)) == UNSUP and s4(r=P(4), ro=P(4), r_stride=8192) == ALIAS


def ar8(n=2, inputs=None, rows=4, hidden=4096, dt=rq.BF16, r=None, ro=None, g=None, out=None, sc=None):
    ins = [P(6 + i) for i in range(n)] if inputs is None else inputs
    arr = (ctypes.c_void_p * max(1, len(ins)))(*ins)
    r = P(4) if r is None else r
    ro = P(5) if ro is None else ro
    g = P(1) if g is None else g
    out = P(2) if out is None else out
    sc = P(3) if sc is None else sc
    return rq.lib().allreduce_residual_rmsnorm_fp8(rows, hidden, dt, n, arr, r, ro, g, 1e-6, 0.0, 1200.0,
                                                  rq.E4M3FN, out, rq.F32, sc, None)


def test_allreduce_argument_checks():
    z = ctypes.c_void_p(0)
    assert ar8() == UNSUP and ar8(n=1) == UNSUP and ar8(n=8) == UNSUP   # every check passed
    assert ar8(n=0) == VALUE and ar8(n=9, inputs=[P(6 + i) for i in range(9)]) == VALUE
    assert ar8(inputs=[P(6), z]) == NULL and ar8(r=z) == NULL and ar8(ro=z) == NULL
    assert ar8(hidden=4100) == SHAPE and ar8(rows=-1) == SHAPE
    assert ar8(inputs=[P(6), ctypes.c_void_p(BASE + 7 * MB + 2)]) == ALIGN
    assert ar8(ro=P(4)) == UNSUP                       # in place over residual
    assert ar8(inputs=[P(6), P(6)]) == UNSUP           # inputs may share memory
    assert ar8(inputs=[P(6), P(4)]) == UNSUP           # and may be the residual (read only)
    assert ar8(ro=P(6)) == ALIAS                       # residual_out over an input
    assert ar8(out=P(7)) == ALIAS                      # codes over an input
    assert ar8(ro=ctypes.c_void_p(BASE + 4 * MB + 64)) == ALIAS   # partial overlap with residual
    assert ar8(rows=0, inputs=[z, z], r=z, ro=z) == OK


def test_fp4_scale_bytes():
    L = rq.lib()
    assert L.rmsq_fp4_scale_bytes(130, 80, 16, rq.SF_ROW_MAJOR) == 650
    assert L.rmsq_fp4_scale_bytes(130, 80, 16, rq.SF_SWIZZLED) == 2048   # 2 m-tiles x 2 k-tiles x 512
    assert L.rmsq_fp4_scale_bytes(16384, 7168, 32, rq.SF_SWIZZLED) == 128 * 56 * 512
    assert L.rmsq_fp4_scale_bytes(0, 7168, 16, rq.SF_SWIZZLED) == 0
    assert L.rmsq_fp4_scale_bytes(4, 64, 8, rq.SF_ROW_MAJOR) == VALUE
    assert L.rmsq_fp4_scale_bytes(4, 64, 16, 3) == DTYPE
    assert L.rmsq_fp4_scale_bytes(4, 24, 16, rq.SF_ROW_MAJOR) == SHAPE
    assert rq.fp4_scale_bytes(256, 4096, 32, swizzled=True) == 2 * 32 * 512


def test_convert_errors():
    L = rq.lib()
    assert L.rmsq_convert(99, P(0), P(1), 8, None) == DTYPE
    assert L.rmsq_convert(rq.CVT_F32_TO_E2M1, P(0), P(1), 7, None) == SHAPE
    assert L.rmsq_convert(rq.CVT_F32_TO_BF16, P(0), P(1), -1, None) == SHAPE
    assert L.rmsq_convert(rq.CVT_F32_TO_BF16, ctypes.c_void_p(0), P(1), 8, None) == NULL
    assert L.rmsq_convert(rq.CVT_F32_TO_BF16, ctypes.c_void_p(BASE + 4), P(1), 8, None) == ALIGN
    assert L.rmsq_convert(rq.CVT_F32_TO_BF16, P(0), ctypes.c_void_p(BASE + 16), 8, None) == ALIAS


def test_tuning_and_query_shape():
    L = rq.lib()
    assert L.rmsq_set_tuning(17, 0, 0) == VALUE
    assert L.rmsq_set_tuning(0, 8, 0) == VALUE
    assert L.rmsq_set_tuning(0, 0, -1) == VALUE
    rq.set_tuning(0, 0, 0)
    try:
        s = rq.query_shape(8192, 4096, rq.torch.bfloat16)
        assert s["waves_per_row"] * 64 * s["vectors_per_lane"] * 8 >= 4096
        # small batches: 2 vectors per lane over up to 16 waves
        assert rq.query_shape(1, 8192, rq.torch.float16) == {"waves_per_row": 8, "vectors_per_lane": 2,
                                                              "rows_per_block": 1}
        assert rq.query_shape(1, 16384, rq.torch.float32)["waves_per_row"] == 16
        assert rq.query_shape(1, 32768, rq.torch.bfloat16) == {"waves_per_row": 16, "vectors_per_lane": 4,
                                                               "rows_per_block": 1}
        assert rq.query_shape(1, 512, rq.torch.bfloat16) == {"waves_per_row": 1, "vectors_per_lane": 1,
                                                             "rows_per_block": 4}
        rq.set_tuning(1, 1, 0)
        with pytest.raises(rq.RmsqError):
            rq.query_shape(8, 4096, rq.torch.bfloat16)  # 64 lanes x 1 vector cannot hold 512 vectors
        rq.set_tuning(4, 4, 0)
        assert rq.query_shape(8, 4096, rq.torch.bfloat16)["rows_per_block"] == 1
        # the element-wise kernel takes the forced wave count, not the vectors
        rq.set_tuning(8, 4, 0)
        assert rq.query_shape(8, 4100, rq.torch.bfloat16, elementwise=True) == {
            "waves_per_row": 8, "vectors_per_lane": 12, "rows_per_block": 1}
        rq.set_tuning(0, 0, 0)
        # automatic element-wise shapes: the fewest element slots, ties to more waves
        assert rq.query_shape(512, 7, rq.torch.bfloat16, elementwise=True) == {
            "waves_per_row": 1, "vectors_per_lane": 1, "rows_per_block": 4}
        assert rq.query_shape(512, 100, rq.torch.float16, elementwise=True) == {
            "waves_per_row": 2, "vectors_per_lane": 1, "rows_per_block": 2}
        assert rq.query_shape(512, 4100, rq.torch.bfloat16, elementwise=True) == {
            "waves_per_row": 12, "vectors_per_lane": 8, "rows_per_block": 1}
        assert rq.query_shape(1, 16384, rq.torch.float32, elementwise=True) == {
            "waves_per_row": 16, "vectors_per_lane": 16, "rows_per_block": 1}
        for bad in (16385, 0):
            with pytest.raises(rq.RmsqError):
                rq.query_shape(1, bad, rq.torch.bfloat16, elementwise=True)
    finally:
        rq.set_tuning(1, 1, 0)


@pytest.mark.parametrize("fp4,residual", [(False, False), (False, True), (True, False), (True, True)])
def test_automatic_shape_fills_simds(fp4, residual):
    """Large batches get blocks of a multiple of 4 wavefronts whose lanes hold
    the row, with the fewest idle lanes among the allowed shapes (rows of
    more than 256 vectors: at least 4 waves, and, except for residual FP4,
    one vector per lane only at 4 waves)."""
    rq.set_tuning(0, 0, 0)
    try:
        for dt, epv in ((rq.torch.bfloat16, 8), (rq.torch.float16, 8), (rq.torch.float32, 4)):
            if fp4 and dt == rq.torch.float32:
                continue
            for hidden in range(64 * epv if not fp4 else 128, 4096 * epv + 1, 16 * epv):
                nvec = hidden // epv
                s = rq.query_shape(4096, hidden, dt, fp4, residual)
                w, v, r = s["waves_per_row"], s["vectors_per_lane"], s["rows_per_block"]
                if fp4 and not residual and dt != rq.torch.float32 and 256 < nvec <= 768:
                    # the wave-per-row FP4 kernel: one wavefront per row, 4 per
                    # block, the fewest compiled vectors per lane that hold it
                    assert (w, r) == (1, 4), (hidden, s)
                    assert v == min(vv for vv in (8, 12) if vv * 64 >= nvec), (hidden, s)
                    continue
                assert (w * r) % 4 == 0 and w * r <= 16, (hidden, s)
                assert r == (1 if w >= 4 else 4 // w), (hidden, s)
                idle = w * 64 * v - nvec
                assert idle >= 0, (hidden, s)
                allowed = [(ww, vv) for ww in (1, 2, 4, 8, 12, 16) for vv in (1, 2, 4)
                           if nvec <= 256 or (ww >= 4 and (vv > 1 or ww == 4 or (fp4 and residual)))]
                best = min(ww * 64 * vv - nvec for ww, vv in allowed if ww * 64 * vv >= nvec)
                assert idle == best, (hidden, s, best)
                if dt == rq.torch.float32 and residual and not fp4 and w == 16:
                    # fp32 residual FP8: 16-wave blocks only where nothing smaller holds the row
                    assert nvec > 12 * 64 * 4 or not any(ww < 16 and ww * 64 * vv >= nvec
                                                         and ww * 64 * vv - nvec == best for ww, vv in allowed)
                assert (w, v) in allowed, (hidden, s)
        # the measured preferences on ties
        q = lambda rows, h, dt, fp4=False, res=False: rq.query_shape(rows, h, dt, fp4, res)
        shape = lambda s: (s["waves_per_row"], s["vectors_per_lane"])
        assert shape(q(8192, 4096, rq.torch.bfloat16)) == (4, 2)
        assert shape(q(8192, 4096, rq.torch.bfloat16, res=True)) == (4, 2)
        assert shape(q(16384, 8192, rq.torch.bfloat16)) == (4, 4)
        assert shape(q(16384, 8192, rq.torch.bfloat16, res=True)) == (8, 2)
        assert shape(q(16384, 16384, rq.torch.bfloat16)) == (8, 4)
        assert shape(q(16384, 8192, rq.torch.float32, res=True)) == (8, 4)  # not 16 x 2: one such block per CU
        assert shape(q(16384, 7168, rq.torch.bfloat16, True)) == (4, 4)  # the block kernel
        assert shape(q(16384, 6144, rq.torch.bfloat16, True)) == (1, 12)  # the wave-per-row kernel
        assert shape(q(16384, 7168, rq.torch.bfloat16, True, True)) == (16, 1)
        assert shape(q(16384, 5120, rq.torch.bfloat16, True)) == (1, 12)
        assert shape(q(256, 7168, rq.torch.bfloat16, True)) == (7, 2)  # small batches: the block kernel, latency shape
        assert shape(q(16384, 16384, rq.torch.bfloat16, True, True)) == (16, 2)
    finally:
        rq.set_tuning(1, 1, 0)


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    """With the library absent the binding raises instead of computing anything."""
    monkeypatch.setattr(rq, "_lib", None)
    monkeypatch.setattr(rq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        rq.lib()


def test_binding_rejects_host_tensors():
    """The kernels get raw device pointers: the binding refuses tensors that
    are not on a GPU before anything reaches the library."""
    import torch

    x = torch.zeros(4, 1024, dtype=torch.bfloat16)
    g = torch.ones(1024, dtype=torch.bfloat16)
    for call in (lambda: rq.rmsnorm_fp8(x, g), lambda: rq.residual_rmsnorm_fp8(x, x.clone(), g),
                 lambda: rq.rmsnorm_fp4(x, g), lambda: rq.rmsnorm_fp4quant(x, g, block_size=32),
                 lambda: rq.residual_rmsnorm_fp4quant(x, x.clone(), g),
                 lambda: rq.allreduce_residual_rmsnorm_fp8([x.clone()], x, g),
                 lambda: rq.rmsnorm_fp8_strided(x, g), lambda: rq.rmsnorm_fp4quant_strided(x, g),
                 lambda: rq.convert(rq.CVT_F32_TO_E4M3FN, x.float(), torch.empty(4096, dtype=torch.uint8))):
        with pytest.raises(ValueError, match="GPU"):
            call()


def test_wide_rows_limits_and_shapes():
    """Rows of whole vectors above 4096 of them take the wide-row kernels (16
    waves, the row in LDS or registers) up to 10112 vectors; a forced shape other
    than 16 waves cannot hold them, and wider rows are refused before any
    launch."""
    bf, f32 = rq.torch.bfloat16, rq.torch.float32
    wide16, wide32 = 8 * 10112, 4 * 10112
    # the module's forced shape (1 wave x 1 vector) does not fit a wide row
    assert fp8(hidden=65536) == UNSUP and rfp8(hidden=65536) == UNSUP and fp4(hidden=65536) == UNSUP
    rq.set_tuning(0, 0, 0)
    try:
        assert fp8(hidden=wide16 + 8) == UNSUP and rfp8(hidden=wide16 + 8) == UNSUP
        assert fp8(hidden=wide32 + 4, dt=rq.F32) == UNSUP
        assert fp4(hidden=wide16 + 16) == UNSUP
        assert rq.query_shape(3, 65536, bf) == {"waves_per_row": 16, "vectors_per_lane": 8, "rows_per_block": 1}
        assert rq.query_shape(3, wide16, bf, fp4=True) == {"waves_per_row": 16, "vectors_per_lane": 10,
                                                            "rows_per_block": 1}
        assert rq.query_shape(3, wide32, f32, residual=True) == {"waves_per_row": 16, "vectors_per_lane": 10,
                                                                  "rows_per_block": 1}
        for kw in (dict(hidden=wide16 + 8), dict(hidden=65537), dict(hidden=65536, summed=True)):
            with pytest.raises(rq.RmsqError):
                rq.query_shape(3, kw.pop("hidden"), bf, **kw)
        rq.set_tuning(16, 0, 5)
        assert rq.query_shape(3, 65536, bf)["waves_per_row"] == 16
        for waves, vpt in ((8, 0), (0, 2)):
            rq.set_tuning(waves, vpt, 0)
            with pytest.raises(rq.RmsqError):
                rq.query_shape(3, 65536, bf)
    finally:
        rq.set_tuning(1, 1, 0)


def user_fp8(rows=4, hidden=4096, dt=rq.BF16, a=None, g=None, eps=1e-6, ub=1200.0, fmt=rq.E4M3FN, out=None,
             sdt=rq.F32, sc=None):
    """rmsq_fused.hpp's template, instantiated by a caller's translation unit
    (tests/cpp_source/user_source.hip); its checks, like the library's, run
    before any HIP call."""
    path = os.path.join(ROOT, "tests", "cpp_source", "libuser_source.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: __graft_entry__.build() builds it")
    L = ctypes.CDLL(path)
    Pt, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.user_abs_rmsnorm_fp8.argtypes = [I64, I64, I, Pt, Pt, F, F, F, I, Pt, I, Pt, Pt]
    L.user_abs_rmsnorm_fp8.restype = I
    a = P(0) if a is None else a
    g = P(1) if g is None else g
    out = P(2) if out is None else out
    sc = P(3) if sc is None else sc
    return L.user_abs_rmsnorm_fp8(rows, hidden, dt, a, g, eps, 0.0, ub, fmt, out, sdt, sc, None)


@pytest.fixture
def caller_links_no_launch():
    """The caller's library resolves rmsq_query_shape from the librmsq.so it
    was linked against, which is not the library the tests load when they run
    against a sanitized build: force the one-wave shape there too."""
    base = ctypes.CDLL(os.path.join(ROOT, "fp4_activation_quantization_amd", "librmsq.so"))
    base.rmsq_set_tuning(1, 1, 0)
    yield
    base.rmsq_set_tuning(0, 0, 0)


def test_public_template_argument_errors(caller_links_no_launch):
    assert user_fp8(sdt=5) == DTYPE and user_fp8(fmt=3) == DTYPE
    assert user_fp8(rows=-1) == SHAPE and user_fp8(hidden=4100) == SHAPE
    assert user_fp8(eps=-1.0) == VALUE and user_fp8(ub=0.0) == VALUE
    assert user_fp8(hidden=8 * 4096 + 8) == UNSUP
    z = ctypes.c_void_p(0)
    assert user_fp8(rows=0, g=z, out=z, sc=z) == OK  # nothing to do
    assert user_fp8(g=z) == NULL and user_fp8(out=z) == NULL and user_fp8(sc=z) == NULL
    near = lambda i, k: ctypes.c_void_p(BASE + i * MB + k)  # noqa: E731
    assert user_fp8(g=near(1, 8)) == ALIGN and user_fp8(out=near(2, 8)) == ALIGN
    assert user_fp8(sc=near(3, 2)) == ALIGN
    assert user_fp8(sc=near(2, 16)) == ALIAS     # scales inside the codes
    assert user_fp8(out=near(1, 0)) == ALIAS     # codes over gamma
    assert user_fp8(sc=near(1, 64)) == ALIAS     # scales inside gamma
    assert user_fp8(sc=near(2, 4 * 4096)) == UNSUP   # scales right after the last code: adjacent, no overlap
    assert user_fp8() == UNSUP
