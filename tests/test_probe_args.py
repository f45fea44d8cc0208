"""librmsq_probe's argument checks: every rejection happens before a launch,
so no device is needed.  The pointers are never dereferenced."""
import ctypes

from fp4_activation_quantization_amd import probe

BASE = 1 << 32
P = lambda off: ctypes.c_void_p(BASE + off)  # noqa: E731
NULL, RANGE, ALIGN = -1, -2, -3


def test_chunk_probe_rejections():
    L = probe.lib()
    ok = dict(rv=4, wv=3, block=256, nl=16, per_cu=0, inter=0)

    def call(src=P(0), rb=64, dst=P(1 << 20), wb=64, **kw):
        a = {**ok, **kw}
        return L.rmsq_probe_chunks(src, rb, dst, wb, a["rv"], a["wv"], a["block"], a["nl"], a["per_cu"],
                                   a["inter"], None)

    assert call(rb=0) == RANGE and call(wb=0) == RANGE and call(rb=24) == RANGE
    assert call(src=ctypes.c_void_p(0)) == NULL and call(dst=ctypes.c_void_p(0)) == NULL
    assert call(src=P(8)) == ALIGN
    assert call(dst=P(32)) == RANGE  # overlapping source and destination
    assert call(rv=0) == RANGE and call(wv=65) == RANGE and call(block=96) == RANGE and call(block=2048) == RANGE
    assert call(nl=3) == RANGE and call(per_cu=-1) == RANGE


def test_row_probe_rejections():
    L = probe.lib()
    I64 = ctypes.c_int64

    def call(rows=4, ins=(P(0),), row=1024, outs=(P(1 << 20),), ob=(512,), block=64, vpt=1, grid=0, phased=0, lds=0):
        ia = (ctypes.c_void_p * len(ins))(*ins)
        oa = (ctypes.c_void_p * len(outs))(*outs)
        ba = (I64 * len(ob))(*ob)
        return L.rmsq_probe_rows(rows, len(ins), ia, row, len(outs), oa, ba, block, vpt, grid, phased, lds, None)

    assert call(rows=-1) == RANGE and call(row=1000) == RANGE and call(row=0) == RANGE
    assert call(ins=(ctypes.c_void_p(0),)) == NULL and call(outs=(ctypes.c_void_p(0),)) == NULL
    assert call(ins=(P(4),)) == ALIGN and call(outs=(P(8),)) == ALIGN
    assert call(row=2048) == RANGE                     # 64 lanes x 1 vector cannot hold 2048 bytes
    assert call(vpt=3) == RANGE and call(block=100) == RANGE
    assert call(ins=(P(0),) * 9, vpt=2, block=64, row=2048) == RANGE  # 18 loads in flight per lane
    assert call(ins=(P(0),) * 10) == RANGE and call(outs=(P(1 << 20),) * 4, ob=(16,) * 4) == RANGE
    assert call(ob=(2048,)) == RANGE                   # a vector output wider than the input row
    assert call(ob=(6,)) == RANGE and call(ob=(260,)) == RANGE  # not a multiple of 4; more than 4 x block
    assert call(lds=-1) == RANGE and call(lds=64 * 1024 + 1) == RANGE and call(phased=4) == RANGE
    assert call(rows=0) == 0 and call(rows=0, phased=3, lds=65536) == 0  # nothing to do: no launch
