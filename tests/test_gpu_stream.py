"""The streaming reference kernels (librmsq_probe) bench.py takes its
bandwidth ceiling from: they run, write exactly the bytes they are given
(guard bytes past the end keep their values) and only read their sources."""
import pytest
import torch

from fp4_activation_quantization_amd import probe
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.mark.parametrize("read_bytes,write_bytes,rv,wv,block,nl,per_cu,inter", [
    (16, 16, 1, 1, 256, 16, 0, False),                     # one vector each
    (134225920, 100696064, 4, 3, 256, 16, 0, False),       # the 8192 x 4096 residual workload's split
    (234895376, 66060288, 7, 2, 512, 8, 4, True),          # the 16384 x 7168 FP4 split, persistent, interleaved
    (4096 * 16 + 48, 16 * 3, 64, 1, 1024, 4, 0, True),     # ragged, read-heavy
    (16 * 5, 4096 * 16 + 32, 1, 64, 64, 1, 1, False),      # write-heavy
])
def test_chunk_probe_writes_exactly_its_range(read_bytes, write_bytes, rv, wv, block, nl, per_cu, inter):
    say(f"[chunk probe] read {read_bytes} write {write_bytes} rv:wv {rv}:{wv} block {block} nl {nl}")
    src = torch.full((read_bytes + GUARD,), 7, dtype=torch.uint8, device=DEV)
    dst = torch.full((write_bytes + GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    before = src.clone()
    probe.Chunks(src, read_bytes, dst, write_bytes, rv=rv, wv=wv, block=block, loads_in_flight=nl,
                 blocks_per_cu=per_cu, interleave=inter)()
    torch.cuda.synchronize()
    assert torch.equal(src, before)
    assert bool((dst[write_bytes:] == 0xA5).all())
    # each written vector is its lane's XOR of 7s plus the chunk index, never
    # the fill: every 16-byte vector of the range was written
    v = dst[:write_bytes].view(-1, 16)
    assert not bool((v == 0xA5).all(dim=1).any())


@pytest.mark.parametrize("rows,nin,row_bytes,outs,block,vpt,grid,phased,lds", [
    (1, 1, 16, [16, 4], 64, 1, 0, 0, 0),
    (300, 2, 16384, [16384, 8192, 4], 512, 2, 0, 3, 65536),  # the residual FP8 layout (bf16 8192 wide), phased, mapped
    (257, 1, 14336, [3584, 448], 256, 4, 64, 2, 40960),      # the FP4 layout (4-byte code pieces), a strided grid
    (33, 9, 8192, [8192, 4096, 4], 512, 1, 0, 1, 0),         # eight summed inputs and the residual
    (5, 2, 32768, [32768, 8192, 4], 1024, 2, 3, 3, 54272),   # fp32 rows: 4-byte code pieces
    (7, 1, 16384, [16384, 4096, 4], 256, 4, 0, 2, 0),
])
def test_row_probe_writes_exactly_its_rows(rows, nin, row_bytes, outs, block, vpt, grid, phased, lds):
    """phased carries both flag bits: 1 = barrier after the first output, 2 = mapped pieces."""
    say(f"[row probe] rows {rows} nin {nin} row {row_bytes} outs {outs} block {block} vpt {vpt} grid {grid} "
        f"phased {phased} lds {lds}")
    ins = [torch.full((rows * row_bytes + GUARD,), 3 + i, dtype=torch.uint8, device=DEV) for i in range(nin)]
    ous = [torch.full((rows * b + GUARD,), 0xA5, dtype=torch.uint8, device=DEV) for b in outs]
    before = [t.clone() for t in ins]
    probe.Rows(rows, ins, row_bytes, ous, outs, block=block, vpt=vpt, grid=grid, phased=bool(phased & 1),
               mapped=bool(phased & 2), lds_bytes=lds)()
    torch.cuda.synchronize()
    for t, b in zip(ins, before):
        assert torch.equal(t, b)
    for t, b in zip(ous, outs):
        assert bool((t[rows * b:] == 0xA5).all())
        gran = 16 if b % 16 == 0 else 4
        assert not bool((t[:rows * b].view(-1, gran) == 0xA5).all(dim=1).any())
