"""The streaming reference kernel (rmsq_stream_probe) used as the bandwidth
reference in bench.py: it runs, writes exactly write_bytes of its destination
(guard bytes past the end keep their values) and reads only its source."""
import pytest
import torch

import fp4_activation_quantization_amd as rq
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.mark.parametrize("read_bytes,write_bytes", [
    (16, 16),                         # one vector each
    (134225920, 100696064),           # the 8192 x 4096 residual workload's split (4 : 3)
    (234895376, 66060288),            # the 16384 x 7168 FP4 workload's split (about 7 : 2)
    (4096 * 16 + 48, 16 * 3),         # ragged, read-heavy beyond 32 : 1
    (16 * 5, 4096 * 16 + 32),         # write-heavy
])
def test_stream_probe_writes_exactly_its_range(read_bytes, write_bytes):
    say(f"[stream] read {read_bytes} write {write_bytes}")
    src = torch.full((read_bytes + GUARD,), 7, dtype=torch.uint8, device=DEV)
    dst = torch.full((write_bytes + GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    before = src.clone()
    rq.stream_probe(src, read_bytes, dst, write_bytes)
    torch.cuda.synchronize()
    assert torch.equal(src, before)
    assert bool((dst[write_bytes:] == 0xA5).all())
    # every written vector holds the XOR of the source vectors a block read
    # (7s cancel in pairs) plus the chunk index: the range was written
    assert not bool((dst[:write_bytes] == 0xA5).all())
