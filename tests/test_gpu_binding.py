"""GPU: the Python binding refuses buffers whose sizes differ from what the
kernels write or read (the C ABI receives bare pointers and cannot check
them), before anything is launched; nothing is written to a refused buffer."""
import pytest
import torch

import fp4_activation_quantization_amd as rq
from gpu_common import DEV

pytestmark = pytest.mark.gpu


def _t(shape, dt=torch.bfloat16, fill=0):
    return torch.full(shape, fill, dtype=dt, device=DEV)


def test_fp8_buffers():
    x, g = _t((8, 1024), fill=1), _t((1024,), fill=1)
    small = _t((8, 1000), torch.uint8, 0xA5)
    cases = {
        "out too small": lambda: rq.rmsnorm_fp8(x, g, out=small),
        "gamma too short": lambda: rq.rmsnorm_fp8(x, _t((512,))),
        "gamma dtype": lambda: rq.rmsnorm_fp8(x, g.float()),
        "scales count": lambda: rq.rmsnorm_fp8(x, g, scales=_t((7,), torch.float32)),
        "scales dtype": lambda: rq.rmsnorm_fp8(x, g, scales=_t((8,), torch.int32)),
        "residual_out dtype": lambda: rq.residual_rmsnorm_fp8(x, x.clone(), g, residual_out=_t((8, 1024), torch.float16)),
        "out not contiguous": lambda: rq.rmsnorm_fp8(x, g, out=_t((1024, 8), torch.uint8).t()),
        "summed out": lambda: rq.allreduce_residual_rmsnorm_fp8([x], x.clone(), g, out=small),
        "strided out width": lambda: rq.rmsnorm_fp8_strided(x, g, out=small),
    }
    for name, call in cases.items():
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    assert torch.all(small == 0xA5), "a refused buffer was written"


def test_fp4_and_convert_buffers():
    x, g = _t((8, 1024), fill=1), _t((1024,), fill=1)
    cases = {
        "packed too small": lambda: rq.rmsnorm_fp4(x, g, out=_t((8, 500), torch.uint8)),
        "row-major scales too small": lambda: rq.rmsnorm_fp4quant(x, g, block_scales=_t((8, 60), torch.uint8)),
        "swizzled scales too small": lambda: rq.rmsnorm_fp4quant(x, g, swizzled=True,
                                                                 block_scales=_t((1000,), torch.uint8)),
        "global scale on host": lambda: rq.rmsnorm_fp4(x, g, global_scale=torch.ones(1)),
        "residual shape": lambda: rq.residual_rmsnorm_fp4quant(x, _t((8, 512)), g),
        "strided packed width": lambda: rq.rmsnorm_fp4quant_strided(x, g, out=_t((8, 1024), torch.uint8)),
        "convert dst too small": lambda: rq.convert(rq.CVT_F32_TO_BF16, _t((100,), torch.float32),
                                                    _t((100,), torch.uint8)),
    }
    for name, call in cases.items():
        with pytest.raises(ValueError):
            call()
