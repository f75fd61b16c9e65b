"""The binding refuses operands that are not all on the input's GPU, and
rotation factors of the wrong shape, before any library call: a host pointer
or an undersized factor buffer handed to a kernel would fault the device.
Nothing here launches a kernel with a bad argument."""
import numpy as np
import pytest
import torch

import mxfp4_w4a4_quantized_amd as mx

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_mixed_device_operands_raise():
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device=DEV)
    c = torch.zeros((8, 64), dtype=torch.uint8, device=DEV)
    s = torch.zeros((8, 4), dtype=torch.uint8, device=DEV)
    ch, sh = c.cpu(), s.cpu()
    with pytest.raises(ValueError, match="codes"):
        mx.quantize_rotate(x, codes=torch.empty((4, 64), dtype=torch.uint8))
    with pytest.raises(ValueError, match="b_codes"):
        mx.gemm(c, s, ch, s)
    with pytest.raises(ValueError, match="y"):
        mx.gemm(c, s, c, s, y=torch.empty((8, 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="w_codes"):
        mx.linear_small(x, ch, sh)
    with pytest.raises(ValueError, match="b_scales"):
        mx.gemm_requant(c, s, c, sh)
    with pytest.raises(ValueError, match="device"):
        mx.quantize_rotate(x, mx.Kron(torch.eye(4), torch.eye(8, device=DEV)))


def test_bad_rotation_factors_raise():
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="one factor per column"):
        mx.quantize_rotate(x, mx.Smooth.from_host(np.ones(64, np.float32), DEV))
    with pytest.raises(ValueError, match="Kron"):
        mx.quantize_rotate(x, mx.Kron(torch.eye(4, device=DEV), torch.eye(4, device=DEV)))
    wc = torch.zeros((8, 64), dtype=torch.uint8, device=DEV)
    ws = torch.zeros((8, 4), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="one factor per column"):
        mx.linear_small(x, wc, ws, mx.Smooth.from_host(np.ones(256, np.float32), DEV))
