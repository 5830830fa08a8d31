"""GPU parity of the NVFP4 quantizers: the library's weight and activation
quantizers must give the oracle's codes, scales and global scales bit for bit
(both take every code decision in fp32 with correct rounding)."""
import numpy as np
import pytest
import torch

import nvfp4_expert_layer_amd as nv
from oracle import nvfp4
from tests.gpu_helpers import log, require_gpu
from tests.oracle_helpers import to_f64

pytestmark = pytest.mark.gpu


def _weights(seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    w = torch.randn(4, 96, 256, generator=g, device="cuda")
    w[0] *= 0.02
    w[1, 5, 32:48] = 0.0                          # an all-zero block
    w[1, 6, :16] = 1e-30                          # underflows to scale 0 after /(6g)
    w[2] *= 3e4                                   # large values
    w[3] = torch.exp(torch.randn(96, 256, generator=g, device="cuda") * 4)   # wide dynamic range
    w[3, ::7] *= -1
    return w.to(torch.bfloat16)


def test_weight_quantizer_bit_exact():
    require_gpu()
    log("test_weight_quantizer_bit_exact: n=4 R=96 C=256")
    w = _weights(5)
    n, R, C = w.shape
    codes = torch.empty(n, R, C // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n, R, C // 16, dtype=torch.uint8, device="cuda")
    glob = torch.empty(n, dtype=torch.float32, device="cuda")
    nv.moe_nvfp4_quantize_weights(w, codes, scales, glob)
    torch.cuda.synchronize()
    for i in range(n):
        q = nvfp4.quantize_weight(to_f64(w[i]).astype(np.float32))
        assert glob[i].item() == float(q["g"]), i
        assert np.array_equal(scales[i].cpu().numpy(), q["scales"]), i
        assert np.array_equal(codes[i].cpu().numpy(), q["codes"]), i


def test_all_zero_weight_tensor_gets_global_one():
    require_gpu()
    w = torch.zeros(2, 16, 32, dtype=torch.bfloat16, device="cuda")
    codes = torch.full((2, 16, 16), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((2, 16, 2), 0xAA, dtype=torch.uint8, device="cuda")
    glob = torch.zeros(2, dtype=torch.float32, device="cuda")
    nv.moe_nvfp4_quantize_weights(w, codes, scales, glob)
    torch.cuda.synchronize()
    assert glob.tolist() == [1.0, 1.0]
    assert not codes.any().item() and not scales.any().item()


def _act_with_ties(seed):
    """Random activations plus blocks built so x / scale lands exactly on every
    E2M1 midpoint (ties) and past the saturation point."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(64, 512, generator=g, device="cuda") * 2.0
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75,
                         -2.5, -3.5, -5.0, -6.0], device="cuda")
    for r in range(8):
        s = 2.0 ** (r - 4)                        # block amax 6*s -> scale exactly s
        x[r, :16] = mids * s
        x[r, 16:32] = mids.flip(0) * s
    x[9, :16] = 0.0
    x[10, :16] = 0.03                             # amax/6 rounds to a subnormal E4M3 scale (3 * 2^-9)
    x[10, 5] = -0.021
    x[11, :16] = 1e-5                             # amax/6 rounds to scale 0 -> all-zero codes
    return x.to(torch.bfloat16)


def test_activation_quantizer_bit_exact_including_ties():
    require_gpu()
    log("test_activation_quantizer_bit_exact_including_ties: R=64 C=512")
    x = _act_with_ties(9)
    R, C = x.shape
    codes = torch.empty(R, C // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(R, C // 16, dtype=torch.uint8, device="cuda")
    nv.moe_nvfp4_quantize_activations(x, codes, scales)
    torch.cuda.synchronize()
    q = nvfp4.quantize_act(to_f64(x).astype(np.float32))
    assert np.array_equal(scales.cpu().numpy(), q["scales"])
    assert np.array_equal(codes.cpu().numpy(), q["codes"])
