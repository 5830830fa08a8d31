"""Static W4A4 on the GPU against the oracle: the activation quantizer with a
calibrated global bit for bit (codes and scales, saturating and underflowing
blocks included), the layer within the W4A4 tolerance on both kernel paths
(the packed tiled kernels, the 16-bit tiled kernels and weight streaming), at
the T=512 shard's full size on sampled rows, and unit globals equal to
dynamic W4A4 bit for bit.

The globals are calibrated the usual way, amax / (6 * 448), on the first 32
tokens of the batch (the hidden rows, and the SwiGLU output of those tokens
through the shared or first local expert, computed by the oracle), so the
rest of the batch can exceed the calibrated range and saturate."""
import numpy as np
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from oracle import moe, nvfp4
from tests.gpu_helpers import Layer, log, rel_err, require_gpu, tol
from tests.oracle_helpers import to_f64

pytestmark = pytest.mark.gpu

W4A4, STATIC = workloads.W4A4, nv.W4A4_STATIC

MID = workloads.Workload("mid_static", T=200, d=512, F=256, E=24, k=4, offset=0, L=24, has_shared=True,
                         mode=W4A4, hidden_seed=23, gate_seed=23, weight_seed=23, gate_std=0.05)
ODD = workloads.Workload("odd_static", T=150, d=384, F=384, E=8, k=2, offset=2, L=5, has_shared=True,
                         mode=W4A4, hidden_seed=29, gate_seed=29, weight_seed=29, gate_std=0.05)

_layers = {}


def get_layer(w, experts_range=None):
    if w.name not in _layers:
        _layers[w.name] = Layer(w, experts_range=experts_range)
    return _layers[w.name]


def calibrate(lay, n=32):
    """(g of h, g of the SwiGLU output): amax / 2688 over the first n tokens."""
    x = lay.x64[:n]
    g1 = nvfp4.global_scale(x)
    q = lay.oracle_expert(lay.w.E) if lay.w.has_shared else lay.oracle_expert(lay.w.offset)
    w13, _ = moe.dequant_expert(q)
    F = w13.shape[0] // 2
    u = nvfp4.fake_quant_act(x, g1) @ w13.T
    a = moe.silu(u[:, :F]) * u[:, F:]
    return g1, nvfp4.global_scale(a)


@pytest.mark.parametrize("g", [1.0, 0.37, 2.0 ** -9, 1e-3, 31.0])
def test_static_activation_quantizer_bit_exact(g):
    require_gpu()
    log(f"static activation quantizer g={g}")
    gen = torch.Generator(device="cuda").manual_seed(31)
    R, C = 48, 512
    x = (torch.randn(R, C, generator=gen, device="cuda") * 3.0).to(torch.bfloat16)
    x[0, :16] = 0                                     # an all-zero block
    x[1, :16] = 1e-6                                  # a block whose scale underflows for g >= 2^-9
    x[2, :16] = 4e4                                   # a block that saturates for g <= 1
    codes = torch.empty(R, C // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(R, C // 16, dtype=torch.uint8, device="cuda")
    nv.moe_nvfp4_quantize_activations_static(x, g, codes, scales)
    torch.cuda.synchronize()
    q = nvfp4.quantize_act(to_f64(x).astype(np.float32), np.float32(g))
    assert np.array_equal(scales.cpu().numpy(), q["scales"])
    assert np.array_equal(codes.cpu().numpy(), q["codes"])
    if g <= 1.0:
        assert q["scales"][2, 0] == 0x7E


@pytest.mark.parametrize("path", [nv.PATH_DECODE, nv.PATH_PREFILL, nv.PATH_MID])
@pytest.mark.parametrize("wl", [MID, ODD], ids=["packed", "f16"])
def test_static_layer_full_output(wl, path):
    if path == nv.PATH_MID and wl.d % 256:
        pytest.skip("the dense weight-streaming path needs d % 256 == 0")
    require_gpu()
    lay = get_layer(wl)
    w = lay.w
    ag = calibrate(lay)
    log(f"static layer {w.name} path={path} globals=({ag[0]:.4g}, {ag[1]:.4g})")
    out = lay.run(w.offset, w.L, w.has_shared, STATIC, path, act_global=ag)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, STATIC, act_global=ag)["out"]
    err = rel_err(out, ref)
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(W4A4)
    dyn = lay.oracle_full(w.offset, w.L, w.has_shared, W4A4)["out"]
    assert np.linalg.norm(dyn - ref) > 1e-3 * np.linalg.norm(ref)     # the globals change the result
    hq = moe.quantize_input(lay.x64, STATIC, ag)
    assert np.any(np.abs(hq) == 6 * 448 * float(ag[0]))                 # some hidden blocks saturate


@pytest.mark.parametrize("path", [nv.PATH_DECODE, nv.PATH_PREFILL, nv.PATH_MID])
def test_unit_globals_equal_dynamic_w4a4(path):
    require_gpu()
    lay = get_layer(MID)
    w = lay.w
    log(f"static with unit globals == dynamic, path={path}")
    a = lay.run(w.offset, w.L, w.has_shared, W4A4, path)
    b = lay.run(w.offset, w.L, w.has_shared, STATIC, path, act_global=(1.0, 1.0))
    assert torch.equal(a, b)


def test_static_full_size_t512_shard_whole_output():
    require_gpu()
    w = workloads.WORKLOADS["shard1_w4a4_t512"]
    lay = Layer(w, experts_range=(w.offset, w.L))
    ag = calibrate(lay)
    log(f"static T=512 shard, globals=({ag[0]:.4g}, {ag[1]:.4g}), path={nv.moe_nvfp4_resolved_path(nv.make_problem(w.T, w.d, w.F, w.E, w.k, w.offset, w.L, w.has_shared, STATIC))}")
    out = lay.run(w.offset, w.L, w.has_shared, STATIC, act_global=ag)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, STATIC, act_global=ag)
    err = rel_err(out, ref["out"])
    log(f"  whole-output normwise rel err {err:.3e}")
    assert err <= tol(W4A4)
