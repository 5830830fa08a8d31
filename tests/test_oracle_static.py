"""Pins of the oracle's static W4A4 rule (a calibrated activation global g_a;
block scale E4M3(amax / (6 g_a)), code E2M1(x / (scale g_a)), value code *
scale * g_a): g_a = 1 reduces to dynamic W4A4; a power-of-two g_a only shifts
the binade; saturation and underflow follow their closed forms; the layer
matches the independent brute-force loops."""
import numpy as np
import pytest

from oracle import brute, moe, nvfp4
from tests.oracle_helpers import tiny_problem


def rows(seed, R=6, C=64, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((R, C)) * scale).astype(np.float32)


def test_unit_global_is_dynamic_w4a4():
    x = rows(1)
    a, b = nvfp4.quantize_act(x), nvfp4.quantize_act(x, 1.0)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    assert np.array_equal(nvfp4.fake_quant_act(x), nvfp4.fake_quant_act(x, 1.0))


@pytest.mark.parametrize("m", [-6, -3, 2, 5])
def test_power_of_two_global_shifts_the_binade(m):
    # with g = 2^m, quantizing x equals quantizing x / 2^m with g = 1, scaled
    # back by 2^m (every product and quotient is exact up to the shift, as long
    # as the block scales stay normal E4M3 numbers)
    g = np.float32(2.0 ** m)
    x = rows(2, scale=float(g))
    want = nvfp4.fake_quant_act((x / g).astype(np.float32)) * float(g)
    got = nvfp4.fake_quant_act(x, g)
    assert np.array_equal(got, want)
    qs = nvfp4.quantize_act(x, g)
    assert np.array_equal(qs["scales"], nvfp4.quantize_act((x / g).astype(np.float32))["scales"])


def test_saturation_clips_at_6_times_448_g():
    g = np.float32(0.01)
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 1e4, -1e4, 3.0                    # amax far above 6 * 448 * g = 26.88
    q = nvfp4.quantize_act(x, g)
    assert q["scales"][0, 0] == 0x7E                                # 448
    v = nvfp4.fake_quant_act(x, g)
    assert v[0, 0] == 6 * 448 * float(g) and v[0, 1] == -6 * 448 * float(g)
    # 3.0 / (448 g) = 0.6696 -> nearest E2M1 is 0.5
    assert v[0, 2] == 0.5 * 448 * float(g)


def test_small_block_underflows_to_zero():
    g = np.float32(1.0)
    x = np.full((1, 16), 1e-4, np.float32)                          # amax / 6 < 2^-10: scale rounds to 0
    q = nvfp4.quantize_act(x, g)
    assert q["scales"][0, 0] == 0 and not q["codes"].any()
    assert not nvfp4.fake_quant_act(x, g).any()
    # the same block with a smaller global is representable again
    v = nvfp4.fake_quant_act(x, np.float32(1e-5))
    assert np.allclose(v, 1e-4, rtol=0.1)


def test_matches_brute_force_rows():
    for seed, g in ((3, 0.37), (4, 1e-3), (5, 12.5)):
        x = rows(seed, R=3, C=48, scale=g * 300)
        got = nvfp4.fake_quant_act(x, np.float32(g))
        ref = np.array([brute.fake_quant_row(r.tolist(), g) for r in x])
        assert np.array_equal(got, ref), (seed, g)


@pytest.mark.parametrize("offset,L,with_shared", [(0, 8, True), (2, 3, False)])
def test_static_layer_matches_brute_force_loops(offset, L, with_shared):
    w, x, G, experts, shared = tiny_problem(seed=7)
    ag = (np.float32(0.0005), np.float32(0.0007))                  # small enough that some blocks saturate
    sh = shared if with_shared else None
    got = moe.forward(x, G, experts[offset:offset + L], sh, w.k, offset, L, moe.W4A4_STATIC, act_global=ag)["out"]
    ref = np.array(brute.layer(x.tolist(), G.tolist(), experts[offset:offset + L], sh, w.k, offset, L,
                               act_global=(float(ag[0]), float(ag[1]))))
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    dyn = moe.forward(x, G, experts[offset:offset + L], sh, w.k, offset, L, moe.W4A4)["out"]
    assert not np.allclose(got, dyn)                                # the globals matter here
    hq = moe.quantize_input(x, moe.W4A4_STATIC, ag)
    assert np.any(np.abs(hq) == 6 * 448 * float(ag[0]))            # some hidden blocks saturate


def test_static_with_unit_globals_is_the_dynamic_layer():
    w, x, G, experts, shared = tiny_problem(seed=9)
    a = moe.forward(x, G, experts, shared, w.k, 0, w.E, moe.W4A4)["out"]
    b = moe.forward(x, G, experts, shared, w.k, 0, w.E, moe.W4A4_STATIC, act_global=(1.0, 1.0))["out"]
    assert np.array_equal(a, b)
