"""Pins of the oracle's checkpoint preparation (oracle/checkpoint.py): a
hand-computed single-expert example, round trips from the oracle's own
quantizer through both global-scale conventions and both gate/up orders,
correct rounding of the inverted global scale, and shard slicing."""
import numpy as np
import pytest

from oracle import checkpoint as ckp
from oracle import nvfp4
from tests.oracle_helpers import quantize_expert_oracle
import workloads


def _ck_from_experts(qs, convention, order):
    """A checkpoint in the given conventions, written from kernel-layout experts
    (the inverse of what preparation does): global stored as fp32(1 / g) for the
    inverse convention, w13 halves swapped for up-then-gate."""
    w13 = np.stack([q["w13"] for q in qs])
    w13s = np.stack([q["w13_scale"] for q in qs])
    if order == ckp.UP_GATE:
        w13, w13s = ckp.swap_halves(w13), ckp.swap_halves(w13s)
    g13 = np.array([q["g13"] for q in qs], dtype=np.float32)
    g2 = np.array([q["g2"] for q in qs], dtype=np.float32)
    if convention == ckp.GLOBAL_INVERSE:
        g13 = (np.float32(1) / g13).astype(np.float32)
        g2 = (np.float32(1) / g2).astype(np.float32)
    return {"w13": w13, "w13_scale": w13s, "w13_global": g13,
            "w2": np.stack([q["w2"] for q in qs]), "w2_scale": np.stack([q["w2_scale"] for q in qs]),
            "w2_global": g2}


def test_hand_example_inverse_and_up_gate():
    # one expert, d = 16, F = 1: w13 has an up row (first) and a gate row
    up_codes = np.array([[0x21, 0, 0, 0, 0, 0, 0, 0]], dtype=np.uint8)     # e0 = +0.5, e1 = +1.0
    gate_codes = np.array([[0x9F, 0, 0, 0, 0, 0, 0, 0]], dtype=np.uint8)   # e0 = -6 (0xF), e1 = -0.5 (0x9)
    ck = {"w13": np.concatenate([up_codes, gate_codes])[None],
          "w13_scale": np.array([[[0x38], [0x40]]], dtype=np.uint8),      # up scale 1.0, gate scale 2.0
          "w13_global": np.array([4.0], dtype=np.float32),                # stored inverse: g = 0.25
          "w2": np.zeros((1, 16, 0), dtype=np.uint8),
          "w2_scale": np.zeros((1, 16, 0), dtype=np.uint8),
          "w2_global": np.array([8.0], dtype=np.float32)}
    out = ckp.prepare(ck, ckp.GLOBAL_INVERSE, ckp.UP_GATE, 0, 1)
    assert out["w13_global"][0] == np.float32(0.25) and out["w2_global"][0] == np.float32(0.125)
    assert np.array_equal(out["w13"][0, 0], gate_codes[0]) and np.array_equal(out["w13"][0, 1], up_codes[0])
    w = nvfp4.dequantize(out["w13"][0], out["w13_scale"][0], out["w13_global"][0])
    assert w[0, 0] == -6 * 2.0 * 0.25 and w[0, 1] == -0.5 * 2.0 * 0.25      # gate row first
    assert w[1, 0] == 0.5 * 1.0 * 0.25 and w[1, 1] == 1.0 * 1.0 * 0.25
    assert np.all(w[:, 2:] == 0)


@pytest.fixture(scope="module")
def experts():
    w = workloads.Workload("ck", T=1, d=128, F=128, E=5, k=1, offset=0, L=5, has_shared=False,
                           mode=workloads.W4A16, hidden_seed=1, gate_seed=1, weight_seed=31)
    return [quantize_expert_oracle(*workloads.gen_expert(w, e)) for e in range(w.E)]


@pytest.mark.parametrize("convention", [ckp.GLOBAL_MULTIPLIER, ckp.GLOBAL_INVERSE])
@pytest.mark.parametrize("order", [ckp.GATE_UP, ckp.UP_GATE])
def test_round_trip_through_each_convention(experts, convention, order):
    ck = _ck_from_experts(experts, convention, order)
    out = ckp.prepare(ck, convention, order, 0, len(experts))
    for e, q in enumerate(experts):
        assert np.array_equal(out["w13"][e], q["w13"]) and np.array_equal(out["w13_scale"][e], q["w13_scale"])
        assert np.array_equal(out["w2"][e], q["w2"]) and np.array_equal(out["w2_scale"][e], q["w2_scale"])
        for key, g in (("w13_global", q["g13"]), ("w2_global", q["g2"])):
            if convention == ckp.GLOBAL_MULTIPLIER:
                assert out[key][e] == g
            else:   # two correctly rounded reciprocals: within one fp32 rounding of g
                assert abs(float(out[key][e]) / float(g) - 1.0) <= 2.0 ** -23
        ref = nvfp4.dequantize(q["w13"], q["w13_scale"], q["g13"])
        got = nvfp4.dequantize(out["w13"][e], out["w13_scale"][e], out["w13_global"][e])
        tol = 0.0 if convention == ckp.GLOBAL_MULTIPLIER else 2.0 ** -23
        assert np.all(np.abs(got - ref) <= tol * np.abs(ref))


def test_inverse_is_correctly_rounded(experts):
    rng = np.random.default_rng(5)
    stored = rng.uniform(0.5, 4000.0, size=1000).astype(np.float32)
    ck = {"w13": np.zeros((1000, 2, 8), np.uint8), "w13_scale": np.zeros((1000, 2, 1), np.uint8),
          "w13_global": stored, "w2": np.zeros((1000, 16, 1), np.uint8), "w2_scale": np.zeros((1000, 16, 0), np.uint8),
          "w2_global": stored}
    out = ckp.prepare(ck, ckp.GLOBAL_INVERSE, ckp.GATE_UP, 0, 1000)
    g = out["w13_global"].astype(np.float64)
    exact = 1.0 / stored.astype(np.float64)
    ulp = np.spacing(out["w13_global"]).astype(np.float64)
    assert np.all(np.abs(g - exact) <= 0.5 * ulp)


def test_shard_slice_equals_full_prepare_sliced(experts):
    ck = _ck_from_experts(experts, ckp.GLOBAL_INVERSE, ckp.UP_GATE)
    full = ckp.prepare(ck, ckp.GLOBAL_INVERSE, ckp.UP_GATE, 0, len(experts))
    part = ckp.prepare(ck, ckp.GLOBAL_INVERSE, ckp.UP_GATE, 2, 3)
    for k in full:
        assert np.array_equal(part[k], full[k][2:5])
    assert ckp.prepare(ck, ckp.GLOBAL_INVERSE, ckp.UP_GATE, 5, 0)["w13"].shape[0] == 0


def test_bad_arguments(experts):
    ck = _ck_from_experts(experts, ckp.GLOBAL_MULTIPLIER, ckp.GATE_UP)
    with pytest.raises(ValueError):
        ckp.prepare(ck, ckp.GLOBAL_MULTIPLIER, ckp.GATE_UP, 3, 3)
    with pytest.raises(ValueError):
        ckp.prepare(ck, 7, ckp.GATE_UP, 0, 1)
    with pytest.raises(ValueError):
        ckp.prepare(ck, ckp.GLOBAL_MULTIPLIER, 9, 0, 1)
