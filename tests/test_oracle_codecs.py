"""Pins of the oracle's NVFP4 codecs and quantizers against the format definition,
an independent library implementation of E4M3, exhaustive enumeration and
constructed round trips.  CPU only."""
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                rows.append((int(a, 0), float(b)))
    return rows


def test_e2m1_value_set_matches_format():
    rows = _read_pairs("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = nvfp4.e2m1_decode(np.array([code]))[0]
        assert got == val and np.signbit(got) == np.signbit(val) or (val == 0 and got == 0), code
    vals = set(float(v) for v in nvfp4.e2m1_decode(np.arange(16)))
    assert vals == {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0}


def test_e2m1_encode_inverts_decode():
    for code in range(16):
        v = nvfp4.e2m1_decode(np.array([code]))[0]
        want = 0 if code == 8 else code          # -0 encodes as +0
        assert nvfp4.e2m1_encode(np.array([v]))[0] == want


@pytest.mark.parametrize("v,want", [
    (0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0),
    (0.2499, 0.0), (0.2501, 0.5), (4.99, 4.0), (5.01, 6.0), (6.0, 6.0), (7.0, 6.0), (1e30, 6.0),
    (-0.25, 0.0), (-0.75, -1.0), (-5.0, -4.0), (-9.0, -6.0), (-0.1, 0.0),
])
def test_e2m1_rounding_ties_to_even_and_saturation(v, want):
    c = nvfp4.e2m1_encode(np.array([v], dtype=np.float64))[0]
    assert nvfp4.e2m1_decode(np.array([c]))[0] == want
    if want == 0.0:
        assert c == 0                               # zero magnitude -> +0 code


def test_e2m1_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-8, 8, 20000), np.arange(-7, 7.01, 0.125)])
    codes = nvfp4.e2m1_encode(v)
    allv = nvfp4.e2m1_decode(np.arange(16))
    for x, c in zip(v, codes):
        xs = min(max(x, -6.0), 6.0)
        d = np.abs(allv - xs)
        best = d.min()
        assert abs(nvfp4.e2m1_decode(np.array([c]))[0] - xs) == best
        cands = [cc for cc in range(16) if d[cc] == best and not (cc == 8)]
        if len(set(allv[cands])) > 1:               # a tie between two values: even magnitude code
            assert (c & 7) % 2 == 0


def test_e4m3_decode_matches_closed_form_golden_and_torch():
    for byte, val in _read_pairs("e4m3_landmarks.txt"):
        got = nvfp4.e4m3_decode(np.array([byte]))[0]
        assert got == val and np.signbit(got) == np.signbit(val)
    ours = nvfp4.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0


def test_e4m3_encode_matches_torch_cast_rne():
    rng = np.random.default_rng(7)
    v = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 200000)).astype(np.float32)
    grid = nvfp4.e4m3_decode(np.arange(127))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)          # exact midpoints
    v = np.concatenate([v, mids, grid.astype(np.float32), np.float32([0.0, 448.0])])
    ours = nvfp4.e4m3_encode_nonneg(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_at_448():
    v = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e9], dtype=np.float32)
    assert list(nvfp4.e4m3_encode_nonneg(v)) == [0x7E] * 6


def test_code_times_scale_is_exact_in_bf16():
    codes = nvfp4.e2m1_decode(np.arange(16))
    scales = nvfp4.e4m3_decode(np.arange(256))
    scales = scales[np.isfinite(scales)]
    prod = (codes[:, None] * scales[None, :]).reshape(-1)          # exact in fp64
    as_bf16 = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, prod)


def test_nibble_order_low_nibble_is_even_element():
    packed = nvfp4.pack_nibbles(np.array([[1, 2, 15, 8]], dtype=np.uint8))
    assert packed.tolist() == [[0x21, 0x8F]]
    assert nvfp4.unpack_nibbles(packed).tolist() == [[1, 2, 15, 8]]


def _grid_tensor(rng, R, C, g):
    """A tensor built on the NVFP4 grid: every block holds a +-6 code, so
    quantizing it must give back exactly its codes, scales and g."""
    nb = C // 16
    sbytes = rng.integers(0x08, 0x7F, size=(R, nb)).astype(np.uint8)    # normal scales
    codes = rng.integers(0, 16, size=(R, C)).astype(np.uint8)
    codes[codes == 8] = 0
    codes.reshape(R, nb, 16)[:, :, 3] = np.where(rng.random((R, nb)) < 0.5, 7, 15)
    sbytes[0, 0] = 0x7E                                  # the tensor amax block: scale 448
    codes[0, 3] = 7
    w = nvfp4.dequantize(nvfp4.pack_nibbles(codes), sbytes, g)
    return w, codes, sbytes


def test_quantize_weight_round_trip_on_grid():
    rng = np.random.default_rng(11)
    g = np.float32(2.0 ** -10)
    w, codes, sbytes = _grid_tensor(rng, 24, 96, g)
    q = nvfp4.quantize_weight(w.astype(np.float32))
    assert q["g"] == g
    assert np.array_equal(q["scales"], sbytes)
    assert np.array_equal(nvfp4.unpack_nibbles(q["codes"]), codes)
    # and quantizing the dequantized result again is a fixed point
    w2 = nvfp4.dequantize(q["codes"], q["scales"], q["g"])
    q2 = nvfp4.quantize_weight(w2.astype(np.float32))
    assert np.array_equal(q2["codes"], q["codes"]) and np.array_equal(q2["scales"], q["scales"])


def test_quantize_act_round_trip_on_grid():
    rng = np.random.default_rng(12)
    w, codes, sbytes = _grid_tensor(rng, 8, 64, np.float32(1.0))
    q = nvfp4.quantize_act(w.astype(np.float32))
    assert np.array_equal(q["scales"], sbytes)
    assert np.array_equal(nvfp4.unpack_nibbles(q["codes"]), codes)


def test_weight_amax_element_uses_scale_448_and_code_6():
    rng = np.random.default_rng(13)
    w = torch.randn(64, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    w = w.to(torch.float32).numpy()
    q = nvfp4.quantize_weight(w)
    r, c = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert q["g"] == np.float32(np.float32(np.abs(w).max()) / np.float32(2688.0))
    assert q["scales"][r, c // 16] == 0x7E
    assert nvfp4.unpack_nibbles(q["codes"])[r, c] & 7 == 7
    del rng


def test_quantization_error_within_half_grid_step():
    w = torch.randn(128, 256, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    w = w.to(torch.float32).numpy() * 0.05
    q = nvfp4.quantize_weight(w)
    deq = nvfp4.dequantize(q["codes"], q["scales"], q["g"])
    s = nvfp4.e4m3_decode(q["scales"]).repeat(16, axis=1) * float(q["g"])
    r = np.abs(w) / s
    step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    # half a grid step, plus slack for the fp32 rounding of w / (s*g)
    assert np.all(np.abs(w - deq) <= (0.5 * step + 1e-6) * s)
    # the scale is never too small: no element of a block exceeds 6 * s * g by more than rounding
    assert np.all(r <= 6.0 * (1 + 2 ** -3))


def test_all_zero_tensor_and_block():
    q = nvfp4.quantize_weight(np.zeros((2, 32), np.float32))
    assert q["g"] == 1.0 and not q["codes"].any() and not q["scales"].any()
    x = np.zeros((1, 32), np.float32)
    x[0, 20] = 3.0
    qa = nvfp4.quantize_act(x)
    assert qa["scales"][0, 0] == 0 and nvfp4.dequantize(qa["codes"], qa["scales"])[0, 20] == 3.0
