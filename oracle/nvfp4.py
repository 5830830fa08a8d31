"""NVFP4 codecs and quantizers, written from the format definition.

Test infrastructure only (see the package docstring).

Format (NVIDIA NVFP4; the page "Serving Solar Open 2 on DGX Spark", section
"b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록 만들기", names its three parts:
packed FP4 weights, FP8 block scales clamped to 448, a per-expert global scale):
  * element: E2M1, 4 bits `s e1 e0 m`; magnitude 0, 0.5 (subnormal) or
    2**(e-1) * (1 + m/2); value set {0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6}.
    Two codes per byte, the even element in the low nibble.
  * block scale: FP8 E4M3 "fn" (bias 7, subnormals m/8 * 2**-6, max 448,
    0x7F/0xFF NaN), one per 16 consecutive elements along the reduction axis.
  * global scale: one fp32 multiplier per tensor; a weight decodes as
    code * block_scale * global_scale.

Rounding (the plain reading of "round to nearest"): both encoders round to the
nearest representable value, ties to the even code, and saturate at the largest
finite value (448 for E4M3, 6 for E2M1).  A zero magnitude always encodes as the
+0 code.

Quantizer arithmetic that decides a code is done in fp32 (numpy float32
operations are IEEE single with round-to-nearest-even):
  weights:      g  = amax_tensor / 2688           (2688 = 6 * 448; g = 1 if amax = 0)
                s  = E4M3(amax_block / (6 * g))
                c  = E2M1(w / (s * g))            (c = 0 where s = 0)
  activations:  s  = E4M3(amax_block / 6)         (no global scale)
                c  = E2M1(x / s)
  static W4A4 activations (a calibrated per-tensor activation global g_a,
  fixed ahead of time; the page's "static" W4A4 variant names the idea and
  leaves the rule open -- read as the weight rule's block step with g = g_a):
                s  = E4M3(amax_block / (6 * g_a))
                c  = E2M1(x / (s * g_a))          value = c * s * g_a
"""
import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0
BLOCK = 16


# ----------------------------------------------------------------------------
# E2M1
# ----------------------------------------------------------------------------
def e2m1_magnitudes():
    """The 8 non-negative E2M1 values for magnitude codes 0..7, from the bit
    fields: exponent field e = code >> 1, mantissa bit m = code & 1."""
    out = np.empty(8, dtype=np.float64)
    for code in range(8):
        e, m = code >> 1, code & 1
        out[code] = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return out


_E2M1_MAG = e2m1_magnitudes()


def e2m1_decode(codes):
    """4-bit codes (any integer array, values 0..15) -> fp64 values."""
    codes = np.asarray(codes).astype(np.int64)
    mag = _E2M1_MAG[codes & 7]
    return np.where(codes & 8, -mag, mag)


def _round_to_grid(v, grid):
    """Round non-negative fp64 `v` to the nearest entry of the ascending `grid`
    whose indices are the codes; ties go to the even code; values at or above
    the top saturate.  Comparisons are against exact midpoints (each midpoint of
    these grids has few significant bits, so it is exact in fp64)."""
    v = np.asarray(v, dtype=np.float64)
    top = len(grid) - 1
    lo = np.searchsorted(grid, v, side="right") - 1          # grid[lo] <= v
    lo = np.clip(lo, 0, top)
    hi = np.minimum(lo + 1, top)
    mid = (grid[lo] + grid[hi]) * 0.5
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(v >= grid[top], top, code)
    return code.astype(np.int64)


def e2m1_encode(r):
    """fp32/fp64 values -> 4-bit codes, round-to-nearest-even, saturating at 6.
    Zero magnitude (after rounding) gives code 0 (+0).

    The magnitude code is the number of midpoints between neighbouring grid
    values that |r| lies above; at a midpoint exactly, it rounds up only when
    the upper neighbour has an even code.  Values past the last midpoint get
    code 7 (6.0), which is the saturation."""
    r = np.asarray(r)
    if r.dtype != np.float64:
        r = r.astype(np.float32)
    a = np.abs(r)
    mag_code = np.zeros(a.shape, dtype=np.uint8)
    for i in range(7):
        mid = (_E2M1_MAG[i] + _E2M1_MAG[i + 1]) * 0.5      # exact in fp32 and fp64
        up = (a >= mid) if (i + 1) % 2 == 0 else (a > mid)
        mag_code += up.astype(np.uint8)
    sign = (r < 0) & (mag_code != 0)
    return mag_code | np.where(sign, np.uint8(8), np.uint8(0))


# ----------------------------------------------------------------------------
# E4M3 (fn)
# ----------------------------------------------------------------------------
def e4m3_value(byte):
    """One E4M3fn byte -> fp64 by the closed form (NaN for 0x7F / 0xFF)."""
    s, e, m = (byte >> 7) & 1, (byte >> 3) & 15, byte & 7
    if e == 15 and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


_E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
_E4M3_POS = _E4M3_TABLE[:127].copy()     # codes 0x00..0x7E, ascending, finite


def e4m3_decode(bytes_):
    return _E4M3_TABLE[np.asarray(bytes_).astype(np.int64)]


def e4m3_encode_nonneg(v):
    """Non-negative fp32/fp64 values -> E4M3fn code bytes (0x00..0x7E),
    round-to-nearest-even on the code, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("block scales are non-negative and finite")
    return _round_to_grid(v, _E4M3_POS).astype(np.uint8)


# ----------------------------------------------------------------------------
# nibble packing: element 2i in the low nibble, 2i+1 in the high nibble
# ----------------------------------------------------------------------------
def pack_nibbles(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    return (codes[..., 0::2] & 15) | ((codes[..., 1::2] & 15) << 4)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


# ----------------------------------------------------------------------------
# quantizers (fp32 decisions)
# ----------------------------------------------------------------------------
def global_scale(w):
    """fp32 per-tensor scale g = amax / (6 * 448) (decode multiplier); 1 if the
    tensor is all zero."""
    amax = np.float32(np.max(np.abs(np.asarray(w, dtype=np.float32))))
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E2M1_MAX * E4M3_MAX))


def _quantize_rows(x32, g):
    """x32: fp32 [R, C] with C % 16 == 0; g: fp32 global scale.
    Returns (codes uint8 [R, C] unpacked, scale bytes uint8 [R, C/16])."""
    R, C = x32.shape
    blocks = x32.reshape(R, C // BLOCK, BLOCK)
    bmax = np.max(np.abs(blocks), axis=2)                       # fp32, exact
    denom6 = np.float32(np.float32(E2M1_MAX) * g)               # fp32 product
    v = (bmax / denom6).astype(np.float32)                      # fp32 division
    sbytes = e4m3_encode_nonneg(v)
    s = e4m3_decode(sbytes).astype(np.float32)                  # exact in fp32
    sg = (s * g).astype(np.float32)                             # fp32 product
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (blocks / sg[:, :, None]).astype(np.float32)        # fp32 division
    r = np.where(sg[:, :, None] > 0, r, np.float32(0))
    codes = e2m1_encode(r).reshape(R, C)
    return codes, sbytes.astype(np.uint8)


def quantize_weight(w):
    """One weight tensor [R, C] (bf16-exact values), blocks of 16 along C.
    Returns dict(codes=packed uint8 [R, C/2], scales=uint8 [R, C/16], g=fp32)."""
    w32 = np.asarray(w, dtype=np.float32)
    g = global_scale(w32)
    codes, sbytes = _quantize_rows(w32, g)
    return {"codes": pack_nibbles(codes), "scales": sbytes, "g": np.float32(g)}


def quantize_act(x, g=1.0):
    """Activations [R, C] (fp32 values), blocks of 16 along C; g = 1 (dynamic
    W4A4, no global scale) or a static activation global g_a (fp32).
    Returns dict(codes=packed uint8 [R, C/2], scales=uint8 [R, C/16])."""
    x32 = np.asarray(x, dtype=np.float32)
    codes, sbytes = _quantize_rows(x32, np.float32(g))
    return {"codes": pack_nibbles(codes), "scales": sbytes}


def dequantize(codes_packed, scales, g=1.0):
    """Exact fp64 value of NVFP4 data: code * block scale * global scale."""
    c = e2m1_decode(unpack_nibbles(codes_packed))
    s = e4m3_decode(scales)
    R, C = c.shape
    v = c.reshape(R, C // BLOCK, BLOCK) * s[:, :, None]
    return v.reshape(R, C) * np.float64(g)


def fake_quant_act(x, g=1.0):
    """Quantize then dequantize activations (the W4A4 activation step; g: the
    static activation global, 1 for dynamic W4A4)."""
    q = quantize_act(x, g)
    return dequantize(q["codes"], q["scales"], np.float32(g))
