"""Checkpoint preparation, as the oracle computes it (test infrastructure only).

The page "Serving Solar Open 2 on DGX Spark", section "b12x 버전이 실제 NVFP4
체크포인트를 읽어들이도록 만들기", describes a loader that takes pre-quantized
NVFP4 checkpoints -- packed FP4 weights, FP8 block scales and per-expert global
scales -- in either of two conventions for the global scale (the served
checkpoint stores it as an inverse), copes with the row order of the fused
gate/up projection, and slices the scales of an expert shard.

The kernel layout this library consumes is the plain one (w13 rows [0, F) gate,
[F, 2F) up; global scale a multiplier), so preparation is:
  * experts [first, first + count) of the checkpoint;
  * w13 row halves swapped when the checkpoint stores up before gate;
  * the global scale as is (multiplier convention) or fp32(1 / stored) (inverse
    convention; one correctly rounded fp32 division, numpy's float32 divide);
  * codes and block scales copied bit for bit.
The page's loader also folds the global scale into the FP8 block scales with
re-rounding (clamped at 448) for its own kernels; this library keeps the fp32
global multiplier instead (applied after fp32 accumulation), so no re-rounding
takes place and the prepared weights decode to the checkpoint's values.
"""
import numpy as np

GLOBAL_MULTIPLIER, GLOBAL_INVERSE = 0, 1
GATE_UP, UP_GATE = 0, 1


def swap_halves(w13):
    """Rows [0, R/2) and [R/2, R) of every expert exchanged (axis 1)."""
    h = w13.shape[1] // 2
    return np.concatenate([w13[:, h:], w13[:, :h]], axis=1)


def prepare(ck, global_convention, w13_order, first, count):
    """ck: dict of numpy arrays w13 u8 [E, 2F, d/2], w13_scale u8 [E, 2F, d/16],
    w13_global f32 [E], w2 u8 [E, d, F/2], w2_scale u8 [E, d, F/16], w2_global
    f32 [E].  Returns the same keys for experts [first, first + count) in the
    kernel layout."""
    E = ck["w13"].shape[0]
    if not (0 <= first and count >= 0 and first + count <= E):
        raise ValueError("expert range outside the checkpoint")
    if global_convention not in (GLOBAL_MULTIPLIER, GLOBAL_INVERSE):
        raise ValueError("unknown global convention")
    if w13_order not in (GATE_UP, UP_GATE):
        raise ValueError("unknown w13 order")
    sl = slice(first, first + count)
    out = {k: np.array(v[sl], copy=True) for k, v in ck.items()}
    if w13_order == UP_GATE:
        out["w13"] = swap_halves(out["w13"])
        out["w13_scale"] = swap_halves(out["w13_scale"])
    if global_convention == GLOBAL_INVERSE:
        one = np.float32(1.0)
        out["w13_global"] = (one / out["w13_global"].astype(np.float32)).astype(np.float32)
        out["w2_global"] = (one / out["w2_global"].astype(np.float32)).astype(np.float32)
    return out
