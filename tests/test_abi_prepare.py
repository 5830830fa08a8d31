"""moe_nvfp4_prepare's device-free argument checks, on the CPU.  The pointers are
fake, well separated, aligned addresses: every case here must be rejected
before anything is dereferenced or launched."""
import ctypes

import pytest

import nvfp4_expert_layer_amd as nv

E, D, F = 8, 256, 128
SRC = [0x1000_0000_0000 + i * 0x1000_0000 for i in range(6)]
DST = [0x2000_0000_0000 + i * 0x1000_0000 for i in range(6)]


def call(ck_over=None, dst_over=None, first=0, count=4, null_ck=False, null_dst=False):
    f = dict(zip(("w13", "w13_scale", "w13_global", "w2", "w2_scale", "w2_global"), SRC))
    f.update(num_experts=E, d_model=D, d_ff=F, global_convention=nv.GLOBAL_INVERSE, w13_order=nv.UP_GATE)
    f.update(ck_over or {})
    ck = nv.moe_nvfp4_checkpoint(f["w13"], f["w13_scale"], f["w13_global"], f["w2"], f["w2_scale"],
                                 f["w2_global"], f["num_experts"], f["d_model"], f["d_ff"],
                                 f["global_convention"], f["w13_order"])
    dp = dict(zip(("w13", "w13_scale", "w13_global", "w2", "w2_scale", "w2_global"), DST))
    dp.update(dst_over or {})
    dw = nv.moe_nvfp4_weights(dp["w13"], dp["w13_scale"], dp["w13_global"], dp["w2"], dp["w2_scale"],
                              dp["w2_global"])
    return nv.lib().moe_nvfp4_prepare(None if null_ck else ctypes.byref(ck), first, count,
                                      None if null_dst else ctypes.byref(dw), None)


@pytest.mark.parametrize("kw,status", [
    (dict(null_ck=True), nv.ERR_INVALID_ARG),
    (dict(null_dst=True), nv.ERR_INVALID_ARG),
    (dict(ck_over={"d_model": 200}), nv.ERR_UNSUPPORTED_SHAPE),
    (dict(ck_over={"d_model": 32768}), nv.ERR_UNSUPPORTED_SHAPE),
    (dict(ck_over={"d_ff": 64}), nv.ERR_UNSUPPORTED_SHAPE),
    (dict(ck_over={"global_convention": 2}), nv.ERR_INVALID_ARG),
    (dict(ck_over={"w13_order": -1}), nv.ERR_INVALID_ARG),
    (dict(ck_over={"num_experts": 0}, count=0), nv.ERR_INVALID_ARG),
    (dict(first=-1), nv.ERR_INVALID_ARG),
    (dict(count=-1), nv.ERR_INVALID_ARG),
    (dict(first=5, count=4), nv.ERR_INVALID_ARG),
    (dict(first=2**31 - 1, count=2), nv.ERR_INVALID_ARG),
    (dict(ck_over={"num_experts": 70000}, count=65536), nv.ERR_INVALID_ARG),
    (dict(ck_over={"w13": 0}), nv.ERR_INVALID_ARG),
    (dict(ck_over={"w2_scale": SRC[4] + 8}), nv.ERR_INVALID_ARG),        # codes/scales 16-byte aligned
    (dict(ck_over={"w13_global": SRC[2] + 2}), nv.ERR_INVALID_ARG),      # fp32 4-byte aligned
    (dict(dst_over={"w2_global": 0}), nv.ERR_INVALID_ARG),
    (dict(dst_over={"w13": DST[0] + 4}), nv.ERR_INVALID_ARG),
    (dict(dst_over={"w13": SRC[0] + 3 * 2 * F * (D // 2)}), nv.ERR_INVALID_ARG),   # inside expert 3
    (dict(dst_over={"w2_global": SRC[5] + 4 * 7}), nv.ERR_INVALID_ARG),
])
def test_prepare_rejects(kw, status):
    assert call(**kw) == status
    assert nv.moe_nvfp4_last_error() != ""

