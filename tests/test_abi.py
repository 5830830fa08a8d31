"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, and its device-free validation reports every error class."""
import os
import re

import pytest

import nvfp4_expert_layer_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_nvfp4_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = nv.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_and_last_error():
    assert nv.moe_nvfp4_strerror(0) == "ok"
    assert "workspace" in nv.moe_nvfp4_strerror(nv.ERR_WORKSPACE_TOO_SMALL)
    assert nv.moe_nvfp4_strerror(99) == "unknown status"


def good():
    return nv.make_problem(64, 4096, 1024, 320, 8, 0, 160, True, nv.W4A16)


def test_workspace_size_and_validation_ok():
    p = good()
    n = nv.moe_nvfp4_workspace_size(p)
    assert n > 64 * 8 * 4096 * 2              # at least the per-pair bf16 expert outputs
    assert nv.moe_nvfp4_validate(p, n, "gfx950:sramecc+:xnack-") == nv.OK
    assert nv.moe_nvfp4_validate(p, n, None) == nv.OK


@pytest.mark.parametrize("field,value,status", [
    ("num_tokens", -1, nv.ERR_INVALID_ARG),
    ("mode", 7, nv.ERR_INVALID_ARG),
    ("path", 9, nv.ERR_INVALID_ARG),
    ("has_shared", 2, nv.ERR_INVALID_ARG),
    ("top_k", 0, nv.ERR_INVALID_ARG),
    ("top_k", 33, nv.ERR_INVALID_ARG),
    ("num_local_experts", 0, nv.ERR_INVALID_ARG),
    ("local_expert_offset", -1, nv.ERR_INVALID_ARG),
    ("local_expert_offset", 161, nv.ERR_INVALID_ARG),          # 161 + 160 > 320
    ("num_experts", 2000, nv.ERR_UNSUPPORTED_SHAPE),
    ("d_model", 4000, nv.ERR_UNSUPPORTED_SHAPE),
    ("d_ff", 1000, nv.ERR_UNSUPPORTED_SHAPE),
    ("d_model", 64, nv.ERR_UNSUPPORTED_SHAPE),
])
def test_validation_errors(field, value, status):
    p = good()
    setattr(p, field, value)
    assert nv.moe_nvfp4_validate(p, 1 << 40, None) == status
    assert nv.moe_nvfp4_last_error() != ""


def test_top_k_above_num_experts_and_any_offset_binds():
    p = nv.make_problem(4, 256, 128, 6, 7, 0, 6, False, nv.W4A16)
    assert nv.moe_nvfp4_validate(p, 1 << 40, None) == nv.ERR_INVALID_ARG
    # any shard offset (scale tensors need no 16-expert alignment)
    for off in (0, 1, 3, 159, 160, 317):
        p = nv.make_problem(64, 4096, 1024, 320, 8, off, 320 - off if off > 160 else 3, True, nv.W4A4)
        assert nv.moe_nvfp4_validate(p, 1 << 40, None) == nv.OK


def test_workspace_too_small_and_arch():
    p = good()
    n = nv.moe_nvfp4_workspace_size(p)
    assert nv.moe_nvfp4_validate(p, n - 1, None) == nv.ERR_WORKSPACE_TOO_SMALL
    assert nv.moe_nvfp4_validate(p, n, "gfx942:sramecc+:xnack-") == nv.ERR_ARCH
    assert nv.moe_nvfp4_validate(p, n, "sm_121") == nv.ERR_ARCH


def test_workspace_grows_with_tokens_and_empty_batch_is_valid():
    small = nv.moe_nvfp4_workspace_size(nv.make_problem(64, 4096, 1024, 320, 8, 0, 160, True, nv.W4A4))
    big = nv.moe_nvfp4_workspace_size(nv.make_problem(8192, 4096, 1024, 320, 8, 0, 320, True, nv.W4A4))
    assert big > small
    p = nv.make_problem(0, 4096, 1024, 320, 8, 0, 160, True, nv.W4A16)
    assert nv.moe_nvfp4_validate(p, nv.moe_nvfp4_workspace_size(p), None) == nv.OK


def test_resolved_path_crossover():
    # expected local pairs per local expert T*k/E: W4A16 streams with the
    # block-diagonal kernels up to 3.9, with the dense ones up to 64 (d % 256
    # == 0), then tiles; W4A4 with NVFP4 activations (d, F multiples of 256, at
    # most 8192) up to 5 and 18; larger packed W4A4 streams up to 6; W4A4 whose
    # d or F is not a multiple of 256 streams up to 9
    def path(T, mode, d=4096, F=1024, force=nv.PATH_AUTO):
        return nv.moe_nvfp4_resolved_path(nv.make_problem(T, d, F, 320, 8, 0, 160, True, mode, force))
    assert path(64, nv.W4A16) == nv.PATH_DECODE
    assert path(156, nv.W4A16) == nv.PATH_DECODE          # 3.9
    assert path(157, nv.W4A16) == nv.PATH_MID
    assert path(2560, nv.W4A16) == nv.PATH_MID            # 64.0
    assert path(2561, nv.W4A16) == nv.PATH_PREFILL
    assert path(360, nv.W4A16, d=3968) == nv.PATH_DECODE  # d % 256 != 0: no dense path, threshold 9
    assert path(361, nv.W4A16, d=3968) == nv.PATH_PREFILL
    assert path(200, nv.W4A4) == nv.PATH_DECODE           # 5.0
    assert path(201, nv.W4A4) == nv.PATH_MID
    assert path(720, nv.W4A4) == nv.PATH_MID              # 18.0
    assert path(721, nv.W4A4) == nv.PATH_PREFILL
    assert path(240, nv.W4A4, d=16384) == nv.PATH_DECODE  # packed, beyond the dense path's 8192: 6.0
    assert path(241, nv.W4A4, d=16384) == nv.PATH_PREFILL
    assert path(300, nv.W4A4, F=384) == nv.PATH_DECODE    # not packed: threshold 9
    assert path(8192, nv.W4A16, force=nv.PATH_DECODE) == nv.PATH_DECODE
    assert path(1, nv.W4A4, force=nv.PATH_PREFILL) == nv.PATH_PREFILL
    assert path(1, nv.W4A4, force=nv.PATH_MID) == nv.PATH_MID
    with pytest.raises(nv.MoeNvfp4Error):
        path(64, nv.W4A16, d=100)


def test_static_globals_are_validated():
    # static W4A4 needs finite activation globals in 2^-100..2^100; other modes ignore them
    for bad in (0.0, -1.0, float("inf"), float("nan"), 1e-35, 1e35):
        p = nv.make_problem(64, 512, 256, 24, 4, 0, 24, True, nv.W4A4_STATIC, nv.PATH_AUTO, (bad, 1.0))
        assert nv.moe_nvfp4_validate(p, 1 << 30) == nv.ERR_INVALID_ARG
        p = nv.make_problem(64, 512, 256, 24, 4, 0, 24, True, nv.W4A4_STATIC, nv.PATH_AUTO, (1.0, bad))
        assert nv.moe_nvfp4_validate(p, 1 << 30) == nv.ERR_INVALID_ARG
    p = nv.make_problem(64, 512, 256, 24, 4, 0, 24, True, nv.W4A4_STATIC, nv.PATH_AUTO, (2.0 ** -100, 2.0 ** 100))
    assert nv.moe_nvfp4_validate(p, 1 << 30) == nv.OK
    p = nv.make_problem(64, 512, 256, 24, 4, 0, 24, True, nv.W4A4, nv.PATH_AUTO, (0.0, 0.0))
    assert nv.moe_nvfp4_validate(p, 1 << 30) == nv.OK
    # the static mode resolves its path like W4A4 and needs the same workspace
    ps = nv.make_problem(300, 4096, 1024, 320, 8, 0, 160, True, nv.W4A4_STATIC, nv.PATH_AUTO, (0.01, 0.01))
    pd = nv.make_problem(300, 4096, 1024, 320, 8, 0, 160, True, nv.W4A4)
    assert nv.moe_nvfp4_resolved_path(ps) == nv.moe_nvfp4_resolved_path(pd) == nv.PATH_MID
    assert nv.moe_nvfp4_workspace_size(ps) == nv.moe_nvfp4_workspace_size(pd)


def test_mid_path_needs_d_multiple_of_256():
    p = nv.make_problem(64, 384, 256, 16, 2, 0, 16, True, nv.W4A16, nv.PATH_MID)
    assert nv.moe_nvfp4_validate(p, 1 << 30, None) == nv.ERR_UNSUPPORTED_SHAPE
    p = nv.make_problem(64, 512, 256, 16, 2, 0, 16, True, nv.W4A16, nv.PATH_MID)
    assert nv.moe_nvfp4_validate(p, 1 << 30, None) == nv.OK
    assert nv.moe_nvfp4_resolved_path(p) == nv.PATH_MID
    bad = nv.make_problem(64, 512, 256, 16, 2, 0, 16, True, nv.W4A16, 5)
    assert nv.moe_nvfp4_validate(bad, 1 << 30, None) == nv.ERR_INVALID_ARG


def test_micro_path_limits():
    def st(T, d=4096, F=1024, E=320, k=8, L=160):
        return nv.moe_nvfp4_validate(nv.make_problem(T, d, F, E, k, 0, L, True, nv.W4A16, nv.PATH_MICRO), 1 << 30)
    assert st(1) == nv.OK and st(16) == nv.OK
    assert st(0) == nv.OK                                   # an empty batch enqueues nothing
    assert st(17) == nv.ERR_UNSUPPORTED_SHAPE
    assert st(8, d=8192) == nv.ERR_UNSUPPORTED_SHAPE
    assert st(8, F=8192) == nv.ERR_UNSUPPORTED_SHAPE
    assert st(8, d=384) == nv.ERR_UNSUPPORTED_SHAPE          # d % 256
    assert st(8, E=1024, k=32, L=1024) == nv.OK
