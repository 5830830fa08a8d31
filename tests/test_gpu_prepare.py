"""Checkpoint preparation on the GPU (moe_nvfp4_prepare) against the oracle's
(oracle/checkpoint.py): checkpoints in both global-scale conventions and both
gate/up orders, written from NVFP4 experts, are prepared for an expert shard;
every prepared byte and global must equal the oracle's, nothing outside the
destination range may change, and a forward through the prepared shard must
match the forward through the original weights (bit for bit when the global is
stored as a multiplier; within the layer's tolerance of the oracle otherwise)."""
import numpy as np
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from oracle import checkpoint as ckp
from tests.gpu_helpers import Layer, log, rel_err, require_gpu, tol

pytestmark = pytest.mark.gpu

W4A16, W4A4 = workloads.W4A16, workloads.W4A4
KEYS = ("w13", "w13_scale", "w13_global", "w2", "w2_scale", "w2_global")

PREP = workloads.Workload("prepare", T=96, d=256, F=384, E=12, k=3, offset=4, L=6, has_shared=True,
                          mode=W4A16, hidden_seed=41, gate_seed=41, weight_seed=41, gate_std=0.05)


def host(experts):
    return {k: getattr(experts, k).cpu().numpy() for k in KEYS}


def checkpoint_arrays(kernel_layout, convention, order):
    """Host checkpoint written from kernel-layout experts: halves swapped for
    up-then-gate, globals stored as fp32(1 / g) for the inverse convention."""
    ck = {k: v.copy() for k, v in kernel_layout.items()}
    if order == ckp.UP_GATE:
        ck["w13"], ck["w13_scale"] = ckp.swap_halves(ck["w13"]), ckp.swap_halves(ck["w13_scale"])
    if convention == ckp.GLOBAL_INVERSE:
        for k in ("w13_global", "w2_global"):
            ck[k] = (np.float32(1) / ck[k]).astype(np.float32)
    return ck


def to_device(arrs):
    return nv.NVFP4Experts(*(torch.from_numpy(np.ascontiguousarray(arrs[k])).cuda() for k in KEYS))


@pytest.fixture(scope="module")
def layer():
    require_gpu()
    return Layer(PREP)


@pytest.mark.parametrize("convention", [ckp.GLOBAL_MULTIPLIER, ckp.GLOBAL_INVERSE])
@pytest.mark.parametrize("order", [ckp.GATE_UP, ckp.UP_GATE])
def test_prepare_matches_oracle_bit_for_bit(layer, convention, order):
    w = layer.w
    log(f"prepare convention={convention} order={order}")
    ck_h = checkpoint_arrays(host(layer.experts), convention, order)
    ck_d = to_device(ck_h)
    # destination: L experts plus one sentinel expert after them
    dst_all = nv.NVFP4Experts.empty(w.L + 1, w.d, w.F)
    for k in KEYS:
        t = getattr(dst_all, k)
        if t.dtype == torch.uint8:
            t.fill_(0xA5)
        else:
            t.fill_(-7.0)
    dst = dst_all.slice(0, w.L)
    nv.moe_nvfp4_prepare(ck_d, convention, order, w.offset, w.L, dst)
    torch.cuda.synchronize()
    ref = ckp.prepare(ck_h, convention, order, w.offset, w.L)
    got = host(dst_all)
    for k in KEYS:
        assert np.array_equal(got[k][:w.L].view(np.uint8), ref[k].view(np.uint8)), k
        if got[k].dtype == np.uint8:
            assert np.all(got[k][w.L] == 0xA5), f"{k}: wrote past the destination"
        else:
            assert got[k][w.L] == np.float32(-7.0), f"{k}: wrote past the destination"
    # the checkpoint is read only
    for k in KEYS:
        assert np.array_equal(getattr(ck_d, k).cpu().numpy().view(np.uint8), ck_h[k].view(np.uint8)), k


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("convention", [ckp.GLOBAL_MULTIPLIER, ckp.GLOBAL_INVERSE])
def test_forward_through_prepared_shard(layer, mode, convention):
    w = layer.w
    log(f"prepared forward mode={mode} convention={convention}")
    ck_d = to_device(checkpoint_arrays(host(layer.experts), convention, ckp.UP_GATE))
    dst = nv.NVFP4Experts.empty(w.L, w.d, w.F)
    nv.moe_nvfp4_prepare(ck_d, convention, ckp.UP_GATE, w.offset, w.L, dst)
    p = nv.make_problem(w.T, w.d, w.F, w.E, w.k, w.offset, w.L, True, mode)
    ws = nv.alloc_workspace(p)
    out = torch.empty(w.T, w.d, dtype=torch.bfloat16, device="cuda")
    nv.moe_nvfp4_forward(p, layer.x, layer.gate_w, dst, layer.shared, ws, out)
    torch.cuda.synchronize()
    base = layer.run(w.offset, w.L, True, mode)
    if convention == ckp.GLOBAL_MULTIPLIER:
        assert torch.equal(out, base)
    else:
        err = rel_err(out, layer.oracle_full(w.offset, w.L, True, mode)["out"])
        assert err <= tol(mode), err
        d = (out.float() - base.float()).norm() / base.float().norm()
        assert d.item() <= 2e-3, d.item()


def test_prepare_zero_experts_and_adjacent_destination(layer):
    w = layer.w
    log("prepare count=0 and destination adjacent to the checkpoint")
    kl = host(layer.experts)
    # one allocation per tensor: the checkpoint's E experts, then the destination's 2
    both = nv.NVFP4Experts.empty(w.E + 2, w.d, w.F)
    for k in KEYS:
        getattr(both, k)[:w.E].copy_(torch.from_numpy(kl[k]))
    ck_d, dst = both.slice(0, w.E), both.slice(w.E, 2)
    nv.moe_nvfp4_prepare(ck_d, ckp.GLOBAL_MULTIPLIER, ckp.GATE_UP, w.E - 2, 2, dst)
    before = host(both)
    nv.moe_nvfp4_prepare(ck_d, ckp.GLOBAL_MULTIPLIER, ckp.GATE_UP, 0, 0, dst)     # a no-op
    torch.cuda.synchronize()
    after = host(both)
    for k in KEYS:
        assert np.array_equal(after[k], before[k]), k
        assert np.array_equal(after[k][w.E:].view(np.uint8), kl[k][w.E - 2:].view(np.uint8)), k
    # a destination that overlaps the checkpoint is refused
    with pytest.raises(nv.MoeNvfp4Error):
        nv.moe_nvfp4_prepare(ck_d, ckp.GLOBAL_MULTIPLIER, ckp.GATE_UP, 0, 2, both.slice(w.E - 1, 2))
