"""The one-launch small-batch layer (PATH_MICRO, 1..16 tokens) against the
oracle: whole output within 1e-2 (W4A16) / 3e-2 (W4A4), every mode, shards with
and without the shared expert, the tiny, mid and full-size layers; the grid
barrier's error word stays 0; graph replays match the eager call."""
import numpy as np
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from tests.gpu_helpers import Layer, log, rel_err, require_gpu, tol

pytestmark = pytest.mark.gpu

W4A16, W4A4, STATIC = workloads.W4A16, workloads.W4A4, workloads.W4A4_STATIC
MID = workloads.Workload("micro_mid", T=16, d=512, F=256, E=24, k=4, offset=0, L=24, has_shared=True,
                         mode=W4A16, hidden_seed=71, gate_seed=71, weight_seed=71, gate_std=0.05)
_layers = {}


def get(w):
    if w.name not in _layers:
        _layers[w.name] = Layer(w)
    return _layers[w.name]


def run_micro(lay, T, offset, L, shared, mode, act_global=(1.0, 1.0)):
    w = lay.w
    x = lay.x[:T].contiguous()
    p = nv.make_problem(T, w.d, w.F, w.E, w.k, offset, L, shared, mode, nv.PATH_MICRO, act_global)
    ws = nv.alloc_workspace(p)
    ws.fill_(0xFF)                                  # the launch must clear what it uses
    out = torch.full((T, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    nv.moe_nvfp4_forward(p, x, lay.gate_w, lay.local_weights(offset, L), lay.shared if shared else None, ws, out)
    torch.cuda.synchronize()
    err_word = int(ws[4:8].view(torch.int32).item())  # the barrier's error word (second dword of the workspace)
    assert err_word == 0, "a grid barrier timed out"
    return out


def oracle(lay, T, offset, L, shared, mode, act_global=(1.0, 1.0)):
    saved = lay.x, lay._x64
    lay.x, lay._x64 = lay.x[:T].contiguous(), None
    try:
        return lay.oracle_full(offset, L, shared, mode, act_global=act_global)["out"]
    finally:
        lay.x, lay._x64 = saved


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("T", [1, 3, 8, 16])
@pytest.mark.parametrize("offset,L,shared", [(0, 24, True), (8, 12, False)])
def test_micro_mid_layer(T, mode, offset, L, shared):
    require_gpu()
    lay = get(MID)
    log(f"micro mid T={T} mode={mode} offset={offset} L={L} shared={shared}")
    out = run_micro(lay, T, offset, L, shared, mode)
    err = rel_err(out, oracle(lay, T, offset, L, shared, mode))
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


def test_micro_tiny_workload_and_static():
    require_gpu()
    lay = get(workloads.WORKLOADS["tiny_w4a16"])
    w = lay.w
    for mode, ag in ((W4A16, (1.0, 1.0)), (W4A4, (1.0, 1.0)), (STATIC, (0.0021, 0.0043))):
        out = run_micro(lay, w.T, w.offset, w.L, w.has_shared, mode, ag)
        err = rel_err(out, oracle(lay, w.T, w.offset, w.L, w.has_shared, mode, ag))
        log(f"micro tiny T={w.T} mode={mode}: normwise rel err {err:.3e}")
        assert err <= tol(mode if mode != STATIC else W4A4)


_full = {}


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("T", [1, 5, 15, 16])
def test_micro_full_size_shard(T, mode):
    """The 4096 x 1024, 320-expert layer's first shard (160 experts + shared)."""
    require_gpu()
    if "lay" not in _full:
        _full["lay"] = Layer(workloads.WORKLOADS["decode_shard0_w4a16"], experts_range=(0, 160))
    lay = _full["lay"]
    log(f"micro full-size T={T} mode={mode}")
    out = run_micro(lay, T, 0, 160, True, mode)
    err = rel_err(out, oracle(lay, T, 0, 160, True, mode))
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


def test_micro_graph_replays_match_eager():
    """Captured once (reset kernel + persistent layer kernel), replayed with new
    token rows between replays; every replay equals the eager call on them."""
    require_gpu()
    from tests.test_gpu_graph import _graph_vs_eager
    lay = get(MID)
    assert _graph_vs_eager(lay, 0, lay.w.L, True, W4A16, nv.PATH_MICRO)
    assert _graph_vs_eager(lay, 8, 12, False, W4A4, nv.PATH_MICRO)
