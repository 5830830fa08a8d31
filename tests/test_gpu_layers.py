"""One workspace serving many layers in turn (the page's shared scratch pool:
"수정 사항 › b12x에서의 Expert Parallelism 구현 추가" replaces a per-layer
workspace of every MoE layer by one module-level pool).  A stack of layers with
different weights, shapes and modes runs back to back on a single workspace,
eagerly and captured as one HIP graph; every layer's output must equal the same
layer run alone on a fresh workspace, bit for bit (nothing of one call's scratch
state may leak into the next)."""
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from tests.gpu_helpers import Layer, log, require_gpu

pytestmark = pytest.mark.gpu

W4A16, W4A4, STATIC = workloads.W4A16, workloads.W4A4, workloads.W4A4_STATIC


def stack():
    """Twelve small layers: three shapes, all modes, every kernel path."""
    out = []
    shapes = [(96, 512, 256, 24, 4), (40, 256, 384, 16, 2), (300, 512, 512, 8, 2)]
    for i in range(12):
        T, d, F, E, k = shapes[i % 3]
        mode = (W4A16, W4A4, STATIC)[i % 3 if i < 9 else (i + 1) % 3]
        w = workloads.Workload(f"stack{i}", T=T, d=d, F=F, E=E, k=k, offset=(i % 2) * (E // 2), L=E // 2,
                               has_shared=i % 2 == 0, mode=mode, hidden_seed=300 + i, gate_seed=300 + i,
                               weight_seed=300 + i, gate_std=0.05,
                               act_global=(0.0021, 0.0043) if mode == STATIC else (1.0, 1.0))
        path = (nv.PATH_DECODE, nv.PATH_PREFILL, nv.PATH_MID, nv.PATH_AUTO)[i % 4]
        out.append((Layer(w, experts_range=(w.offset, w.L)), path))
    return out


def problem(lay, path):
    w = lay.w
    return nv.make_problem(w.T, w.d, w.F, w.E, w.k, w.offset, w.L, w.has_shared, w.mode, path, w.act_global)


def test_one_workspace_for_a_stack_of_layers():
    require_gpu()
    layers = stack()
    probs = [problem(l, p) for l, p in layers]
    size = max(nv.moe_nvfp4_workspace_size(p) for p in probs)
    log(f"{len(layers)} layers, shared workspace {size} bytes")
    ws = torch.empty(size, dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    outs = [torch.empty(l.w.T, l.w.d, dtype=torch.bfloat16, device="cuda") for l, _ in layers]
    refs = []
    for (lay, _), p in zip(layers, probs):
        r = torch.empty(lay.w.T, lay.w.d, dtype=torch.bfloat16, device="cuda")
        nv.moe_nvfp4_forward(p, lay.x, lay.gate_w, lay.local_weights(lay.w.offset, lay.w.L),
                             lay.shared if lay.w.has_shared else None, nv.alloc_workspace(p), r)
        refs.append(r)
    torch.cuda.synchronize()

    def run_all():
        for (lay, _), p, o in zip(layers, probs, outs):
            nv.moe_nvfp4_forward(p, lay.x, lay.gate_w, lay.local_weights(lay.w.offset, lay.w.L),
                                 lay.shared if lay.w.has_shared else None, ws, o)

    for rep in range(2):                               # twice: the second pass starts from the first's scratch
        for o in outs:
            o.fill_(float("nan"))
        run_all()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"eager pass {rep}, layer {i}"

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        ws.fill_(0x5A if rep % 2 else 0xFF)           # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"graph replay {rep}, layer {i}"
