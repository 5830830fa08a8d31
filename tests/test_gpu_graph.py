"""The forward enqueues only kernels (no allocation, no host synchronisation, no
memset nodes), so a caller can capture it in a HIP graph.  A captured forward is
replayed several times, with the inputs rewritten by eager work between the
replays; every replay must equal the eager forward on the same inputs bit for
bit (the kernels are deterministic)."""
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from tests.gpu_helpers import Layer, log, require_gpu

pytestmark = pytest.mark.gpu

W4A16, W4A4 = workloads.W4A16, workloads.W4A4

MID = workloads.Workload("mid_graph", T=200, d=512, F=256, E=24, k=4, offset=0, L=24, has_shared=True,
                         mode=W4A16, hidden_seed=17, gate_seed=17, weight_seed=17, gate_std=0.05)


def _graph_vs_eager(lay, offset, L, shared, mode, path, n_replays=3):
    w = lay.w
    p = nv.make_problem(w.T, w.d, w.F, w.E, w.k, offset, L, shared, mode, path)
    ws = nv.alloc_workspace(p)
    local = lay.local_weights(offset, L)
    sh = lay.shared if shared else None
    x = lay.x.clone()
    out = torch.empty(w.T, w.d, dtype=torch.bfloat16, device="cuda")
    # eager first (one-time set-up happens outside the capture)
    nv.moe_nvfp4_forward(p, x, lay.gate_w, local, sh, ws, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.moe_nvfp4_forward(p, x, lay.gate_w, local, sh, ws, out)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    for r in range(n_replays):
        gen.manual_seed(1000 + r)
        new_x = torch.randn(w.T, w.d, generator=gen, device="cuda").to(torch.bfloat16)
        if r == 1:
            new_x[min(3, w.T - 1)] = 0                     # a zero token in one replay
        x.copy_(new_x)                                     # eager work between replays
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(out)
        ws2 = nv.alloc_workspace(p)
        nv.moe_nvfp4_forward(p, new_x, lay.gate_w, local, sh, ws2, ref)
        torch.cuda.synchronize()
        assert not torch.isnan(got).any().item(), f"replay {r} left NaNs"
        assert torch.equal(got, ref), f"replay {r} differs from the eager forward"
    return True


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("path", [nv.PATH_DECODE, nv.PATH_PREFILL, nv.PATH_MID])
def test_graph_replays_match_eager_mid(mode, path):
    require_gpu()
    lay = Layer(MID)
    log(f"graph replay mid mode={mode} path={path}")
    _graph_vs_eager(lay, 4, 16, True, mode, path)


@pytest.mark.parametrize("T,path", [(1, nv.PATH_AUTO), (64, nv.PATH_AUTO), (256, nv.PATH_DECODE),
                                    (384, nv.PATH_AUTO)])
def test_graph_replays_match_eager_decode_shard(T, path):
    """T = 1: selection and permutation in one workgroup, GEMM1 in two K slices
    per workgroup; T = 64: exact routing, 4-row weight-streaming tiles; T = 256
    (block-diagonal path forced): certified routing, one-workgroup permutation,
    8-row tiles with more than 64 KB of LDS; T = 384: the dense weight-streaming
    path AUTO picks there."""
    require_gpu()
    w = workloads.replace(workloads.WORKLOADS["decode_shard0_w4a16"], T=T)
    lay = Layer(w, experts_range=(0, w.L))
    log(f"graph replay decode shard T={T} path={path}")
    _graph_vs_eager(lay, w.offset, w.L, True, w.mode, path)
