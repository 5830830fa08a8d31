"""The no-allocation forward (library-owned scratch) against the workspace
forward and the oracle: two calls in a row on one device, the second with a
smaller input (the scratch keeps the first call's contents), and a problem too
large for the scratch rejected before anything is enqueued."""
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from tests.gpu_helpers import Layer, log, rel_err, require_gpu, tol

pytestmark = pytest.mark.gpu

MID = workloads.Workload("noalloc_mid", T=200, d=512, F=256, E=24, k=4, offset=0, L=24, has_shared=True,
                         mode=workloads.W4A16, hidden_seed=41, gate_seed=41, weight_seed=41, gate_std=0.05)


def _both(lay, x, offset, L, shared, mode, path):
    w = lay.w
    p = nv.make_problem(x.shape[0], w.d, w.F, w.E, w.k, offset, L, shared, mode, path)
    ref = torch.empty(x.shape[0], w.d, dtype=torch.bfloat16, device="cuda")
    nv.moe_nvfp4_forward(p, x, lay.gate_w, lay.local_weights(offset, L), lay.shared if shared else None,
                         nv.alloc_workspace(p), ref)
    out = torch.full_like(ref, float("nan"))
    nv.moe_nvfp4_forward_noalloc(p, x, lay.gate_w, lay.local_weights(offset, L), lay.shared if shared else None,
                                 out)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("mode", [workloads.W4A16, workloads.W4A4])
def test_noalloc_matches_workspace_forward_twice_shrinking(mode):
    require_gpu()
    lay = Layer(MID)
    w = lay.w
    # first call: all 200 tokens on the tiled path; second: 37 tokens on weight
    # streaming, a smaller problem over the scratch the first call left behind
    for T, offset, L, shared, path in ((200, 0, 24, True, nv.PATH_PREFILL), (37, 6, 12, False, nv.PATH_DECODE)):
        x = lay.x[:T].contiguous()
        log(f"noalloc mode={mode} T={T} offset={offset} L={L} shared={shared} path={path}")
        out, ref = _both(lay, x, offset, L, shared, mode, path)
        assert torch.equal(out, ref)
        lay_x, lay.x, lay._x64 = lay.x, x, None
        try:
            oref = lay.oracle_full(offset, L, shared, mode)["out"]
        finally:
            lay.x, lay._x64 = lay_x, None
        err = rel_err(out, oref)
        log(f"  bit-identical to the workspace forward; normwise rel err vs oracle {err:.3e}")
        assert err <= tol(mode)


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    require_gpu()
    p = nv.make_problem(8192, 4096, 1024, 320, 8, 0, 320, True, nv.W4A4)
    assert nv.moe_nvfp4_workspace_size(p) > nv.NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(1, dtype=torch.uint8, device="cuda")
    h = torch.empty(1, 1, dtype=torch.bfloat16, device="cuda")
    st = nv.lib().moe_nvfp4_forward_noalloc(nv.ctypes.byref(p), h.data_ptr(), h.data_ptr(), None, None,
                                            dummy.data_ptr(), None)
    assert st == nv.ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in nv.moe_nvfp4_last_error()
