"""The library's stated limits, on the GPU against the oracle:
  * d = 16384 (the largest model width) with F = 128, and F = 16384 with
    d = 128: the weight-streaming kernels then stage the token rows in
    chunks (the whole K no longer fits in LDS), and the tiled kernels run 256
    K steps and the widest column grids;
  * E = 1024 experts with top-32 (the largest routing), through the exact
    (few-token) and both certified selection kernels, at d = 256 and at the
    widest model d = 16384, and a full layer over all 1024 local experts (every
    permutation counter at its widest).
Full outputs within 1e-2 (W4A16) / 3e-2 (W4A4); routing ids, counts, offsets
and permutation bit-exact."""
import pytest

import nvfp4_expert_layer_amd as nv
import workloads
from tests.gpu_helpers import Layer, log, rel_err, require_gpu, tol
from tests.test_gpu_route import _check

pytestmark = pytest.mark.gpu

W4A16, W4A4 = workloads.W4A16, workloads.W4A4

WIDE_D = workloads.Workload("max_d", T=40, d=16384, F=128, E=6, k=2, offset=0, L=6, has_shared=True,
                            mode=W4A16, hidden_seed=61, gate_seed=61, weight_seed=61, gate_std=0.01)
WIDE_F = workloads.Workload("max_f", T=40, d=128, F=16384, E=6, k=2, offset=1, L=4, has_shared=True,
                            mode=W4A16, hidden_seed=62, gate_seed=62, weight_seed=62, gate_std=0.1)
MANY_E = workloads.Workload("max_e", T=24, d=128, F=128, E=1024, k=32, offset=0, L=1024, has_shared=True,
                            mode=W4A16, hidden_seed=63, gate_seed=63, weight_seed=63, gate_std=0.2)

_layers = {}


def get(w):
    if w.name not in _layers:
        _layers[w.name] = Layer(w)
    return _layers[w.name]


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("path", [nv.PATH_DECODE, nv.PATH_PREFILL, nv.PATH_MID])
@pytest.mark.parametrize("wl", [WIDE_D, WIDE_F], ids=["d16384", "F16384"])
def test_widest_layers(wl, path, mode):
    if path == nv.PATH_MID and wl.d % 256:
        pytest.skip("the dense weight-streaming path needs d % 256 == 0")
    require_gpu()
    lay = get(wl)
    w = lay.w
    log(f"{w.name}: d={w.d} F={w.F} mode={mode} path={path}")
    out = lay.run(w.offset, w.L, w.has_shared, mode, path)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, mode)["out"]
    err = rel_err(out, ref)
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


@pytest.mark.parametrize("T", [2, 3, 16, 40, 600, 1100])
def test_route_1024_experts_top32(T):
    """E = 1024, top-32: a workgroup per token for the selection (T = 2, 3, 16,
    40), four waves per token (T = 600), a wave per token (T = 1100)."""
    require_gpu()
    w = workloads.replace(MANY_E, T=T, d=256)
    log(f"route E=1024 k=32 T={T}")
    x = workloads.gen_hidden(w, "cuda")
    G = workloads.gen_gate(w, "cuda")
    amb, diff, P = _check(x, G, w, 100, 900, True)
    log(f"  ambiguous {amb}, differing {diff}, local pairs {P}")
    assert P > 0


@pytest.mark.parametrize("T", [24, 40])
def test_route_1024_experts_widest_model(T):
    """E = 1024, top-32, d = 16384: 24 tokens take the exact fp64 logits with
    five ragged K slices (T E d <= 2^29), 40 tokens the certified path."""
    require_gpu()
    w = workloads.replace(MANY_E, T=T, d=16384, gate_std=0.02)
    log(f"route E=1024 k=32 d=16384 T={T}")
    x = workloads.gen_hidden(w, "cuda")
    G = workloads.gen_gate(w, "cuda")
    amb, diff, P = _check(x, G, w, 0, 1024, True)
    log(f"  ambiguous {amb}, differing {diff}, local pairs {P}")
    assert P == T * 32


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("T,d", [(10, 16384), (30, 8192), (30, 4096)], ids=["4row-chunked", "8row-chunked", "8row-whole"])
def test_decode_token_stage_variants(T, d, mode):
    """Weight streaming whose token stage does not fit in LDS whole: 4-row tiles
    at K = 16384 and 8-row tiles at K = 8192 stage 512-element chunks; 8-row
    tiles at K = 4096 stage the whole K (65.7 KB of LDS).  Full output."""
    require_gpu()
    lay = get(workloads.replace(WIDE_D, name=f"stage_{T}_{d}", T=T, d=d))
    w = lay.w
    log(f"decode token stage T={T} d={d} mode={mode}")
    out = lay.run(w.offset, w.L, w.has_shared, mode, nv.PATH_DECODE)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, mode)["out"]
    err = rel_err(out, ref)
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


@pytest.mark.parametrize("path", [nv.PATH_DECODE, nv.PATH_PREFILL])
def test_layer_1024_local_experts_top32(path):
    require_gpu()
    lay = get(MANY_E)
    w = lay.w
    log(f"E=1024 k=32 full layer, path={path}")
    out = lay.run(w.offset, w.L, w.has_shared, W4A16, path)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, W4A16)["out"]
    err = rel_err(out, ref)
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(W4A16)
