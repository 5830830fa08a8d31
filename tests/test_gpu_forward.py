"""GPU parity of the fused layer against the oracle: normwise relative error
<= 1e-2 (W4A16) / 3e-2 (W4A4) over the whole [T, d] output, on problems the
oracle finishes in seconds (several tiles, ragged tails, every kernel path) and
at the full workload sizes in the launch configuration the benchmark times (the
oracle's expert terms then run on a CPU process pool).  Also the
expert-parallel partial-sum contract, determinism, poisoned workspaces and
degenerate cases."""
import numpy as np
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from oracle import moe
from tests.gpu_helpers import Layer, log, rel_err, require_gpu, tol
from tests.oracle_helpers import to_f64

pytestmark = pytest.mark.gpu

W4A16, W4A4 = workloads.W4A16, workloads.W4A4
PATHS = [nv.PATH_DECODE, nv.PATH_PREFILL, nv.PATH_MID]

_layers = {}


def layer(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _layers:
        w = workloads.WORKLOADS[name] if name in workloads.WORKLOADS else LOCAL[name]
        if kw:
            w = workloads.replace(w, **kw)
        _layers[key] = Layer(w)
    return _layers[key]


# A mid-size layer: several M and N tiles, ragged token count, E not a power of 2.
MID = workloads.Workload("mid", T=200, d=512, F=256, E=24, k=4, offset=0, L=24, has_shared=True,
                         mode=W4A16, hidden_seed=7, gate_seed=7, weight_seed=7, gate_std=0.05)
# Odd widths and heavy experts: d % 256 == 128 (a half-filled column block in the
# down projection's 256-wide tiles), ~240 pairs per expert plus 600 shared rows
# (experts spanning several 256-row tiles, ragged last tiles).
WIDE = workloads.Workload("wide", T=600, d=384, F=384, E=5, k=2, offset=0, L=5, has_shared=True,
                          mode=W4A16, hidden_seed=9, gate_seed=9, weight_seed=9, gate_std=0.05)
LOCAL = {"mid": MID, "wide": WIDE}


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("path", PATHS)
def test_tiny_workload_full_output(mode, path):
    require_gpu()
    lay = layer("tiny_w4a16")
    w = lay.w
    log(f"tiny full output mode={mode} path={path}")
    out = lay.run(w.offset, w.L, w.has_shared, mode, path)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, mode)
    err = rel_err(out, ref["out"])
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("path", PATHS + [nv.PATH_AUTO])
@pytest.mark.parametrize("offset,L,shared", [(0, 24, True), (8, 12, True), (12, 12, False), (23, 1, False)])
def test_mid_layer_full_output(mode, path, offset, L, shared):
    require_gpu()
    lay = layer("mid")
    log(f"mid full output mode={mode} path={path} offset={offset} L={L} shared={shared}")
    out = lay.run(offset, L, shared, mode, path)
    ref = lay.oracle_full(offset, L, shared, mode)
    err = rel_err(out, ref["out"])
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("path", [nv.PATH_DECODE, nv.PATH_PREFILL])
@pytest.mark.parametrize("offset,L,shared", [(0, 5, True), (1, 3, False)])
def test_wide_layer_full_output(mode, path, offset, L, shared):
    require_gpu()
    lay = layer("wide")
    log(f"wide full output mode={mode} path={path} offset={offset} L={L} shared={shared}")
    out = lay.run(offset, L, shared, mode, path)
    ref = lay.oracle_full(offset, L, shared, mode)
    err = rel_err(out, ref["out"])
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


@pytest.mark.parametrize("mode", [W4A16, W4A4])
def test_mid_half_shards_sum_to_unsharded(mode):
    require_gpu()
    lay = layer("mid")
    E = lay.w.E
    a = lay.run(0, E // 2, True, mode).float()
    b = lay.run(E // 2, E // 2, False, mode).float()
    full = lay.run(0, E, True, mode).float()
    ref = lay.oracle_full(0, E, True, mode)["out"]
    err = moe.normwise_rel_err((a + b).cpu().double().numpy(), ref)
    log(f"half-shard sum vs unsharded oracle: {err:.3e}")
    assert err <= tol(mode)
    # GPU shards against the GPU unsharded output (bf16 rounding of each term only)
    gerr = moe.normwise_rel_err((a + b).cpu().double().numpy(), full.cpu().double().numpy())
    assert gerr <= 1e-2


def test_deterministic_and_poison_proof():
    require_gpu()
    lay = layer("mid")
    w = lay.w
    p = nv.make_problem(w.T, w.d, w.F, w.E, w.k, 4, 16, True, W4A4)
    ws = nv.alloc_workspace(p)
    o1 = lay.run(4, 16, True, W4A4, ws=ws, ws_fill=0)
    o2 = lay.run(4, 16, True, W4A4, ws=ws, ws_fill=0xFF,
                 out=torch.full((w.T, w.d), float("nan"), dtype=torch.bfloat16, device="cuda"))
    assert not torch.isnan(o2).any().item()
    assert torch.equal(o1, o2)
    for path in PATHS:
        a = lay.run(0, w.E, True, W4A16, path)
        b = lay.run(0, w.E, True, W4A16, path, ws_fill=0xFF)
        assert torch.equal(a, b)


def test_single_token_and_all_pairs_dropped():
    require_gpu()
    lay = layer("mid")
    w = lay.w
    # T = 1
    x1 = lay.x[:1].contiguous()
    out = lay.run(0, w.E, True, W4A16, x=x1)
    r = moe.forward(lay.x64[:1], lay.G64, lambda l: lay.oracle_expert(l), lay.oracle_expert(w.E),
                    w.k, 0, w.E, W4A16)
    assert rel_err(out, r["out"]) <= 1e-2
    # every token routes to experts 0..k-1 (large logits through a constant channel);
    # the shard [E/2, E) then keeps no pair: the output is the shared expert alone, or 0.
    x = lay.x.clone()
    x[:, 0] = 4.0
    G = lay.G.clone()
    G[0, :] = 0
    G[0, :w.k] = 8.0
    lay2_gate = G.t().contiguous()
    saved = lay.gate_w
    try:
        lay.gate_w = lay2_gate
        out_s = lay.run(w.E // 2, w.E // 2, True, W4A16, x=x)
        out_n = lay.run(w.E // 2, w.E // 2, False, W4A16, x=x)
    finally:
        lay.gate_w = saved
    assert not out_n.any().item()
    shared_only = moe.expert_mlp(to_f64(x), *moe.dequant_expert(lay.oracle_expert(w.E)), W4A16)
    assert rel_err(out_s, shared_only) <= 1e-2


# ----------------------------------------------------------------------------
# full workload sizes: the whole output against the oracle
# ----------------------------------------------------------------------------
_full = {}


def full_layer(name):
    """The 320-expert weight set shared by the full-size workloads (one GPU copy,
    one cache of oracle-quantized experts)."""
    w = workloads.WORKLOADS[name]
    if "weights" not in _full:
        log("building the 320-expert NVFP4 weight set on the GPU")
        _full["weights"] = Layer(workloads.WORKLOADS["decode_shard0_w4a16"])
    base = _full["weights"]
    lay = Layer.__new__(Layer)
    lay.__dict__.update(base.__dict__)
    lay.w = w
    lay.x = workloads.gen_hidden(w, "cuda")
    lay.G = workloads.gen_gate(w, "cuda")
    lay.gate_w = lay.G.t().contiguous()
    lay._x64 = None
    lay._G64 = None
    return lay


def whole_output_check(lay, offset, L, has_shared, mode, what, path=nv.PATH_AUTO):
    """GPU forward against the oracle's whole output; logs the error, the
    routing ambiguity count and the worst token row's error."""
    w = lay.w
    out = lay.run(offset, L, has_shared, mode, path)
    assert not torch.isnan(out).any().item()
    ref = lay.oracle_full(offset, L, has_shared, mode)
    err = rel_err(out, ref["out"])
    y = out.double().cpu().numpy()
    row = np.linalg.norm(y - ref["out"], axis=1) / np.maximum(np.linalg.norm(ref["out"], axis=1), 1e-300)
    log(f"  {what}: T={w.T} offset={offset} L={L} shared={has_shared} mode={mode}: whole-output normwise "
        f"rel err {err:.3e} (limit {tol(mode):g}); worst row {row.max():.3e}; "
        f"ambiguous tokens {int(ref['ambiguous'].sum())}; local pairs {int(ref['offsets'][-1])}")
    assert err <= tol(mode)
    return out, ref


FULL = ["decode_shard0_w4a16", "shard1_w4a4_t512", "shard1_w4a4_static_t512", "prefill_all_w4a4",
        "prefill_zipf_shard0_w4a16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_output(name):
    """Each full-size workload through the path and launch configuration the
    benchmark times, the whole [T, d] output against the oracle."""
    require_gpu()
    lay = full_layer(name)
    w = lay.w
    log(f"full-size {name}")
    whole_output_check(lay, w.offset, w.L, w.has_shared, w.mode, name)


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("T", [12, 30, 31, 36, 37, 72, 73])
def test_decode_tile_heights(T, mode):
    """Weight streaming takes 4-row tiles up to T k = 6E pairs, 8-row tiles up
    to 12E, 16-row tiles beyond; above 5E pairs the down projection merges two
    4-row tiles of one expert: both sides of each bound, full output."""
    require_gpu()
    lay = layer("mid", T=T)
    w = lay.w
    log(f"decode tile heights T={T} (T k / E = {T * w.k / w.E:.2f}) mode={mode}")
    out = lay.run(w.offset, w.L, w.has_shared, mode, nv.PATH_DECODE)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, mode)
    err = rel_err(out, ref["out"])
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


@pytest.mark.parametrize("T", [32, 128, 240, 360])
def test_full_size_decode_other_token_counts(T):  # forced onto the block-diagonal path
    """The 320-expert shard on block-diagonal weight streaming at T = 32 (two row groups per
    wave in GEMM1), 128 (4-row tiles at 4 pairs per expert), 240 (6 pairs per
    expert: the down projection merges two 4-row tiles) and 360 (8-row tiles,
    whose whole-K token stage of 65.7 KB takes more than 64 KB of LDS); the
    whole output against the oracle."""
    require_gpu()
    base = workloads.WORKLOADS["decode_shard0_w4a16"]
    lay = full_layer("decode_shard0_w4a16")
    w = workloads.replace(base, T=T, hidden_seed=base.hidden_seed + T)
    lay.w = w
    lay.x = workloads.gen_hidden(w, "cuda")
    log(f"full-size decode T={T}")
    whole_output_check(lay, w.offset, w.L, w.has_shared, w.mode, f"decode T={T}", nv.PATH_DECODE)


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
def test_full_size_decode_small_batches(T, mode):
    """The 320-expert shard at 1-16 tokens, where few experts are touched (at
    T = 1 GEMM1's workgroups split d = 4096 into two K slices of 2048 between
    two groups of four waves).  Whole output against the oracle, on a workspace
    poisoned with 0xFF bytes, and bit-identical on a second call."""
    require_gpu()
    base = workloads.WORKLOADS["decode_shard0_w4a16"]
    lay = full_layer("decode_shard0_w4a16")
    w = workloads.replace(base, T=T, mode=mode, hidden_seed=base.hidden_seed + 1000 + T)
    lay.w = w
    lay.x = workloads.gen_hidden(w, "cuda")
    log(f"full-size decode small batch T={T} mode={mode}")
    p = nv.make_problem(T, w.d, w.F, w.E, w.k, w.offset, w.L, w.has_shared, mode)
    assert nv.moe_nvfp4_resolved_path(p) == nv.PATH_DECODE
    ws = nv.alloc_workspace(p)
    ws.fill_(0xFF)
    out = lay.run(w.offset, w.L, w.has_shared, mode, ws=ws)
    again = lay.run(w.offset, w.L, w.has_shared, mode, ws=ws)
    assert torch.equal(out, again)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, mode)
    err = rel_err(out, ref["out"])
    log(f"  whole-output normwise rel err {err:.3e} (limit {tol(mode):g})")
    assert err <= tol(mode)


def test_full_size_two_shards_sum_to_unsharded_oracle():
    """Shard 0 (experts 0-159, with the shared expert) plus shard 1 (160-319) at
    the second shard's token count, W4A4: each shard's whole output against the
    oracle's shard, and their sum against the unsharded oracle."""
    require_gpu()
    lay = full_layer("shard1_w4a4_t512")
    a, ra = whole_output_check(lay, 0, 160, True, W4A4, "shard 0")
    b, rb = whole_output_check(lay, 160, 160, False, W4A4, "shard 1")
    full = lay.oracle_full(0, 320, True, W4A4)["out"]
    # the oracle's own shards add up to its unsharded output (fp64 rounding only)
    assert np.max(np.abs(ra["out"] + rb["out"] - full)) <= 1e-10 * np.max(np.abs(full))
    s = a.double() + b.double()
    err = moe.normwise_rel_err(s.cpu().numpy(), full)
    log(f"two shards vs unsharded oracle, whole output: {err:.3e}")
    assert err <= tol(W4A4)


@pytest.mark.parametrize("mode", [W4A16, W4A4])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 100, 200])
def test_mid_path_tile_edges(T, mode):
    """The dense weight-streaming path: on 16-row tiles (up to 12 expected pairs
    per expert) one token, one short of a tile, exactly a tile and one past it
    (an expert with two tiles); on 32-row tiles about half a tile per expert and
    more than a tile per expert; whole output."""
    require_gpu()
    lay = layer("mid", T=T)
    w = lay.w
    log(f"mid path T={T} mode={mode}")
    out = lay.run(w.offset, w.L, w.has_shared, mode, nv.PATH_MID)
    ref = lay.oracle_full(w.offset, w.L, w.has_shared, mode)
    err = rel_err(out, ref["out"])
    log(f"  normwise rel err {err:.3e}")
    assert err <= tol(mode)


@pytest.mark.parametrize("name", ["shard1_w4a4_t512", "decode_shard0_w4a16"])
def test_full_size_mid_path(name):
    """The full-size shards through the dense weight-streaming path (whatever
    AUTO picks for them), whole output against the oracle."""
    require_gpu()
    lay = full_layer(name)
    w = lay.w
    log(f"full-size {name} on the mid path")
    whole_output_check(lay, w.offset, w.L, w.has_shared, w.mode, f"{name} mid path", nv.PATH_MID)


@pytest.mark.parametrize("T", [384, 880])
def test_full_size_mid_path_auto(T):
    """The 320-expert W4A16 shard where AUTO picks the dense weight-streaming
    path (9.6 and 22 pairs per expert), whole output."""
    require_gpu()
    base = workloads.WORKLOADS["decode_shard0_w4a16"]
    lay = full_layer("decode_shard0_w4a16")
    w = workloads.replace(base, T=T, hidden_seed=base.hidden_seed + T)
    lay.w = w
    lay.x = workloads.gen_hidden(w, "cuda")
    p = nv.make_problem(w.T, w.d, w.F, w.E, w.k, w.offset, w.L, w.has_shared, w.mode)
    assert nv.moe_nvfp4_resolved_path(p) == nv.PATH_MID
    log(f"full-size mid (AUTO) T={T}")
    whole_output_check(lay, w.offset, w.L, w.has_shared, w.mode, f"mid T={T}")
