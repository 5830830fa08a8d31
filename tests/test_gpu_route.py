"""GPU parity of routing and permutation against the oracle on all five
workloads at their full token counts: expert ids, counts, offsets and the
permutation bit-exact; routing weights within 1e-6 relative.  Tokens whose k-th
and (k+1)-th fp64 logits are closer than the oracle's ambiguity threshold may
pick either expert; the permutation is then checked against the GPU's own
choice."""
import numpy as np
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from oracle import moe
from tests.gpu_helpers import log, require_gpu
from tests.oracle_helpers import to_f64

pytestmark = pytest.mark.gpu


def _route_gpu(x, gate_w, w, offset, L, has_shared):
    T = x.shape[0]
    p = nv.make_problem(T, w.d, w.F, w.E, w.k, offset, L, has_shared, w.mode)
    ws = nv.alloc_workspace(p)
    ids = torch.full((T, w.k), -7, dtype=torch.int32, device="cuda")
    wts = torch.full((T, w.k), -7.0, dtype=torch.float32, device="cuda")
    counts = torch.full((L,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((L + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * w.k,), -7, dtype=torch.int32, device="cuda")
    nv.moe_nvfp4_route(p, x, gate_w, ws, ids, wts, counts, offsets, perm)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), wts.cpu().numpy(), counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy()


def _check(x, G, w, offset, L, has_shared=True):
    gate_w = G.t().contiguous()
    ids, wts, counts, offsets, perm = _route_gpu(x, gate_w, w, offset, L, has_shared)
    r = moe.route(to_f64(x), to_f64(G), w.k)
    amb = r["ambiguous"]
    diff = np.any(ids != r["ids"], axis=1)
    assert not np.any(diff & ~amb), f"unambiguous tokens differ: {np.nonzero(diff & ~amb)[0][:10]}"
    ok = ~diff
    rel = np.abs(wts[ok] - r["weights"][ok]) / np.abs(r["weights"][ok])
    assert rel.max() <= 1e-6, rel.max()
    assert np.allclose(wts.sum(1), 1.0, atol=1e-6)
    # permutation derived from the GPU's own (verified) ids
    pm = moe.permutation(moe.shard_filter(ids, offset, L), L)
    P = int(pm["offsets"][-1])
    assert np.array_equal(counts, pm["counts"])
    assert np.array_equal(offsets, pm["offsets"])
    assert np.array_equal(perm[:P], pm["perm"])
    return int(amb.sum()), int(diff.sum()), P


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_route_parity_full_size(name):
    require_gpu()
    w = workloads.WORKLOADS[name]
    log(f"route parity {name}: T={w.T} E={w.E} k={w.k} offset={w.offset} L={w.L}")
    x = workloads.gen_hidden(w, "cuda")
    G = workloads.gen_gate(w, "cuda")
    amb, diff, P = _check(x, G, w, w.offset, w.L, w.has_shared)
    log(f"  ambiguous tokens {amb}, differing {diff}, local pairs P={P}")


def test_route_zero_tokens_tie_to_lowest_ids():
    require_gpu()
    w = workloads.replace(workloads.WORKLOADS["decode_shard0_w4a16"], T=8)
    x = workloads.gen_hidden(w, "cuda")
    x[2] = 0
    x[5] = 0
    G = workloads.gen_gate(w, "cuda")
    ids, wts, *_ = _route_gpu(x, G.t().contiguous(), w, 0, w.E, True)
    for t in (2, 5):
        assert ids[t].tolist() == list(range(w.k))
        assert np.allclose(wts[t], 1.0 / w.k, rtol=0, atol=1e-7)
    _check(x, G, w, 0, w.E)


@pytest.mark.parametrize("T", [600, 1100])
def test_route_wide_select_zero_tokens_and_shard(T):
    """From 512 tokens the selection runs a wave per token (from 1024) or four
    waves per token, each re-scoring a quarter of K (below): zero tokens (every
    expert a candidate) and a shard filter, against the oracle."""
    require_gpu()
    w = workloads.replace(workloads.WORKLOADS["decode_shard0_w4a16"], T=T)
    x = workloads.gen_hidden(w, "cuda")
    zeros = (0, 63, 64, T - 1)
    for t in zeros:
        x[t] = 0
    G = workloads.gen_gate(w, "cuda")
    ids, wts, *_ = _route_gpu(x, G.t().contiguous(), w, 0, w.E, True)
    for t in zeros:
        assert ids[t].tolist() == list(range(w.k))
        assert np.allclose(wts[t], 1.0 / w.k, rtol=0, atol=1e-7)
    amb, diff, P = _check(x, G, w, 100, 150)
    log(f"  wide select: ambiguous {amb}, differing {diff}, P={P}")


@pytest.mark.parametrize("T,E", [(4096, 200), (4100, 136), (4160, 320)])
def test_route_wide_logits_ragged(T, E):
    """From 4096 tokens and for 129..320 experts the certified logits run on
    workgroups of 64 tokens x all experts, in K slices: expert counts that
    leave part of the staged rows and of the last wave's columns empty, a
    token count that leaves the last workgroup partly empty, and zero tokens,
    against the oracle (ids bit-exact, weights, permutation)."""
    require_gpu()
    w = workloads.replace(workloads.WORKLOADS["decode_shard0_w4a16"], T=T, E=E, L=E // 2, offset=E // 4)
    log(f"wide logits T={T} E={E}")
    x = workloads.gen_hidden(w, "cuda")
    x[T - 1] = 0
    G = workloads.gen_gate(w, "cuda")
    amb, diff, P = _check(x, G, w, w.offset, w.L)
    log(f"  ambiguous {amb}, differing {diff}, P={P}")
    assert P > 0


def test_route_tiny_problem_odd_shapes():
    """T not a multiple of any tile, E not a multiple of 64, k = 1 and k = E."""
    require_gpu()
    base = workloads.WORKLOADS["tiny_w4a16"]
    for T, E, k, off, L in [(1, 16, 1, 0, 16), (37, 40, 3, 5, 30), (300, 72, 7, 40, 32), (5, 6, 6, 0, 6)]:
        w = workloads.replace(base, T=T, E=E, k=k, offset=off, L=L, gate_std=0.3)
        log(f"route odd shape T={T} E={E} k={k} offset={off} L={L}")
        x = workloads.gen_hidden(w, "cuda")
        G = workloads.gen_gate(w, "cuda")
        _check(x, G, w, off, L)


def test_route_empty_batch():
    require_gpu()
    w = workloads.WORKLOADS["tiny_w4a16"]
    p = nv.make_problem(0, w.d, w.F, w.E, w.k, 0, w.L, True, w.mode)
    ws = nv.alloc_workspace(p)
    counts = torch.full((w.L,), 5, dtype=torch.int32, device="cuda")
    offsets = torch.full((w.L + 1,), 5, dtype=torch.int32, device="cuda")
    x = torch.empty(0, w.d, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(w.E, w.d, dtype=torch.bfloat16, device="cuda")
    nv.moe_nvfp4_route(p, x if x.numel() else g, g, ws, None, None, counts, offsets, None)
    torch.cuda.synchronize()
    assert not counts.any().item() and not offsets.any().item()


@pytest.mark.parametrize("T", [1, 2, 3, 7, 16, 17, 33, 64, 65, 128, 129])
def test_route_few_tokens_both_sides_of_the_exact_fp64_path(T):
    """Up to 128 tokens the logits are computed exactly in fp64 on the matrix
    cores (no bounds, no re-scoring; token tiles of 16, 32 and 64 rows, full and
    ragged); up to 2 tokens (640 token-expert logits) the selection and the
    permutation then run in one workgroup, from 3 in a workgroup per token and a
    permutation launch; 129 tokens take the certified bf16-MFMA path."""
    require_gpu()
    w = workloads.replace(workloads.WORKLOADS["decode_shard0_w4a16"], T=T)
    log(f"route few tokens T={T}")
    x = workloads.gen_hidden(w, "cuda")
    if T >= 2:
        x[1] = 0                                           # a zero token: ids 0..k-1, equal weights
    G = workloads.gen_gate(w, "cuda")
    amb, diff, P = _check(x, G, w, w.offset, w.L, w.has_shared)
    if T >= 2:
        ids, wts, *_ = _route_gpu(x, G.t().contiguous(), w, w.offset, w.L, w.has_shared)
        assert ids[1].tolist() == list(range(w.k))
        assert np.allclose(wts[1], 1.0 / w.k, rtol=0, atol=1e-7)


@pytest.mark.parametrize("T,L", [(256, 160), (512, 160), (1024, 160), (1025, 160), (288, 1024), (289, 1024)])
def test_route_permutation_one_workgroup_and_blocked(T, L):
    """Up to 1024 tokens (a bitmask of L x ceil(T/32) words and its 16-bit
    prefix within 56 KB) one workgroup builds the whole permutation; beyond,
    per-256-token blocks, a scan and a scatter.  Both sides of each bound
    (the token bound at L = 160, the LDS bound at L = 1024), against the
    oracle."""
    require_gpu()
    E = max(320, L)
    w = workloads.replace(workloads.WORKLOADS["decode_shard0_w4a16"], T=T, E=E, L=L, offset=0)
    log(f"route permutation T={T} E={E} L={L}")
    x = workloads.gen_hidden(w, "cuda")
    G = workloads.gen_gate(w, "cuda")
    amb, diff, P = _check(x, G, w, 0, L, True)
    log(f"  ambiguous {amb}, differing {diff}, local pairs P={P}")
    assert P > 0
