"""Pins of the oracle's router, shard filter, permutation and layer: closed forms,
invariants of the expert-parallel split (partial sums add up), brute-force loops on
tiny inputs, and a special case that reduces to a dense SwiGLU FFN.  CPU only."""
import os

import numpy as np
import pytest

from oracle import brute, moe, nvfp4
from tests.oracle_helpers import tiny_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _model_shape():
    vals = {}
    with open(os.path.join(GOLDEN, "model_shape.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *rest = line.split()
                vals[key] = [int(r) for r in rest]
    return vals


def test_router_weights_sum_to_one_and_equal_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 48))
    G = rng.standard_normal((48, 40)) * 0.3
    r = moe.route(x, G, 8)
    assert np.allclose(r["weights"].sum(1), 1.0, atol=1e-15, rtol=0)
    logits = x @ G
    full = np.exp(logits - logits.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, r["ids"].astype(np.int64), 1)
    assert np.allclose(sel / sel.sum(1, keepdims=True), r["weights"], rtol=1e-13, atol=0)
    # ids are the k largest logits, in descending order
    srt = np.sort(logits, 1)[:, ::-1][:, :8]
    assert np.array_equal(np.take_along_axis(logits, r["ids"].astype(np.int64), 1), srt)


def test_router_ties_go_to_lower_id_and_zero_token():
    x = np.zeros((1, 16))
    G = np.random.default_rng(2).standard_normal((16, 10))
    r = moe.route(x, G, 3)
    assert r["ids"].tolist() == [[0, 1, 2]]
    assert np.allclose(r["weights"], 1 / 3, rtol=0, atol=1e-16)
    assert r["ambiguous"][0]
    # explicit ties among a few experts
    x = np.ones((1, 1))
    G = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    r = moe.route(x, G, 2)
    assert r["ids"].tolist() == [[1, 2]]


def test_zero_token_gives_zero_output():
    w, x, G, experts, shared = tiny_problem()
    x[2] = 0.0
    out = moe.forward(x, G, experts, shared, w.k, 0, w.E, moe.W4A16)["out"]
    assert np.all(out[2] == 0.0)         # silu(0) * 0 = 0 for every expert, shared included
    assert np.any(out[1] != 0.0)


def test_shard_filter_maps_and_drops():
    ids = np.array([[0, 5, 9], [3, 4, 7]], dtype=np.int32)
    lam = moe.shard_filter(ids, 4, 4)
    assert lam.tolist() == [[-1, 1, -1], [-1, 0, 3]]
    shape = _model_shape()
    lo, hi = shape["shard1"]
    ids = np.arange(shape["routed_experts"][0]).reshape(1, -1)
    lam = moe.shard_filter(ids, lo, hi - lo + 1)
    assert (lam[0, :lo] == -1).all() and lam[0, lo:].tolist() == list(range(hi - lo + 1))


def test_permutation_against_brute_force_sort():
    rng = np.random.default_rng(3)
    T, k, L = 37, 4, 9
    lam = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        chosen = rng.choice(L + 5, size=k, replace=False) - 5      # some dropped (negative)
        lam[t] = np.where(chosen >= 0, chosen, -1)
    pm = moe.permutation(lam, L)
    pairs = sorted((int(lam[t, j]), t, t * k + j) for t in range(T) for j in range(k) if lam[t, j] >= 0)
    assert pm["perm"].tolist() == [p for _, _, p in pairs]
    for l in range(L):
        assert pm["counts"][l] == sum(1 for e, _, _ in pairs if e == l)
    assert pm["offsets"][0] == 0 and pm["offsets"][-1] == len(pairs)
    assert np.array_equal(np.diff(pm["offsets"]), pm["counts"])


@pytest.mark.parametrize("w4a4", [False, True])
@pytest.mark.parametrize("offset,L,with_shared", [(0, 8, True), (2, 3, False), (5, 3, True)])
def test_layer_matches_brute_force_loops(w4a4, offset, L, with_shared):
    w, x, G, experts, shared = tiny_problem(seed=7)
    mode = moe.W4A4 if w4a4 else moe.W4A16
    sh = shared if with_shared else None
    got = moe.forward(x, G, experts[offset:offset + L], sh, w.k, offset, L, mode)["out"]
    ref = np.array(brute.layer(x.tolist(), G.tolist(), experts[offset:offset + L], sh, w.k,
                               offset, L, w4a4=w4a4))
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("mode", [moe.W4A16, moe.W4A4])
def test_half_shard_partial_sums_add_up(mode):
    w, x, G, experts, shared = tiny_problem(T=24, d=64, F=32, E=8, k=3, seed=11)
    E = w.E
    full = moe.forward(x, G, experts, shared, w.k, 0, E, mode)["out"]
    a = moe.forward(x, G, experts[:E // 2], shared, w.k, 0, E // 2, mode)["out"]
    b = moe.forward(x, G, experts[E // 2:], None, w.k, E // 2, E // 2, mode)["out"]
    assert np.max(np.abs(a + b - full)) <= 1e-12 * np.max(np.abs(full))
    assert np.max(np.abs(a - full)) > 1e-3 * np.max(np.abs(full))      # the halves really differ


def test_out_of_shard_experts_are_never_touched():
    """Routing is global, but only experts inside [offset, offset + L) are ever
    evaluated; their ids arrive shard-relative."""
    w, x, G, experts, shared = tiny_problem(T=16, seed=13)
    o, L = 3, 4
    asked = []

    def get(l):
        assert 0 <= l < L
        asked.append(l)
        return experts[o + l]

    res = moe.forward(x, G, get, shared, w.k, o, L, moe.W4A16)
    glob = res["ids"]
    in_shard = sorted(set(int(e) - o for e in glob.reshape(-1) if o <= e < o + L))
    assert sorted(asked) == in_shard
    assert (res["local_ids"] == np.where((glob >= o) & (glob < o + L), glob - o, -1)).all()


def test_single_expert_top1_is_a_dense_swiglu_ffn():
    w, x, G, experts, _ = tiny_problem(E=1, k=1, seed=17)
    got = moe.forward(x, G, experts, None, 1, 0, 1, moe.W4A16)["out"]
    W13 = nvfp4.dequantize(experts[0]["w13"], experts[0]["w13_scale"], experts[0]["g13"])
    W2 = nvfp4.dequantize(experts[0]["w2"], experts[0]["w2_scale"], experts[0]["g2"])
    F = W13.shape[0] // 2
    hg = x @ W13[:F].T
    hu = x @ W13[F:].T
    ffn = (hg * (1 / (1 + np.exp(-hg))) * hu) @ W2.T
    assert np.allclose(got, ffn, rtol=1e-12, atol=1e-12)
    # single expert, top-1: routing weight is exactly 1
    assert np.all(moe.route(x, G, 1)["weights"] == 1.0)


def test_gate_and_up_halves_are_not_interchangeable():
    """The convention is rows [0,F) = gate, [F,2F) = up: zeroing the gate half's
    codes gives silu(0) = 0 and a zero output; a swapped convention would still
    give zero (up = 0); making the gate half very negative must also give ~0,
    while making the up half very negative must not."""
    w, x, G, experts, _ = tiny_problem(E=1, k=1, seed=19)
    q = dict(experts[0])
    F = w.F
    W13 = nvfp4.dequantize(q["w13"], q["w13_scale"], q["g13"])
    big = np.abs(W13).max()
    for half, expect_zero in ((0, True), (1, False)):
        M = W13.copy()
        rows = slice(0, F) if half == 0 else slice(F, 2 * F)
        M[rows] = -big * np.sign(x.sum(0))[None, :] * 16      # strongly negative pre-activations
        qq = nvfp4.quantize_weight(M.astype(np.float32))
        e = dict(q, w13=qq["codes"], w13_scale=qq["scales"], g13=qq["g"])
        out = moe.forward(x, G, [e], None, 1, 0, 1, moe.W4A16)["out"]
        if expect_zero:
            assert np.max(np.abs(out)) < 1e-6
        else:
            assert np.max(np.abs(out)) > 1e-2


def test_ambiguity_flag():
    x = np.array([[1.0]])
    G = np.array([[2.0, 1.0, 1.0 + 1e-12, 0.0]])
    r = moe.route(x, G, 2)
    assert r["ambiguous"][0]
    G = np.array([[2.0, 1.0, 0.5, 0.0]])
    assert not moe.route(x, G, 2)["ambiguous"][0]


@pytest.mark.parametrize("mode", [moe.W4A16, moe.W4A4, moe.W4A4_STATIC])
@pytest.mark.parametrize("offset,L,with_shared", [(0, 8, True), (3, 4, False), (6, 2, True)])
def test_forward_on_a_process_pool_is_bit_identical(mode, offset, L, with_shared):
    """The expert terms evaluated by a process pool (as the full-size parity
    tests do) sum to exactly the serial result, and both equal the brute-force
    loops (W4A16 / dynamic W4A4)."""
    from tests import oracle_pool
    w, x, G, experts, shared = tiny_problem(T=12, d=64, F=32, E=8, k=3, seed=23)
    sh = shared if with_shared else None
    ag = (0.0021, 0.0043) if mode == moe.W4A4_STATIC else (1.0, 1.0)
    serial = moe.forward(x, G, experts[offset:offset + L], sh, w.k, offset, L, mode, act_global=ag)["out"]
    pooled = oracle_pool.forward(x, G, experts[offset:offset + L], sh, w.k, offset, L, mode,
                                 act_global=ag)["out"]
    listed = moe.forward(x, G, experts[offset:offset + L], sh, w.k, offset, L, mode, act_global=ag,
                         map_fn=lambda f, it: list(map(f, it)))["out"]
    assert np.array_equal(serial, pooled)
    assert np.array_equal(serial, listed)
    if mode != moe.W4A4_STATIC:
        ref = np.array(brute.layer(x.tolist(), G.tolist(), experts[offset:offset + L], sh, w.k,
                                   offset, L, w4a4=mode == moe.W4A4))
        assert np.max(np.abs(pooled - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_pool_quantizer_matches_the_oracle_helper():
    """The pool's quantizer of bf16 bit patterns equals the oracle's quantizer of
    the same values (the tests' host-side path)."""
    import torch
    from tests import oracle_pool
    from tests.oracle_helpers import quantize_expert_oracle
    g = torch.Generator().manual_seed(5)
    w13 = (torch.randn(64, 96, generator=g) / 10).to(torch.bfloat16)
    w2 = (torch.randn(96, 32, generator=g) / 6).to(torch.bfloat16)
    a = quantize_expert_oracle(w13, w2)
    b = list(oracle_pool.pool_map(oracle_pool.quantize_expert_bits,
                                  [(w13.view(torch.int16).numpy().view(np.uint16),
                                    w2.view(torch.int16).numpy().view(np.uint16))]))[0]
    for key in a:
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key
