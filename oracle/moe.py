"""Router, shard filter, permutation and the fused MoE layer, in fp64 numpy.

Test infrastructure only (see the package docstring).  Source of each step:

  * routing: the page "Serving Solar Open 2 on DGX Spark" (backend.ai),
    section "Solar Open 2 개요", states 320 routed experts, one shared expert and
    top-8 routing.  The scoring rule it leaves open is read as: logits =
    hidden @ gate over all experts, softmax, keep the top-k, renormalise the k
    weights to sum to 1 (equivalently, softmax over the k selected logits).
    Order of the k slots: descending logit, equal logits -> lower expert id.
  * shard filter and partial sums: same page, section "수정 사항 › b12x에서의
    Expert Parallelism 구현 추가": each node holds a contiguous range of experts;
    the kernel turns the globally routed expert id into a shard-relative index
    and drops token-expert pairs outside the range; a shard's output is a
    partial sum that the caller all-reduces.  Routing is always global (all E
    experts), and the k weights are never renormalised inside a shard, so the
    shards' partial sums add up to the unsharded output.
  * expert MLP: fused gate/up weight w13 with rows [0, F) = gate and
    [F, 2F) = up, SwiGLU a = silu(gate) * up, then the down projection w2
    (same page, section "b12x 버전이 실제 NVFP4 체크포인트를 읽어들이도록
    만들기", mentions the fused gate/up row order; the order used here is the
    library's convention).
  * shared expert: added with weight 1 to every token by the one shard that
    owns it (`has_shared`).
  * W4A4: activations are NVFP4-quantized (block-16 amax/6 -> E4M3, no global
    scale) before both GEMMs: the hidden rows before gate/up (routed and shared
    alike) and the SwiGLU output before down.  The router never sees quantized
    activations.
  * static W4A4 (same page, section "수정 사항": the third fused-MoE backend
    variant is static NVFP4 W4A4): the same two quantization points, each with a
    calibrated per-layer activation global g_a fixed ahead of time (act_global
    = (g_a of h, g_a of the SwiGLU output)), block scale E4M3(amax / (6 g_a)).
"""
import numpy as np

from . import nvfp4

W4A16 = 0
W4A4 = 1
W4A4_STATIC = 2

# Tokens whose k-th and (k+1)-th fp64 logits differ by less than this are
# reported as ambiguous: any GPU selection that differs from the oracle only
# across that boundary is accepted (fp64 dot products summed in another order
# differ by ~1e-13 here).
AMBIGUITY_TAU = 1e-9


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> exact fp64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_logits(x, gate):
    """x: fp64 [T, d]; gate: fp64 [d, E] -> fp64 logits [T, E] (all E experts)."""
    return np.asarray(x, np.float64) @ np.asarray(gate, np.float64)


def route(x, gate, top_k):
    """Global top-k routing.

    Returns dict with
      ids      int32 [T, k]  global expert ids, descending logit, ties -> lower id
      weights  fp64  [T, k]  softmax over the k selected logits
      logits   fp64  [T, E]
      ambiguous bool [T]     k-th / (k+1)-th gap below AMBIGUITY_TAU
    """
    logits = router_logits(x, gate)
    T, E = logits.shape
    assert 1 <= top_k <= E
    order = np.argsort(-logits, axis=1, kind="stable")      # stable: lower id first on ties
    ids = order[:, :top_k].astype(np.int32)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    weights = z / z.sum(axis=1, keepdims=True)
    if top_k < E:
        kth = sel[:, -1]
        nxt = np.take_along_axis(logits, order[:, top_k:top_k + 1], axis=1)[:, 0]
        ambiguous = (kth - nxt) < AMBIGUITY_TAU
    else:
        ambiguous = np.zeros(T, dtype=bool)
    return {"ids": ids, "weights": weights, "logits": logits, "ambiguous": ambiguous}


def shard_filter(ids, offset, num_local):
    """Global ids -> shard-relative ids; -1 marks a dropped (out-of-shard) pair."""
    lam = np.asarray(ids, np.int64) - offset
    keep = (lam >= 0) & (lam < num_local)
    return np.where(keep, lam, -1).astype(np.int32)


def permutation(local_ids, num_local):
    """Group kept pairs by local expert, stable by token.

    local_ids: int32 [T, k] (-1 = dropped).  Pair id p = t * k + j.
    Returns counts int32 [L], offsets int32 [L+1] (exclusive scan, offsets[L] = P),
    perm int32 [P] (pair ids sorted by (local expert, token)).
    """
    T, k = local_ids.shape
    flat = np.asarray(local_ids, np.int64).reshape(-1)
    counts = np.bincount(flat[flat >= 0], minlength=num_local).astype(np.int32)
    offsets = np.zeros(num_local + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    kept = np.nonzero(flat >= 0)[0]
    tok = kept // k
    order = np.lexsort((tok, flat[kept]))                  # primary: expert, secondary: token
    perm = kept[order].astype(np.int32)
    return {"counts": counts, "offsets": offsets, "perm": perm}


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def quantize_input(x, mode, act_global):
    """The activation step before GEMM1 (the identity for W4A16)."""
    if mode == W4A4:
        return nvfp4.fake_quant_act(x)
    if mode == W4A4_STATIC:
        return nvfp4.fake_quant_act(x, act_global[0])
    return x


def expert_mlp(h, w13, w2, mode, act_global=(1.0, 1.0)):
    """h: fp64 [n, d] (already quantized for W4A4); w13: fp64 [2F, d];
    w2: fp64 [d, F] (dequantized).  Returns fp64 [n, d]."""
    F = w13.shape[0] // 2
    u = h @ w13.T
    a = silu(u[:, :F]) * u[:, F:]
    if mode == W4A4:
        a = nvfp4.fake_quant_act(a)
    elif mode == W4A4_STATIC:
        a = nvfp4.fake_quant_act(a, act_global[1])
    return a @ w2.T


def dequant_expert(q):
    """q: dict with w13/w13_scale/g13/w2/w2_scale/g2 for one expert -> fp64 (w13, w2)."""
    w13 = nvfp4.dequantize(q["w13"], q["w13_scale"], q["g13"])
    w2 = nvfp4.dequantize(q["w2"], q["w2_scale"], q["g2"])
    return w13, w2


def expert_term(job):
    """One expert's MLP over its token rows.  job = (quantized expert dict, the
    rows of h it sees (fp64 [n, d]), mode, act_global); returns fp64 [n, d].
    A top-level function of plain values, so that `forward` can hand the
    independent expert terms to a process pool's map."""
    q, h_rows, mode, act_global = job
    w13, w2 = dequant_expert(q)
    return expert_mlp(h_rows, w13, w2, mode, act_global)


def forward(x, gate, experts, shared, top_k, offset, num_local, mode, routing=None, act_global=(1.0, 1.0),
            map_fn=map):
    """The fused MoE layer for one shard.

    x       fp64 [T, d]   (bf16 hidden, exactly widened)
    gate    fp64 [d, E]   (bf16 router weight, exactly widened)
    experts callable or list: experts(l) -> quantized dict for local expert l
            (l in [0, num_local), i.e. global id offset + l)
    shared  quantized dict of the shared expert, or None (has_shared = 0)
    act_global  static W4A4 only: (g_a of h, g_a of the SwiGLU output)
    map_fn  evaluates `expert_term` over the touched experts' jobs, in order
            (the builtin map, or a process pool's); the terms are summed here in
            local-expert order and then the shared term, whatever evaluated them
    Returns dict(out fp64 [T, d], routing..., perm...).
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    r = routing if routing is not None else route(x, gate, top_k)
    lam = shard_filter(r["ids"], offset, num_local)
    pm = permutation(lam, num_local)
    h = quantize_input(x, mode, act_global)
    get = experts if callable(experts) else (lambda l: experts[l])
    flatw = r["weights"].reshape(-1)
    touched = [l for l in range(num_local) if pm["offsets"][l + 1] > pm["offsets"][l]]
    pairs_of = {l: pm["perm"][pm["offsets"][l]:pm["offsets"][l + 1]].astype(np.int64) for l in touched}

    def jobs():
        for l in touched:
            yield (get(l), h[pairs_of[l] // top_k], mode, act_global)
        if shared is not None:
            yield (shared, h, mode, act_global)

    out = np.zeros((T, d), dtype=np.float64)
    terms = iter(map_fn(expert_term, jobs()))
    for l, y in zip(touched, terms):                        # zip stops at `touched` first
        pairs = pairs_of[l]
        out[pairs // top_k] += flatw[pairs][:, None] * y     # at most one pair per (token, expert)
    if shared is not None:
        out += next(terms)
    return {"out": out, "ids": r["ids"], "weights": r["weights"], "logits": r["logits"],
            "ambiguous": r["ambiguous"], "local_ids": lam, **pm}


def normwise_rel_err(y, y_ref):
    """||y - y_ref||_F / ||y_ref||_F over the whole output."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))
