"""Seeded synthetic inputs for the fused NVFP4 MoE layer.

Shared by the tests (which feed both the HIP library and the CPU oracle) and the
benchmark.  Holds none of the layer's arithmetic: it only draws bf16 tensors
(hidden states, router weight, full-precision expert weights) and states the
workload shapes.  Quantization to NVFP4 is done by each consumer on its own side.

The workloads stand in for the model on the page "Serving Solar Open 2 on DGX
Spark" (backend.ai, section "Solar Open 2 개요": 320 routed experts + 1 shared,
top-8) served with two contiguous expert shards 0-159 / 160-319 (section "수정
사항 › b12x에서의 Expert Parallelism 구현 추가").  The pages give no hidden or
expert width; d_model = 4096 and d_ff = 1024 are synthetic choices.

Draws use torch.Generator on the requested device; the same seed gives the same
values on the same device type (CPU and GPU streams differ, so a test generates
on the device it runs on and copies to the host for the oracle).
"""
from dataclasses import dataclass, field
import math

import torch

W4A16 = 0
W4A4 = 1
W4A4_STATIC = 2

# Zipf exponent of the skewed-routing prefill workload, and the bias scale that
# gives its 10 hottest experts ~50% of the T*k assignments.  ZIPF_ALPHA was
# found by bisection with the oracle's router on a T=4096 calibration draw
# (tests/golden/make_zipf_alpha.py writes tests/golden/zipf_alpha.json, and a
# CPU test checks this constant against that file).
ZIPF_S = 1.2
ZIPF_ALPHA = 0.5869140625


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    F: int
    E: int
    k: int
    offset: int
    L: int
    has_shared: bool
    mode: int
    hidden_seed: int
    gate_seed: int
    weight_seed: int
    router: str = "std"        # "std": gate N(0, gate_std); "unit": N(0, 1/sqrt(d)); "zipf"
    gate_std: float = 0.02
    act_global: tuple = (1.0, 1.0)   # static W4A4: activation globals of h and of the SwiGLU output
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_w4a16": Workload("tiny_w4a16", T=16, d=256, F=128, E=16, k=2, offset=0, L=16,
                           has_shared=True, mode=W4A16, hidden_seed=100, gate_seed=100,
                           weight_seed=100, note="tiny layer, full expert range"),
    "decode_shard0_w4a16": Workload("decode_shard0_w4a16", T=64, d=4096, F=1024, E=320, k=8,
                                    offset=0, L=160, has_shared=True, mode=W4A16,
                                    hidden_seed=101, gate_seed=1234, weight_seed=1234,
                                    note="decode, experts 0-159 + shared, memory-bound"),
    "shard1_w4a4_t512": Workload("shard1_w4a4_t512", T=512, d=4096, F=1024, E=320, k=8,
                                 offset=160, L=160, has_shared=False, mode=W4A4,
                                 hidden_seed=102, gate_seed=1234, weight_seed=1234,
                                 note="second shard (experts 160-319), W4A4 dynamic"),
    # the same shard in static W4A4: fixed activation globals amax / (6 * 448)
    # for calibrated amax 5 (the N(0, 1) hidden rows) and 12 (the SwiGLU output)
    "shard1_w4a4_static_t512": Workload("shard1_w4a4_static_t512", T=512, d=4096, F=1024, E=320, k=8,
                                        offset=160, L=160, has_shared=False, mode=W4A4_STATIC,
                                        hidden_seed=102, gate_seed=1234, weight_seed=1234,
                                        act_global=(0.0018601190531626344, 0.004464285913854837),
                                        note="second shard, static W4A4 (calibrated activation globals)"),
    "prefill_all_w4a4": Workload("prefill_all_w4a4", T=8192, d=4096, F=1024, E=320, k=8,
                                 offset=0, L=320, has_shared=True, mode=W4A4,
                                 hidden_seed=103, gate_seed=103, weight_seed=1234,
                                 router="unit", note="prefill, all 320 experts, compute-bound"),
    "prefill_zipf_shard0_w4a16": Workload("prefill_zipf_shard0_w4a16", T=16384, d=4096, F=1024,
                                          E=320, k=8, offset=0, L=160, has_shared=True,
                                          mode=W4A16, hidden_seed=104, gate_seed=104,
                                          weight_seed=1234, router="zipf",
                                          note="skewed routing (Zipf 1.2), shard 0"),
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def replace(w: Workload, **kw) -> Workload:
    d = {k: getattr(w, k) for k in w.__dataclass_fields__}
    d.update(kw)
    return Workload(**d)


def gen_hidden(w: Workload, device="cpu", T=None):
    """bf16 [T, d], N(0, 1); the zipf workload pins column 0 to 1 (the channel
    that carries the per-expert router bias)."""
    T = w.T if T is None else T
    x = torch.randn(T, w.d, generator=_gen(w.hidden_seed * 7919 + 1, device), device=device,
                    dtype=torch.float32)
    if w.router == "zipf":
        x[:, 0] = 1.0
    return x.to(torch.bfloat16)


def zipf_bias(w: Workload, alpha=None):
    """Per-expert router bias alpha * ln(Zipf_s pmf of a seeded rank), up to a
    constant (constants do not change top-k or softmax).  fp64 [E]."""
    alpha = ZIPF_ALPHA if alpha is None else alpha
    g = _gen(w.gate_seed * 7919 + 3, "cpu")
    ranks = torch.randperm(w.E, generator=g).to(torch.float64) + 1.0
    return -ZIPF_S * alpha * torch.log(ranks)


def gen_gate(w: Workload, device="cpu", alpha=None):
    """bf16 [d, E] router weight (row-major, one row per hidden channel)."""
    if w.router == "std":
        std = w.gate_std
    elif w.router == "unit":
        std = 1.0 / math.sqrt(w.d)
    elif w.router == "zipf":
        std = 1.0 / math.sqrt(w.d - 1)
    else:
        raise ValueError(w.router)
    G = torch.randn(w.d, w.E, generator=_gen(w.gate_seed * 7919 + 2, device), device=device,
                    dtype=torch.float32) * std
    if w.router == "zipf":
        G[0, :] = zipf_bias(w, alpha).to(torch.float32).to(device)
    return G.to(torch.bfloat16)


def expert_seed(weight_seed, expert):
    return weight_seed * 100003 + 17 * expert + 5


def gen_expert(w: Workload, expert, device="cpu"):
    """Full-precision weights of one expert, bf16, N(0, 1/sqrt(fan_in)):
    w13 [2F, d] (rows [0,F) gate, [F,2F) up) and w2 [d, F].
    `expert` is the global routed id in [0, E); E denotes the shared expert."""
    g = _gen(expert_seed(w.weight_seed, expert), device)
    w13 = torch.randn(2 * w.F, w.d, generator=g, device=device, dtype=torch.float32)
    w13 = (w13 * (1.0 / math.sqrt(w.d))).to(torch.bfloat16)
    w2 = torch.randn(w.d, w.F, generator=g, device=device, dtype=torch.float32)
    w2 = (w2 * (1.0 / math.sqrt(w.F))).to(torch.bfloat16)
    return w13, w2


SHARED = -1


def global_id(w: Workload, local):
    """Local expert index -> global id used for seeding (SHARED -> E)."""
    return w.E if local == SHARED else w.offset + local
