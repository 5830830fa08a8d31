"""Builds oracle-side inputs (fp64 views and oracle-quantized experts) from the
seeded bf16 draws in `workloads`.  Test infrastructure."""
import numpy as np
import torch

import workloads
from oracle import nvfp4


def to_f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def quantize_expert_oracle(w13_bf16, w2_bf16):
    q13 = nvfp4.quantize_weight(to_f64(w13_bf16).astype(np.float32))
    q2 = nvfp4.quantize_weight(to_f64(w2_bf16).astype(np.float32))
    return {"w13": q13["codes"], "w13_scale": q13["scales"], "g13": q13["g"],
            "w2": q2["codes"], "w2_scale": q2["scales"], "g2": q2["g"]}


class OracleExperts:
    """Lazily quantized experts of one workload (cached), generated on `device`."""

    def __init__(self, w, device="cpu"):
        self.w = w
        self.device = device
        self.cache = {}

    def get_global(self, e):
        if e not in self.cache:
            w13, w2 = workloads.gen_expert(self.w, e, self.device)
            self.cache[e] = quantize_expert_oracle(w13, w2)
        return self.cache[e]

    def local(self, offset):
        return lambda l: self.get_global(offset + l)

    def shared(self):
        return self.get_global(self.w.E)


def tiny_problem(T=4, d=32, F=16, E=8, k=2, seed=0, gate_std=0.5):
    """Random tiny layer (CPU draws) for brute-force comparisons."""
    w = workloads.Workload("tiny_brute", T=T, d=d, F=F, E=E, k=k, offset=0, L=E, has_shared=True,
                           mode=workloads.W4A16, hidden_seed=seed, gate_seed=seed,
                           weight_seed=seed + 1, gate_std=gate_std)
    x = to_f64(workloads.gen_hidden(w))
    G = to_f64(workloads.gen_gate(w))
    ex = OracleExperts(w)
    experts = [ex.get_global(e) for e in range(E)]
    return w, x, G, experts, ex.shared()
