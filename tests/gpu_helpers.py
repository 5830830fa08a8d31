"""Shared set-up of the GPU parity tests: seeded inputs drawn on the GPU, the
library's own NVFP4 weights (quantized by its GPU quantizer), and the oracle's
independent copy (the same bf16 draws, copied to the host and quantized by the
oracle).  Test infrastructure."""
import sys

import numpy as np
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from oracle import moe
from tests import oracle_pool
from tests.oracle_helpers import to_f64


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    nv.lib()   # raises if the HIP library is not built


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Layer:
    """Inputs of one workload on the GPU plus lazily built oracle views."""

    def __init__(self, w, experts_range=None, gen_all=True):
        self.w = w
        self.x = workloads.gen_hidden(w, "cuda")                       # bf16 [T, d]
        self.G = workloads.gen_gate(w, "cuda")                         # bf16 [d, E]
        self.gate_w = self.G.t().contiguous()                          # bf16 [E, d] (ABI layout)
        lo, n = experts_range if experts_range else (0, w.E)
        self.lo, self.n = lo, n
        self.experts = nv.NVFP4Experts.empty(n, w.d, w.F)              # global ids lo .. lo+n-1
        for i in range(n):
            w13, w2 = workloads.gen_expert(w, lo + i, "cuda")
            nv.quantize_experts(w13.unsqueeze(0), w2.unsqueeze(0), self.experts, i)
        w13, w2 = workloads.gen_expert(w, w.E, "cuda")
        self.shared = nv.quantize_experts(w13.unsqueeze(0), w2.unsqueeze(0))
        torch.cuda.synchronize()
        self._oracle_cache = {}
        self._x64 = None
        self._G64 = None

    @property
    def x64(self):
        if self._x64 is None:
            self._x64 = to_f64(self.x)
        return self._x64

    @property
    def G64(self):
        if self._G64 is None:
            self._G64 = to_f64(self.G)
        return self._G64

    def oracle_expert(self, e):
        """Oracle-quantized expert with global id e (E = the shared expert)."""
        if e not in self._oracle_cache:
            self.prefetch_oracle([e])
        return self._oracle_cache[e]

    def prefetch_oracle(self, ids, batch=16):
        """Quantize experts `ids` with the oracle on the CPU process pool: each
        expert's bf16 draw is made on the GPU (the library's own copy comes
        from the same draw) and its bit patterns are copied to the host."""
        todo = sorted({int(e) for e in ids} - set(self._oracle_cache))
        for i in range(0, len(todo), batch):
            part = todo[i:i + batch]
            jobs = []
            for e in part:
                w13, w2 = workloads.gen_expert(self.w, e, "cuda")
                jobs.append((w13.view(torch.int16).cpu().numpy().view(np.uint16),
                             w2.view(torch.int16).cpu().numpy().view(np.uint16)))
            for e, q in zip(part, oracle_pool.pool_map(oracle_pool.quantize_expert_bits, jobs)):
                self._oracle_cache[e] = q

    def local_weights(self, offset, L):
        assert self.lo <= offset and offset + L <= self.lo + self.n
        return self.experts.slice(offset - self.lo, L)

    def run(self, offset, L, has_shared, mode, path=nv.PATH_AUTO, T=None, x=None, out=None, ws=None,
            ws_fill=None, act_global=None):
        w = self.w
        act_global = w.act_global if act_global is None else act_global
        x = self.x if x is None else x
        T = x.shape[0]
        p = nv.make_problem(T, w.d, w.F, w.E, w.k, offset, L, has_shared, mode, path, act_global)
        if ws is None:
            ws = nv.alloc_workspace(p)
        if ws_fill is not None:
            ws.fill_(ws_fill)
        if out is None:
            out = torch.empty(T, w.d, dtype=torch.bfloat16, device="cuda")
        nv.moe_nvfp4_forward(p, x, self.gate_w, self.local_weights(offset, L),
                             self.shared if has_shared else None, ws, out)
        torch.cuda.synchronize()
        return out

    def oracle_full(self, offset, L, has_shared, mode, act_global=None):
        """The oracle's whole [T, d] output for this layer's tokens (expert
        terms on the CPU process pool, summed in the oracle's fixed order)."""
        act_global = self.w.act_global if act_global is None else act_global
        r = moe.route(self.x64, self.G64, self.w.k)
        ids = r["ids"].reshape(-1)
        need = [int(e) for e in np.unique(ids[(ids >= offset) & (ids < offset + L)])]
        self.prefetch_oracle(need + ([self.w.E] if has_shared else []))
        return oracle_pool.forward(self.x64, self.G64, lambda l: self.oracle_expert(offset + l),
                                   self.oracle_expert(self.w.E) if has_shared else None,
                                   self.w.k, offset, L, mode, routing=r, act_global=act_global)


def rel_err(gpu_bf16, ref64):
    return moe.normwise_rel_err(to_f64(gpu_bf16), ref64)


def tol(mode):
    return 1e-2 if mode == workloads.W4A16 else 3e-2


