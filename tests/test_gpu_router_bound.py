"""The hardware assumption behind certified routing, measured.

Above 128 tokens the router computes fp32 logits with bf16 MFMAs and bounds
their error by gamma_n * ||x|| * ||g_e|| (gamma_n = n u / (1 - n u),
u = 2^-23, n = d + number of K slices): the standard bound for n fp32
additions in any order, each with a relative error of at most one fp32 ulp.
bf16 x bf16 products are exact in fp32, so the bound holds if the matrix
core's internal accumulation is at least as precise as fp32 with truncation,
which the instruction set does not state.  Routing (the page "Serving Solar
Open 2 on DGX Spark", section on expert parallelism in b12x: every shard must
agree on the globally routed experts) is bit-exact only while it holds.

This test reads the fp32 logit partials the routing call leaves in its
workspace (white box: the workspace starts with the 8-byte barrier and error
words, padded to 256 bytes, followed by fp32 partials [KS][T][E]) and compares
them with the exact logits, on the prefill workloads' inputs and on rows built
to make every accumulation step round (constant rows of 8-significant-bit
values, whose products have 16 significant bits).  It asserts the bound and
logs the measured margin, both against the bound the router uses and against
the sharper gamma_d * sum |x_i g_i|."""
import math

import numpy as np
import pytest
import torch

import nvfp4_expert_layer_amd as nv
import workloads
from tests.gpu_helpers import log, require_gpu

pytestmark = pytest.mark.gpu

U = 2.0 ** -23
PART_OFFSET = 256


def k_slices(T, E, d):
    """The number of K slices the certified logits kernel splits d into: with
    at most 320 experts (more than 128) and at least 4096 tokens, one
    workgroup per 64 tokens and enough slices for ~256 workgroups; otherwise
    64 x 64 output tiles and enough slices for ~512 (~192 from 512 to 1023
    tokens); at most 16 and at most d / 256 either way."""
    if 128 < E <= 320 and T >= 4096:
        base, want = -(-T // 64), 256
    else:
        base, want = -(-T // 64) * -(-E // 64), (192 if 512 <= T < 1024 else 512)
    ks = -(-want // base)
    return max(1, min(ks, 16, max(1, d // 256)))


def gamma(n):
    return n * U / (1.0 - n * U)


def measure(x, G, name):
    """x bf16 [T, d] and G bf16 [d, E] on the GPU -> (worst error / the router's
    bound, worst error / gamma_d sum|x g|)."""
    T, d = x.shape
    E = G.shape[1]
    assert T > 128, "the certified logits kernel runs above 128 tokens"
    p = nv.make_problem(T, d, 256, E, 8, 0, E, False, workloads.W4A16)
    ws = nv.alloc_workspace(p)
    ws.fill_(0xFF)                                   # NaN everywhere the kernel does not write
    nv.moe_nvfp4_route(p, x, G.t().contiguous(), ws)
    torch.cuda.synchronize()
    KS = k_slices(T, E, d)
    part = ws[PART_OFFSET:PART_OFFSET + KS * T * E * 4].view(torch.float32).view(KS, T, E)
    got = part.double().sum(0).cpu().numpy()         # fp64 sum: only the MFMA partials' error remains
    x64 = x.double().cpu().numpy()
    G64 = G.double().cpu().numpy()
    exact = x64 @ G64                                # bf16 products and their sums are exact enough in fp64
    absdot = np.abs(x64) @ np.abs(G64)
    nx = np.linalg.norm(x64, axis=1)[:, None]
    ng = np.linalg.norm(G64, axis=0)[None, :]
    err = np.abs(got - exact)
    assert np.all(np.isfinite(got)), "a logit partial was not written"
    r_bound = float(np.max(err / (gamma(d + KS) * nx * ng + d * 2.0 ** -126)))
    with np.errstate(invalid="ignore", divide="ignore"):
        sharp = np.where(absdot > 0, err / (gamma(d) * absdot), 0.0)
    r_sharp = float(np.max(sharp))
    log(f"{name}: T={T} d={d} E={E} KS={KS}: worst error = {r_bound:.3e} of the router's bound, "
        f"{r_sharp:.3e} of gamma_d * sum|x g| (max abs error {err.max():.3e})")
    return r_bound, r_sharp


@pytest.mark.parametrize("name", ["prefill_all_w4a4", "prefill_zipf_shard0_w4a16"])
def test_certified_logit_error_within_bound_full_size(name):
    require_gpu()
    w = workloads.WORKLOADS[name]
    x = workloads.gen_hidden(w, "cuda")
    G = workloads.gen_gate(w, "cuda")
    r_bound, r_sharp = measure(x, G, name)
    assert r_bound <= 1.0
    assert r_sharp <= 1.0


def test_certified_logit_error_within_bound_rounding_rows():
    """Constant rows: each product has 16 significant bits and the partial sums
    grow to 4096 times a product, so nearly every fp32 addition rounds."""
    require_gpu()
    T, d, E = 4096, 4096, 512                         # one K slice: 4096-long accumulations
    vals = torch.tensor([1.9921875, 1.4921875, 1.0078125, 1.7421875, -1.9921875, 1.2421875],
                        dtype=torch.float32)
    gen = torch.Generator().manual_seed(77)
    x = torch.randn(T, d, generator=gen)
    G = torch.randn(d, E, generator=gen) * 0.02
    for t in range(0, 192):
        x[t] = vals[t % len(vals)] * (2.0 ** (t % 5))
    for e in range(0, 32):
        G[:, e] = vals[(e * 5) % len(vals)] * (2.0 ** -(e % 7))
    for t in range(192, 256):                        # alternating signs: cancellation
        x[t] = vals[t % len(vals)] * torch.where(torch.arange(d) % 2 == 0, 1.0, -1.0)
    x = x.to(torch.bfloat16).cuda()
    G = G.to(torch.bfloat16).cuda()
    assert math.isclose(float(x[0, 0]), 1.9921875)
    assert k_slices(T, E, d) == 1
    r_bound, r_sharp = measure(x, G, "rounding rows")
    assert r_bound <= 1.0
    assert r_sharp <= 1.0
