"""The seeded workload generators: shapes, determinism, and the Zipf bias
constant against the value its calibration script wrote.  CPU only."""
import json
import os

import numpy as np
import torch

import workloads
from oracle import moe
from tests.oracle_helpers import to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_shapes_and_determinism():
    w = workloads.WORKLOADS["tiny_w4a16"]
    x1, x2 = workloads.gen_hidden(w), workloads.gen_hidden(w)
    assert x1.shape == (16, 256) and x1.dtype == torch.bfloat16 and torch.equal(x1, x2)
    G = workloads.gen_gate(w)
    assert G.shape == (256, 16)
    w13, w2 = workloads.gen_expert(w, 3)
    assert w13.shape == (256, 256) and w2.shape == (256, 128)
    a13, _ = workloads.gen_expert(w, 4)
    assert not torch.equal(w13, a13)
    # std of the draws: N(0, 1/sqrt(fan_in))
    assert abs(w13.float().std().item() * 16 - 1) < 0.05


def test_zipf_alpha_constant_matches_calibration_file():
    with open(os.path.join(GOLDEN, "zipf_alpha.json")) as f:
        cal = json.load(f)
    assert workloads.ZIPF_ALPHA == cal["alpha"]
    assert abs(cal["top10_share"] - 0.5) < 0.01


def test_zipf_share_on_calibration_draw():
    w = workloads.WORKLOADS["prefill_zipf_shard0_w4a16"]
    cal = workloads.replace(w, hidden_seed=w.hidden_seed + 1000)
    x = to_f64(workloads.gen_hidden(cal, T=1024))
    G = to_f64(workloads.gen_gate(w))
    ids = moe.route(x, G, w.k)["ids"]
    counts = np.bincount(ids.reshape(-1), minlength=w.E)
    share = np.sort(counts)[::-1][:10].sum() / ids.size
    assert 0.46 < share < 0.54
