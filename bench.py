#!/usr/bin/env python3
"""Benchmark of the fused NVFP4 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
                    [--workload NAME --tokens T]

A step is one call of moe_nvfp4_forward (router top-k, shard filter,
permutation, [W4A4 activation quantizer], GEMM1 + SwiGLU, GEMM2, weighted
combine with the shared expert) over one batch of synthetic tokens whose
weights and inputs are already resident in HBM.  Prints ONE JSON line for the
headline workload (the T=64 expert-shard decode step), with:
  value      tokens/s of the whole job (T * K / elapsed, wall clock around
             exactly K steps, synchronized on both sides; before the W warm-up
             steps, ~0.3 s of untimed calls let the GPU clocks settle)
  per_call_us  median and min of single calls (HIP events between consecutive
             calls: N = 200 for the decode/shard workloads, 20 for prefill)
  roofline   the dominant kernel (GEMM1 + SwiGLU) against its roof (HBM for
             weight streaming, the 16-bit MFMA peak for tiles): algorithmic
             bytes (or flops) per launch / its average duration from HIP events
             recorded around it in the timed steps, on the kernels' stream
  graph_replay  the same forward captured once in a HIP graph, pre-warmed
             like the direct calls, K replays timed
  cpu_baseline  the CPU oracle timed on a bounded sample of the workload
  secondary  the same measurements for the other four workloads (tiny layer,
             T=512 W4A4 second shard, T=8192 all-expert W4A4 prefill, T=16384
             Zipf-skewed W4A16 shard), each with its own roofline and oracle
--all prints one line per workload instead (a report, not the default line).
--tokens runs the named workload alone at another token count (e.g. the
decode shard at T=1), with every measurement above; its traffic is null.
"""
import argparse
import re
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import nvfp4_expert_layer_amd as nv  # noqa: E402
import workloads  # noqa: E402

METRIC = "NVFP4 MoE layer tokens/s; % of HBM roofline (T=64), % MFMA peak (T=8192)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HEADLINE = "decode_shard0_w4a16"
SECONDARY = ["tiny_w4a16", "shard1_w4a4_t512", "prefill_all_w4a4", "prefill_zipf_shard0_w4a16"]
# per-call timing sample sizes (median and min are reported)
PER_CALL_N = {"tiny_w4a16": 200, "decode_shard0_w4a16": 200, "shard1_w4a4_t512": 200,
              "shard1_w4a4_static_t512": 200, "prefill_all_w4a4": 20, "prefill_zipf_shard0_w4a16": 20}
# tokens of each workload the CPU oracle is timed on (a bounded sample, ~3-15 s
# of host time each; the tiny layer whole, repeated)
CPU_SAMPLE = {"tiny_w4a16": 16, "decode_shard0_w4a16": 24, "shard1_w4a4_t512": 24,
              "shard1_w4a4_static_t512": 24, "prefill_all_w4a4": 16, "prefill_zipf_shard0_w4a16": 32}
STAGES = ["route_permute", "act_quant", "gemm1_swiglu", "gemm2", "combine"]
G1_EVERY = 4                    # timed steps per GEMM1 event pair
TOKENS_OVERRIDDEN = False       # --tokens: the workload runs at another token count
PREWARM_S = 0.3                 # untimed forward calls before the warm-up steps (clock settling)
CSRC = os.path.join(ROOT, "nvfp4_expert_layer_amd", "csrc")
from nvfp4_expert_layer_amd.build import EXTRA_FLAGS as BUILD_FLAGS   # noqa: E402  (plain dict, no compilation)
# sources whose machine code the dominant kernel of each path is built from
KERNEL_SOURCES = {"decode": ["decode.hip", "device_common.h", "kernels.h"],
                  "mid": ["mid.hip", "device_common.h", "kernels.h"],
                  "prefill": ["prefill.hip", "device_common.h", "kernels.h"]}


def kernel_source_hash(path):
    """Hash of what the path's GEMM kernels are built from: their source file,
    the device helpers, and the two argument structs they receive (the rest of
    kernels.h -- other kernels' structs, host-side declarations -- is left out:
    it changes no GEMM kernel)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            text = fh.read()
        t = text.decode()
        if f == "kernels.h":
            t = "".join(re.findall(r"struct (?:ExpertWeights|GemmArgs) \{.*?\n\};", t, flags=re.S))
        t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)          # comments do not change a kernel
        t = re.sub(r"//[^\n]*", "", t)
        t = " ".join(t.split())                                # nor does layout
        h.update(t.encode())
    h.update(" ".join(BUILD_FLAGS.get(KERNEL_SOURCES[path][0], [])).encode())   # per-source compiler options
    return h.hexdigest()[:16]


def measured_traffic(path, workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary profiles/traffic_gemm1_<workload>.txt (FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy's reading), or None when there is none or the kernel
    sources changed since the counters were taken."""
    fn = os.path.join(ROOT, "profiles", f"traffic_gemm1_{workload}.txt")
    if TOKENS_OVERRIDDEN or not os.path.exists(fn):      # (the counters are of the workload's own T)
        return None
    vals = {}
    with open(fn) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != kernel_source_hash(path):
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def prewarm(call):
    """Untimed calls for PREWARM_S seconds (the GPU's clocks settle under load);
    returns how many ran."""
    t_end = time.perf_counter() + PREWARM_S
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            call()
        n += 10
        torch.cuda.synchronize()
    return n


GRAPH_PROBE_CALLS = 50


def graph_probe(name):
    """The forward captured in a HIP graph and replayed untimed for PREWARM_S,
    then GRAPH_PROBE_CALLS direct forward calls and GRAPH_PROBE_CALLS replays,
    for a kernel trace that compares the two (see --trace-summary).  Prints
    both wall times."""
    w = workloads.WORKLOADS[name]
    local, shared = build_weights(w)
    gate_w = workloads.gen_gate(w, "cuda").t().contiguous()
    x = workloads.gen_hidden(w, "cuda")
    p = nv.make_problem(w.T, w.d, w.F, w.E, w.k, w.offset, w.L, w.has_shared, w.mode, nv.PATH_AUTO, w.act_global)
    ws = nv.alloc_workspace(p)
    out = torch.empty(w.T, w.d, dtype=torch.bfloat16, device="cuda")
    prewarm(lambda: nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out)
    # the capture leaves the chip idle for a while: pre-warm again (with
    # replays) so that both timed phases start at a settled clock
    prewarm(graph.replay)
    t0 = time.perf_counter()
    for _ in range(GRAPH_PROBE_CALLS):
        nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out)
    torch.cuda.synchronize()
    direct = (time.perf_counter() - t0) / GRAPH_PROBE_CALLS
    t0 = time.perf_counter()
    for _ in range(GRAPH_PROBE_CALLS):
        graph.replay()
    torch.cuda.synchronize()
    replay = (time.perf_counter() - t0) / GRAPH_PROBE_CALLS
    print(json.dumps({"workload": name, "direct_us": round(direct * 1e6, 1), "graph_replay_us": round(replay * 1e6, 1),
                      "calls": GRAPH_PROBE_CALLS}))


def trace_summary(csv_path, per_call):
    """Per-kernel average durations and the mean gap between kernels in the two
    phases of a --graph-probe run, from rocprofv3's kernel_trace.csv: the last
    GRAPH_PROBE_CALLS forwards are graph replays, the GRAPH_PROBE_CALLS before
    them direct calls (per_call kernels a forward)."""
    import csv
    import collections
    rows = [r for r in csv.DictReader(open(csv_path)) if "moe::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    n, c = len(rows), per_call * GRAPH_PROBE_CALLS
    phases = {"direct": rows[n - 2 * c: n - c], "graph_replay": rows[n - c:]}
    for label, ph in phases.items():
        d = collections.OrderedDict()
        for r in ph:
            d.setdefault(r["Kernel_Name"][:60], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        span = (int(ph[-1]["End_Timestamp"]) - int(ph[0]["Start_Timestamp"])) / 1e3 / GRAPH_PROBE_CALLS
        gaps = [(int(ph[i + 1]["Start_Timestamp"]) - int(ph[i]["End_Timestamp"])) / 1e3 for i in range(len(ph) - 1)]
        print(f"{label}: {span:.1f} us per forward, mean gap between kernels {sum(gaps) / len(gaps):.2f} us")
        for k, v in d.items():
            print(f"   {k:60s} {sum(v) / len(v):9.2f} us  ({len(v)} calls)")


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain copy of known size in one elementwise kernel (y = x + 0, so that
    it is a kernel dispatch and not a DMA blit), for scaling the FETCH_SIZE /
    WRITE_SIZE counters: each dispatch reads and writes nbytes."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.add(src, 0, out=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps, "ms": round(dt * 1e3, 3),
                      "GBps_read_plus_write": round(2 * nbytes / dt / 1e9, 1)}), flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, e):
        """Record event e on torch's current stream (the stream the forward runs on)."""
        if self.lib.hipEventRecord(e, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def build_weights(w):
    """NVFP4 weights of the shard's experts and the shared expert, drawn and
    quantized on the GPU (the library's quantizer)."""
    local = nv.NVFP4Experts.empty(w.L, w.d, w.F)
    for i in range(w.L):
        w13, w2 = workloads.gen_expert(w, w.offset + i, "cuda")
        nv.quantize_experts(w13.unsqueeze(0), w2.unsqueeze(0), local, i)
    shared = None
    if w.has_shared:
        w13, w2 = workloads.gen_expert(w, w.E, "cuda")
        shared = nv.quantize_experts(w13.unsqueeze(0), w2.unsqueeze(0))
    torch.cuda.synchronize()
    return local, shared


def algorithmic(w, counts):
    """Algorithmic bytes / flops of the layer and of its kernels (touched experts
    only, no padding)."""
    d, F, T = w.d, w.F, w.T
    touched = int((counts > 0).sum()) + (1 if w.has_shared else 0)
    P = int(counts.sum())
    rows = P + (T if w.has_shared else 0)
    w13_b = 2 * F * d // 2 + 2 * F * d // 16           # codes + scales per expert
    w2_b = d * F // 2 + d * F // 16
    fp4 = 9 / 16                                       # bytes per element of NVFP4 activations
    w4a4 = w.mode != workloads.W4A16
    a_in = T * d * (fp4 if w4a4 else 2)
    act = rows * F * (fp4 if w4a4 else 2)
    g1_bytes = touched * w13_b + a_in + act
    g2_bytes = touched * w2_b + act + rows * d * 2     # expert outputs are bf16
    layer_bytes = touched * (w13_b + w2_b) + w.E * d * 2 + T * d * 2 + T * d * 2
    g1_flops = 2.0 * rows * d * 2 * F
    g2_flops = 2.0 * rows * F * d
    layer_flops = 2.0 * T * d * w.E + g1_flops + g2_flops
    return dict(touched=touched, P=P, rows=rows, g1_bytes=g1_bytes, g2_bytes=g2_bytes,
                layer_bytes=layer_bytes, g1_flops=g1_flops, g2_flops=g2_flops, layer_flops=layer_flops)


def bench_workload(name, steps, warmup, hip):
    w = workloads.WORKLOADS[name]
    local, shared = build_weights(w)
    x = workloads.gen_hidden(w, "cuda")
    gate_w = workloads.gen_gate(w, "cuda").t().contiguous()
    p = nv.make_problem(w.T, w.d, w.F, w.E, w.k, w.offset, w.L, w.has_shared, w.mode, nv.PATH_AUTO, w.act_global)
    ws = nv.alloc_workspace(p)
    out = torch.empty(w.T, w.d, dtype=torch.bfloat16, device="cuda")
    # pre-warm (untimed): the GPU's clocks need ~0.1-0.2 s of load to settle; at
    # T=64 twenty steps right after set-up measured 409 us/step, 222 after 20
    # more, 217 after 200 (the per-call median is the same in each)
    prewarm_calls = prewarm(lambda: nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out))
    for _ in range(warmup):
        nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out)
    # timed region: K steps.  The dominant kernel's duration is measured live:
    # the two events around GEMM1 (slots 2 and 3), on the stream the kernels run
    # on, in every G1_EVERY-th step (each event record takes ~2.5 us of the
    # stream's time, so they are not recorded in every step)
    sampled = list(range(0, steps, G1_EVERY))
    g1ev = hip.create(2 * len(sampled))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        if s % G1_EVERY == 0:
            i = s // G1_EVERY
            nv.moe_nvfp4_forward_timed(p, x, gate_w, local, shared, ws, out,
                                       [None, None, g1ev[2 * i], g1ev[2 * i + 1]])
        else:
            nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    g1_ms = sum(hip.elapsed_ms(g1ev[2 * i], g1ev[2 * i + 1]) for i in range(len(sampled))) / len(sampled)
    hip.destroy(g1ev)
    # the same forward captured once in a HIP graph and replayed K times (a
    # deployment that removes the host launch gaps); reported beside `value`
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out)
    # the capture leaves the chip idle long enough for its clock to drop:
    # replays are pre-warmed like the direct calls (20 replays right after the
    # capture measured 243 us per forward at T=64, 222 after 0.3 s of replays)
    prewarm(graph.replay)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    tg = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_s = time.perf_counter() - tg
    del graph
    # single calls: an event between consecutive calls (N of them), median and min
    n_calls = max(PER_CALL_N.get(name, 20), steps)
    cev = hip.create(n_calls + 1)
    hip.record(cev[0])
    for i in range(n_calls):
        nv.moe_nvfp4_forward(p, x, gate_w, local, shared, ws, out)
        hip.record(cev[i + 1])
    torch.cuda.synchronize()
    call_us = sorted(hip.elapsed_ms(cev[i], cev[i + 1]) * 1e3 for i in range(n_calls))
    hip.destroy(cev)
    per_call = {"median": round(call_us[n_calls // 2] if n_calls % 2 else
                                0.5 * (call_us[n_calls // 2 - 1] + call_us[n_calls // 2]), 2),
                "min": round(call_us[0], 2), "n": n_calls,
                "tokens_per_s_at_median": None}
    per_call["tokens_per_s_at_median"] = round(w.T / (per_call["median"] * 1e-6), 1)
    # per-stage breakdown from a separate, untimed pass with all six events
    nb = min(steps, 10)
    evs = hip.create(6 * nb)
    for s in range(nb):
        nv.moe_nvfp4_forward_timed(p, x, gate_w, local, shared, ws, out, evs[6 * s:6 * s + 6])
    torch.cuda.synchronize()
    stage_ms = {k: 0.0 for k in STAGES}
    for s in range(nb):
        e = evs[6 * s:6 * s + 6]
        for i, k in enumerate(STAGES):
            stage_ms[k] += hip.elapsed_ms(e[i], e[i + 1]) / nb
    hip.destroy(evs)
    counts = torch.empty(w.L, dtype=torch.int32, device="cuda")
    nv.moe_nvfp4_route(p, x, gate_w, ws, counts=counts)
    torch.cuda.synchronize()
    alg = algorithmic(w, counts.cpu())
    ms = elapsed * 1e3 / steps
    path = {nv.PATH_DECODE: "decode", nv.PATH_MID: "mid", nv.PATH_PREFILL: "prefill"}[nv.moe_nvfp4_resolved_path(p)]
    g1_s = g1_ms * 1e-3
    # the binding roofline of GEMM1 is the one its algorithmic bytes or flops
    # come closer to (HBM for weight streaming, the 16-bit MFMA peak for tiles)
    hbm_ach = alg["g1_bytes"] / g1_s / 1e9
    mfma_ach = alg["g1_flops"] / g1_s / 1e12
    if hbm_ach / HBM_PEAK_GBS >= mfma_ach / BF16_PEAK_TFLOPS:
        roof = {"kernel": "gemm1_swiglu", "bound": "hbm", "achieved": round(hbm_ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(hbm_ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(path, name),
                "algorithmic_bytes_per_launch": int(alg["g1_bytes"]), "launch_us": round(g1_ms * 1e3, 2)}
    else:
        roof = {"kernel": "gemm1_swiglu", "bound": "mfma", "achieved": round(mfma_ach, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(mfma_ach / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(path, name),
                "algorithmic_flops_per_launch": alg["g1_flops"], "launch_us": round(g1_ms * 1e3, 2)}
    roof["path"] = path
    layer_hbm_frac = alg["layer_bytes"] / (HBM_PEAK_GBS * 1e9) / (ms * 1e-3)
    layer_mfma_frac = alg["layer_flops"] / (BF16_PEAK_TFLOPS * 1e12) / (ms * 1e-3)
    res = {"workload": name, "tokens_per_s": w.T * steps / elapsed, "ms_per_step": ms,
           "prewarm": {"seconds": PREWARM_S, "calls": prewarm_calls},
           "graph_tokens_per_s": w.T * steps / graph_s, "graph_ms_per_step": graph_s * 1e3 / steps,
           "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
           "roofline": roof, "per_call_us": per_call, "layer_hbm_frac": round(layer_hbm_frac, 4),
           "layer_mfma_frac": round(layer_mfma_frac, 4),
           "touched_experts": alg["touched"], "local_pairs": alg["P"],
           # the type the GEMMs multiply in: W4A4 on the tiled and dense
           # weight-streaming paths multiplies exact NVFP4 products in f16,
           # everything else in bf16
           "dtype": "f16" if (path != "decode" and w.mode != workloads.W4A16) else "bf16"}
    del local, shared, ws
    torch.cuda.empty_cache()
    return w, res


def cpu_baselines(names):
    """The oracle (numpy fp64, as it stands: experts one after another, BLAS on
    all host cores it may use) timed on the first CPU_SAMPLE[name] tokens of each
    workload; the weights those tokens touch are drawn on the CPU and quantized
    by the oracle on a process pool beforehand (untimed).  Runs before anything
    touches the GPU."""
    import numpy as np
    from oracle import moe
    from tests import oracle_pool
    from tests.oracle_helpers import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    cores = len(os.sched_getaffinity(0))
    res = {}
    cache = {}
    for name in names:
        w = workloads.WORKLOADS[name]
        n = min(CPU_SAMPLE.get(name, 16), w.T)
        x = to_f64(workloads.gen_hidden(w, "cpu", T=n))
        G = to_f64(workloads.gen_gate(w, "cpu"))
        ids = moe.route(x, G, w.k)["ids"].reshape(-1)
        need = sorted({int(e) for e in ids if w.offset <= e < w.offset + w.L})
        if w.has_shared:
            need.append(w.E)
        key = lambda e: (w.weight_seed, w.d, w.F, w.E, e)
        todo = [e for e in need if key(e) not in cache]
        jobs = []
        for e in todo:
            w13, w2 = workloads.gen_expert(w, e, "cpu")
            jobs.append((w13.view(torch.int16).numpy().view(np.uint16), w2.view(torch.int16).numpy().view(np.uint16)))
        for e, q in zip(todo, oracle_pool.pool_map(oracle_pool.quantize_expert_bits, jobs)):
            cache[key(e)] = q
        reps, dt = 0, 0.0
        while reps == 0 or dt < 1.0:          # the tiny layer is repeated to >= 1 s
            t0 = time.perf_counter()
            moe.forward(x, G, lambda l: cache[key(w.offset + l)], cache.get(key(w.E)), w.k, w.offset, w.L,
                        w.mode, act_global=w.act_global)
            dt += time.perf_counter() - t0
            reps += 1
        res[name] = {"value": round(n * reps / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                     "sample": f"first {n} of {w.T} tokens of {name} ({len(need)} experts touched"
                               f"{', x%d' % reps if reps > 1 else ''}); numpy fp64, BLAS threads {threads}, "
                               f"host cores {cores}; {dt:.1f} s"}
    oracle_pool.pool().shutdown()
    return res


def config_of(w):
    c = {"workload": w.name, "T": w.T, "d_model": w.d, "d_ff": w.F, "experts": w.E, "top_k": w.k,
         "local_expert_offset": w.offset, "num_local_experts": w.L, "shared": int(w.has_shared),
         "mode": {workloads.W4A16: "W4A16", workloads.W4A4: "W4A4", workloads.W4A4_STATIC: "W4A4 static"}[w.mode]}
    if w.mode == workloads.W4A4_STATIC:
        c["act_global"] = list(w.act_global)
    return c


def summary(w, r, cpu):
    """The measurements of one workload (a secondary entry)."""
    d = {"config": config_of(w), "dtype": r["dtype"], "tokens_per_s": round(r["tokens_per_s"], 1),
         "ms_per_step": round(r["ms_per_step"], 4), "per_call_us": r["per_call_us"], "roofline": r["roofline"],
         "graph_replay": {"tokens_per_s": round(r["graph_tokens_per_s"], 1),
                          "ms_per_step": round(r["graph_ms_per_step"], 4)},
         "layer_hbm_frac": r["layer_hbm_frac"], "layer_mfma_frac": r["layer_mfma_frac"],
         "stage_us": r["stage_us"], "touched_experts": r["touched_experts"], "local_pairs": r["local_pairs"]}
    if cpu is not None:
        d["cpu_baseline"] = cpu
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=list(workloads.WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--tokens", type=int, default=None,
                    help="run --workload at this many tokens instead (its other sizes and seeds kept; "
                         "no secondary workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hashes and exit")
    ap.add_argument("--graph-probe", action="store_true",
                    help="only run direct calls, then graph replays, of --workload (for a kernel trace) and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="summarise rocprofv3's kernel trace of a --graph-probe run and exit")
    ap.add_argument("--kernels-per-call", type=int, default=6, help="kernels of one forward (--trace-summary)")
    args = ap.parse_args()
    if args.source_hash:
        print(json.dumps({p: kernel_source_hash(p) for p in KERNEL_SOURCES}))
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.kernels_per_call)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this layer runs on one GPU: the expert shard is exercised by running one "
                                   "shard's experts locally; --gpus must be 1"}))
        sys.exit(2)
    if args.tokens is not None:
        if args.tokens < 1 or args.all:
            print(json.dumps({"error": "--tokens needs a positive count and one --workload"}))
            sys.exit(2)
        global TOKENS_OVERRIDDEN
        TOKENS_OVERRIDDEN = True
        workloads.WORKLOADS[args.workload] = workloads.replace(workloads.WORKLOADS[args.workload], T=args.tokens)
        args.no_secondary = True
    if args.all:
        names = list(workloads.WORKLOADS)
    else:
        names = [args.workload] + ([] if args.no_secondary else [n for n in SECONDARY if n != args.workload])
    # the CPU oracle baselines first, before the process initialises the GPU
    cpu = {} if args.no_cpu_baseline or args.copy_calibration else cpu_baselines(names)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.graph_probe:
        graph_probe(args.workload)
        return
    nv.lib()
    hip = HipEvents()
    results = []
    for i, name in enumerate(names):
        # the secondary prefill workloads take fewer timed steps (each is ~10x longer)
        steps = args.steps if (i == 0 or args.all or PER_CALL_N.get(name, 20) >= 200) else max(5, args.steps // 2)
        results.append((name, steps) + bench_workload(name, steps, args.warmup, hip))
    lines = []
    for j, (name, steps, w, r) in enumerate(results):
        line = {"metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
                "steps": steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": r["dtype"],
                "data": "synthetic (seeded bf16 draws, NVFP4-quantized on the GPU)", "config": config_of(w),
                "roofline": r["roofline"], "per_call_us": r["per_call_us"],
                "graph_replay": {"tokens_per_s": round(r["graph_tokens_per_s"], 1),
                                 "ms_per_step": round(r["graph_ms_per_step"], 4)},
                "layer_hbm_frac": r["layer_hbm_frac"],
                "layer_mfma_frac": r["layer_mfma_frac"], "stage_us": r["stage_us"],
                "touched_experts": r["touched_experts"], "local_pairs": r["local_pairs"],
                "prewarm": r["prewarm"]}
        if name in cpu:
            line["cpu_baseline"] = cpu[name]
        if args.all:
            lines.append(line)
            continue
        line["secondary"] = [summary(w2, r2, cpu.get(n2)) for n2, _, w2, r2 in results[1:]]
        lines.append(line)
        break
    for line in lines:
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
