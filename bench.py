#!/usr/bin/env python3
"""Benchmark of the fused NVFP4 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

A step is one call of moe_nvfp4_forward (router top-k, shard filter,
permutation, [W4A4 activation quantizer], GEMM1 + SwiGLU, GEMM2, weighted
combine with the shared expert) over one batch of synthetic tokens whose
weights and inputs are already resident in HBM.  Prints ONE JSON line for the
headline workload (the T=64 expert-shard decode step), with:
  value      tokens/s of the whole job (T * K / elapsed, wall clock around K steps)
  roofline   the dominant kernel against its roof (HBM for decode, bf16 MFMA for
             prefill): algorithmic bytes (or flops) per launch / the kernel's
             average duration from the two HIP events recorded around it in each
             timed step (the per-stage breakdown comes from a separate pass)
  graph_replay  the same forward captured once in a HIP graph, K replays timed
  secondary  the same for the T=8192 all-expert W4A4 prefill step
  cpu_baseline  the CPU oracle timed on a bounded sample of the headline workload
--all prints one line per workload instead (a report, not the default line).
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
SECONDARY = "prefill_all_w4a4"
STAGES = ["route_permute", "act_quant", "gemm1_swiglu", "gemm2", "combine"]
G1_EVERY = 4                    # timed steps per GEMM1 event pair
CSRC = os.path.join(ROOT, "nvfp4_expert_layer_amd", "csrc")
# sources whose machine code the dominant kernel of each path is built from
KERNEL_SOURCES = {"decode": ["decode.hip", "device_common.h", "kernels.h"],
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
        h.update(t.encode())
    return h.hexdigest()[:16]


def measured_traffic(path, workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary profiles/traffic_gemm1_<workload>.txt (FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy's reading), or None when there is none or the kernel
    sources changed since the counters were taken."""
    fn = os.path.join(ROOT, "profiles", f"traffic_gemm1_{workload}.txt")
    if not os.path.exists(fn):
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

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

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
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    tg = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_s = time.perf_counter() - tg
    del graph
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
    path = "decode" if nv.moe_nvfp4_resolved_path(p) == nv.PATH_DECODE else "prefill"
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
           "graph_tokens_per_s": w.T * steps / graph_s, "graph_ms_per_step": graph_s * 1e3 / steps,
           "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
           "roofline": roof, "layer_hbm_frac": round(layer_hbm_frac, 4),
           "layer_mfma_frac": round(layer_mfma_frac, 4),
           "touched_experts": alg["touched"], "local_pairs": alg["P"],
           # the type the GEMMs multiply in: W4A4 on the tiled path multiplies
           # exact NVFP4 products in f16, everything else in bf16
           "dtype": "f16" if (path == "prefill" and w.mode != workloads.W4A16) else "bf16"}
    del local, shared, ws
    torch.cuda.empty_cache()
    return w, res


def _cpu_expert(args):
    wdict, e = args
    import workloads as wl
    from tests.oracle_helpers import quantize_expert_oracle
    w = wl.Workload(**wdict)
    w13, w2 = wl.gen_expert(w, e, "cpu")
    return e, quantize_expert_oracle(w13, w2)


def cpu_baseline(name, sample_tokens):
    """The oracle (numpy fp64) on the first `sample_tokens` tokens of the
    workload; weights drawn on the CPU and quantized by the oracle (untimed)."""
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    # runs before anything touches the GPU; workers are fresh interpreters (spawn)

    from oracle import moe
    from tests.oracle_helpers import to_f64
    w = workloads.WORKLOADS[name]
    x = to_f64(workloads.gen_hidden(w, "cpu", T=sample_tokens))
    G = to_f64(workloads.gen_gate(w, "cpu"))
    ids = moe.route(x, G, w.k)["ids"]
    need = sorted({int(e) for e in ids.reshape(-1) if w.offset <= e < w.offset + w.L})
    if w.has_shared:
        need.append(w.E)
    wdict = {k: getattr(w, k) for k in w.__dataclass_fields__}
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        q = dict(ex.map(_cpu_expert, [(wdict, e) for e in need]))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    t0 = time.perf_counter()
    moe.forward(x, G, lambda l: q[w.offset + l], q.get(w.E), w.k, w.offset, w.L, w.mode, act_global=w.act_global)
    dt = time.perf_counter() - t0
    return {"value": round(sample_tokens / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {sample_tokens} of {w.T} tokens of {name} ({len(need)} experts touched); "
                      f"numpy fp64, BLAS threads {threads}, host cores {len(os.sched_getaffinity(0))}; "
                      f"{dt:.1f} s"}


def config_of(w):
    c = {"workload": w.name, "T": w.T, "d_model": w.d, "d_ff": w.F, "experts": w.E, "top_k": w.k,
         "local_expert_offset": w.offset, "num_local_experts": w.L, "shared": int(w.has_shared),
         "mode": {workloads.W4A16: "W4A16", workloads.W4A4: "W4A4", workloads.W4A4_STATIC: "W4A4 static"}[w.mode]}
    if w.mode == workloads.W4A4_STATIC:
        c["act_global"] = list(w.act_global)
    return c


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=list(workloads.WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=48,
                    help="tokens of the headline batch the CPU oracle is timed on (~10-30 s)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hashes and exit")
    args = ap.parse_args()
    if args.source_hash:
        print(json.dumps({p: kernel_source_hash(p) for p in KERNEL_SOURCES}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this layer runs on one GPU: the expert shard is exercised by running one "
                                   "shard's experts locally; --gpus must be 1"}))
        sys.exit(2)
    names = list(workloads.WORKLOADS) if args.all else [args.workload]
    # the CPU oracle baseline first, before the process initialises the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload if not args.all else HEADLINE, args.cpu_sample)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    nv.lib()
    hip = HipEvents()
    for name in names:
        w, r = bench_workload(name, args.steps, args.warmup, hip)
        line = {"metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": r["dtype"],
                "data": "synthetic (seeded bf16 draws, NVFP4-quantized on the GPU)", "config": config_of(w),
                "roofline": r["roofline"], "graph_replay": {"tokens_per_s": round(r["graph_tokens_per_s"], 1),
                                                            "ms_per_step": round(r["graph_ms_per_step"], 4)},
                "layer_hbm_frac": r["layer_hbm_frac"],
                "layer_mfma_frac": r["layer_mfma_frac"], "stage_us": r["stage_us"],
                "touched_experts": r["touched_experts"], "local_pairs": r["local_pairs"]}
        if not args.all and not args.no_secondary and name != SECONDARY:
            w2, r2 = bench_workload(SECONDARY, max(5, args.steps // 5), args.warmup, hip)
            line["secondary"] = {"config": config_of(w2), "dtype": r2["dtype"],
                                 "tokens_per_s": round(r2["tokens_per_s"], 1),
                                 "ms_per_step": round(r2["ms_per_step"], 4), "roofline": r2["roofline"],
                                 "graph_replay": {"tokens_per_s": round(r2["graph_tokens_per_s"], 1),
                                                  "ms_per_step": round(r2["graph_ms_per_step"], 4)},
                                 "layer_mfma_frac": r2["layer_mfma_frac"], "stage_us": r2["stage_us"]}
        if cpu is not None and (not args.all or name == HEADLINE):
            line["cpu_baseline"] = cpu
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
